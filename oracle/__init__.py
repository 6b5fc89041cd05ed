"""Retention oracle: numpy-facing wrapper around the fp64 C oracle in ``retention_oracle.c``.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package. It shares no code with the GPU library: it never imports ``linear_recurrent_sequence_amd``
and the GPU library never loads ``liboracle.so``.

Every function takes numpy arrays in the layouts below, upcasts them to float64 (exact for fp32 and bf16
values), and returns float64 results:

    q, k   [B, N, H, dk]      v, o   [B, N, H, dv]      state  [B, H, dk, dv]
    gamma  [H]                theta  [dk // 2] or None (no rotation)

Sources: "Hybrid Architectures: RetNet and the Three Computation Paradigms" (sections 2-9) and the RetNet
paper summary (Eq. 5, 6 and 7; "Gating mechanism"; "Retention Score Normalization"). Which function follows
which passage is stated in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "retention_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` (host gcc; no GPU code)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(ctypes.c_double)
    I = ctypes.c_int
    LL = ctypes.c_longlong
    lib.orc_parallel.argtypes = [P, P, P, P, I, I, I, I, I, P, P, LL, I]
    lib.orc_parallel_rows.argtypes = [P, P, P, I, I, I, I, I, P, P, LL, ctypes.POINTER(LL), I, P, I]
    lib.orc_recurrent.argtypes = [P, P, P, P, I, I, I, I, I, P, P, LL, P, P, I]
    lib.orc_chunkwise.argtypes = [P, P, P, P, I, I, I, I, I, P, P, LL, I, P, P, I]
    lib.orc_parallel_normalized.argtypes = [P, P, P, P, I, I, I, I, I, P, P, LL, I, I]
    lib.orc_msr_epilogue.argtypes = [P, P, P, P, P, LL, I, I, ctypes.c_double]
    lib.orc_grad.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P, P, LL, I]
    lib.orc_normalized.argtypes = [P, P, P, P, I, I, I, I, I, P, P, LL, I, I, P, P, P, P, I]
    for f in (lib.orc_parallel, lib.orc_parallel_rows, lib.orc_recurrent, lib.orc_chunkwise,
              lib.orc_parallel_normalized, lib.orc_msr_epilogue, lib.orc_grad, lib.orc_normalized):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shapes(q, k, v):
    if q.ndim != 4 or k.shape != q.shape or v.ndim != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,N,H,dk] and v [B,N,H,dv]")
    B, N, H, dk = q.shape
    return B, N, H, dk, v.shape[3]


def _common(q, k, v, gamma, theta):
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, dk, dv = _shapes(q, k, v)
    g = _f64(gamma).reshape(-1)
    if g.shape[0] != H:
        raise ValueError("gamma must have H entries")
    th = None if theta is None else _f64(theta).reshape(-1)
    if th is not None and th.shape[0] != dk // 2:
        raise ValueError("theta must have dk/2 entries")
    return q, k, v, g, th, (B, N, H, dk, dv)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError("oracle %s failed with status %d" % (name, rc))


def parallel(q, k, v, gamma, theta=None, pos0=0, threads=None):
    """Parallel form O = (Q K^T (.) D) V over the whole sequence (the definition)."""
    q, k, v, g, th, (B, N, H, dk, dv) = _common(q, k, v, gamma, theta)
    o = np.zeros((B, N, H, dv), np.float64)
    rc = _load().orc_parallel(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, N, H, dk, dv, _ptr(g), _ptr(th),
                              int(pos0), threads or default_threads())
    _check(rc, "parallel")
    return o


def parallel_normalized(q, k, v, gamma, theta=None, pos0=0, scale=False, decay=False, scores=False, threads=None):
    """Parallel form with the score normalizations (blog section 8.5; paper summary, "Retention Score
    Normalization"): QK^T / sqrt(d_k) (scale), D~ rows (decay), R~ rows (scores)."""
    q, k, v, g, th, (B, N, H, dk, dv) = _common(q, k, v, gamma, theta)
    o = np.zeros((B, N, H, dv), np.float64)
    norm = (1 if scale else 0) | (2 if decay else 0) | (4 if scores else 0)
    rc = _load().orc_parallel_normalized(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, N, H, dk, dv, _ptr(g), _ptr(th),
                                         int(pos0), norm, threads or default_threads())
    _check(rc, "parallel_normalized")
    return o


def grad(q, k, v, dout, gamma, theta=None, pos0=0, threads=None):
    """Gradients (dq, dk, dv) of sum(dout (.) O) for O the retention output from a zero state, by the adjoint of
    the recurrent scan (see the C file)."""
    q, k, v, g, th, (B, N, H, dk, dv) = _common(q, k, v, gamma, theta)
    do = _f64(dout)
    if do.shape != (B, N, H, dv):
        raise ValueError("dout must be [B,N,H,dv]")
    dq, dk_, dv_ = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    rc = _load().orc_grad(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk_), _ptr(dv_), B, N, H, dk, dv,
                          _ptr(g), _ptr(th), int(pos0), threads or default_threads())
    _check(rc, "grad")
    return dq, dk_, dv_


def msr_epilogue(o, gate=None, weight=None, bias=None, eps=1e-5):
    """y = swish(gate) (.) GroupNorm_h(o) (blog sections 8.4 and 9.1; paper summary, "Gating mechanism").
    o, gate: [..., H, dv] (any leading shape: tokens); weight, bias: [H*dv] or None; one group per head."""
    o = _f64(o)
    H, dv = o.shape[-2], o.shape[-1]
    rows = int(np.prod(o.shape[:-2], dtype=np.int64))
    g = None if gate is None else _f64(gate)
    if g is not None and g.shape != o.shape:
        raise ValueError("gate must have the shape of o")
    w = None if weight is None else _f64(np.reshape(weight, (H * dv,)))
    b = None if bias is None else _f64(np.reshape(bias, (H * dv,)))
    y = np.zeros(o.shape, np.float64)
    rc = _load().orc_msr_epilogue(_ptr(o), _ptr(g), _ptr(w), _ptr(b), _ptr(y), rows, H, dv, float(eps))
    _check(rc, "msr_epilogue")
    return y


def parallel_rows(q, k, v, gamma, rows, theta=None, pos0=0, threads=None):
    """Rows ``rows`` (token indices) of the parallel form, returned as [B, len(rows), H, dv]."""
    q, k, v, g, th, (B, N, H, dk, dv) = _common(q, k, v, gamma, theta)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    o = np.zeros((B, r.shape[0], H, dv), np.float64)
    rc = _load().orc_parallel_rows(_ptr(q), _ptr(k), _ptr(v), B, N, H, dk, dv, _ptr(g), _ptr(th), int(pos0),
                                   r.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong)), r.shape[0], _ptr(o),
                                   threads or default_threads())
    _check(rc, "parallel_rows")
    return o


def recurrent(q, k, v, gamma, theta=None, pos0=0, state_in=None, threads=None):
    """Recurrent form; returns (O, final state)."""
    q, k, v, g, th, (B, N, H, dk, dv) = _common(q, k, v, gamma, theta)
    o = np.zeros((B, N, H, dv), np.float64)
    s_in = None if state_in is None else _f64(state_in)
    if s_in is not None and s_in.shape != (B, H, dk, dv):
        raise ValueError("state_in must be [B,H,dk,dv]")
    s_out = np.zeros((B, H, dk, dv), np.float64)
    rc = _load().orc_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, N, H, dk, dv, _ptr(g), _ptr(th),
                               int(pos0), _ptr(s_in), _ptr(s_out), threads or default_threads())
    _check(rc, "recurrent")
    return o, s_out


def recurrent_step(q, k, v, gamma, state, pos, theta=None, threads=None):
    """One decode step at absolute position ``pos``: q, k [B,H,dk], v [B,H,dv]; returns (o [B,H,dv], S)."""
    q4 = _f64(q)[:, None]
    k4 = _f64(k)[:, None]
    v4 = _f64(v)[:, None]
    o, s = recurrent(q4, k4, v4, gamma, theta=theta, pos0=pos, state_in=state, threads=threads)
    return o[:, 0], s


def chunkwise(q, k, v, gamma, chunk, theta=None, pos0=0, state_in=None, threads=None):
    """Chunkwise form with chunk size ``chunk``; returns (O, final state)."""
    q, k, v, g, th, (B, N, H, dk, dv) = _common(q, k, v, gamma, theta)
    o = np.zeros((B, N, H, dv), np.float64)
    s_in = None if state_in is None else _f64(state_in)
    if s_in is not None and s_in.shape != (B, H, dk, dv):
        raise ValueError("state_in must be [B,H,dk,dv]")
    s_out = np.zeros((B, H, dk, dv), np.float64)
    rc = _load().orc_chunkwise(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, N, H, dk, dv, _ptr(g), _ptr(th),
                               int(pos0), int(chunk), _ptr(s_in), _ptr(s_out), threads or default_threads())
    _check(rc, "chunkwise")
    return o, s_out


def _norm_flags(scale, decay, scores):
    return (1 if scale else 0) | (2 if decay else 0) | (4 if scores else 0)


def normalized(q, k, v, gamma, chunk=0, theta=None, pos0=0, scale=False, decay=False, scores=False,
               state_in=None, z_in=None, threads=None):
    """Recurrent (chunk 0) or chunkwise (chunk > 0) form with the score normalizations, carrying the state S
    [B,H,dk,dv] and the decayed key sum z [B,H,dk] (see the C file for the reading); returns (O, S, z)."""
    q, k, v, g, th, (B, N, H, dk, dv) = _common(q, k, v, gamma, theta)
    o = np.zeros((B, N, H, dv), np.float64)
    s_in = None if state_in is None else _f64(state_in)
    zi = None if z_in is None else _f64(z_in)
    if s_in is not None and s_in.shape != (B, H, dk, dv):
        raise ValueError("state_in must be [B,H,dk,dv]")
    if zi is not None and zi.shape != (B, H, dk):
        raise ValueError("z_in must be [B,H,dk]")
    s_out = np.zeros((B, H, dk, dv), np.float64)
    z_out = np.zeros((B, H, dk), np.float64)
    rc = _load().orc_normalized(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, N, H, dk, dv, _ptr(g), _ptr(th), int(pos0),
                                int(chunk), _norm_flags(scale, decay, scores), _ptr(s_in), _ptr(s_out), _ptr(zi),
                                _ptr(z_out), threads or default_threads())
    _check(rc, "normalized")
    return o, s_out, z_out


def normalized_step(q, k, v, gamma, state, z, pos, theta=None, scale=False, decay=False, scores=False):
    """One normalized decode step at absolute position ``pos``: q, k [B,H,dk], v [B,H,dv]; returns (o, S, z)."""
    o, s, zz = normalized(_f64(q)[:, None], _f64(k)[:, None], _f64(v)[:, None], gamma, 0, theta=theta, pos0=pos,
                          scale=scale, decay=decay, scores=scores, state_in=state, z_in=z)
    return o[:, 0], s, zz
