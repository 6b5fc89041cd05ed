"""Thin ctypes binding of libretention.so (C ABI in include/retention.h).

Argument marshalling only: tensors are checked for shape, dtype, device and contiguity (shapes and dtypes
first, so that a mismatch is reported before any pointer is formed), and their data pointers, gamma/theta
host arrays and torch's current HIP stream are passed to the C entry points of the same names. Every step of
the computation runs in the HIP kernels. If the library is missing this module raises; there is no CPU path.
The library carries a digest of the sources it was built from: a library older than the sources is rebuilt
in-tree before it is loaded (or refused, with build_if_missing=False).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import build as _build

RET_F32, RET_BF16 = 0, 1
RET_NORM_SCALE, RET_NORM_DECAY, RET_NORM_SCORES = 1, 2, 4
_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace", -4: "hip error"}

_lib = None


class RetentionError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__("%s failed: %s (%d): %s" % (fn, _STATUS.get(status, "?"), status, detail))
        self.status = status


def library_path() -> str:
    return _build.LIB_PATH


class Options(ctypes.Structure):
    """ret_options_t: the plan and measurement options of the *_ex entry points (fields as in retention.h)."""
    _fields_ = [("segments", ctypes.c_int), ("target_wgs", ctypes.c_int), ("prerotate", ctypes.c_int),
                ("onchip", ctypes.c_int), ("variant", ctypes.c_int), ("step_cw", ctypes.c_int),
                ("step_wr", ctypes.c_int), ("step_pairs", ctypes.c_int), ("bwd_direct", ctypes.c_int),
                ("step_cache", ctypes.c_int),
                ("chain_spin", ctypes.c_longlong), ("timer", ctypes.c_void_p)]


def _options(options):
    """None -> NULL; a dict of field values (the rest at the library's defaults), an Options or a Timer."""
    if options is None:
        return None
    if isinstance(options, Options):
        return ctypes.byref(options)
    o = Options()
    load().ret_options_default(ctypes.byref(o))
    if isinstance(options, Timer):
        options = {"timer": options}
    for key, val in dict(options).items():
        if key == "timer":
            o.timer = None if val is None else val.handle
        elif key in {f for f, _ in Options._fields_}:
            setattr(o, key, int(val))
        else:
            raise ValueError("unknown option %r" % key)
    return ctypes.byref(o)


class Timer:
    """A ret_timer_t: launch records of the kernels of every call given it (options={"timer": t})."""

    def __init__(self):
        self.handle = load().ret_timer_create()
        if not self.handle:
            raise MemoryError("ret_timer_create")

    def query(self, kernel: str = ""):
        """(total milliseconds, launches) recorded for `kernel` ('' = all kernels); synchronises the events."""
        ms = ctypes.c_double(0.0)
        n = ctypes.c_int64(0)
        st = load().ret_timer_query(self.handle, kernel.encode(), ctypes.byref(ms), ctypes.byref(n))
        if st != 0:
            raise RetentionError("ret_timer_query", st, "")
        return ms.value, n.value

    def reset(self):
        load().ret_timer_reset(self.handle)

    def close(self):
        if self.handle:
            load().ret_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def load(build_if_missing: bool = True):
    """Load libretention.so, building it in-tree first if it does not exist or was built from other sources
    than the ones in the tree (with build_if_missing=False such a library is refused)."""
    global _lib
    if _lib is not None:
        return _lib
    want = _build.source_digest() if os.path.isdir(_build.CSRC) else None
    if not os.path.exists(_build.LIB_PATH):
        if not build_if_missing:
            raise RuntimeError("libretention.so is not built: run linear_recurrent_sequence_amd.build.build()")
        _build.build()
    elif want is not None and _built_digest() != want:
        if not build_if_missing:
            raise RuntimeError("libretention.so was built from other sources than the tree's: rebuild it")
        import sys
        print("libretention.so is older than its sources: rebuilding", file=sys.stderr, flush=True)
        _build.build()
    lib = ctypes.CDLL(_build.LIB_PATH)
    if want is not None:
        lib.ret_source_digest.restype = ctypes.c_char_p
        got = lib.ret_source_digest().decode()
        if got != want:
            raise RuntimeError("libretention.so digest %s does not match the sources (%s)" % (got, want))
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    fp, dp = ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)
    op = ctypes.POINTER(Options)
    lib.ret_abi_version.restype = i32
    lib.ret_source_digest.restype = ctypes.c_char_p
    lib.ret_status_string.argtypes = [i32]
    lib.ret_status_string.restype = ctypes.c_char_p
    lib.ret_last_error.restype = ctypes.c_char_p
    lib.ret_parallel_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, fp, dp, i64, vp]
    lib.ret_parallel_fwd.restype = i32
    lib.ret_chunkwise_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.ret_chunkwise_workspace_bytes.restype = sz
    lib.ret_chunkwise_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, fp, dp, i64, i32, vp, vp,
                                      vp, sz, vp]
    lib.ret_chunkwise_fwd.restype = i32
    lib.ret_recurrent_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, fp, dp, i64, vp]
    lib.ret_recurrent_step.restype = i32
    lib.ret_recurrent_step_positions.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, fp, dp, vp, vp]
    lib.ret_recurrent_step_positions.restype = i32
    lib.ret_msr_epilogue.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, ctypes.c_float, vp]
    lib.ret_msr_epilogue.restype = i32
    lib.ret_chunkwise_msr_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, fp, dp, i64,
                                          i32, vp, vp, vp, vp, ctypes.c_float, vp, sz, vp]
    lib.ret_chunkwise_msr_fwd.restype = i32
    lib.ret_chunkwise_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.ret_chunkwise_bwd_workspace_bytes.restype = sz
    lib.ret_chunkwise_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, fp, dp, i64, i32,
                                      vp, sz, vp]
    lib.ret_chunkwise_bwd.restype = i32
    lib.ret_chunkwise_check.argtypes = [vp, vp]
    lib.ret_chunkwise_check.restype = i32
    lib.ret_chunkwise_workspace_bytes_ex.argtypes = lib.ret_chunkwise_workspace_bytes.argtypes + [op]
    lib.ret_chunkwise_workspace_bytes_ex.restype = sz
    lib.ret_chunkwise_bwd_workspace_bytes_ex.argtypes = lib.ret_chunkwise_bwd_workspace_bytes.argtypes + [op]
    lib.ret_chunkwise_bwd_workspace_bytes_ex.restype = sz
    lib.ret_chunkwise_fwd_ex.argtypes = lib.ret_chunkwise_fwd.argtypes + [op]
    lib.ret_chunkwise_fwd_ex.restype = i32
    lib.ret_chunkwise_msr_fwd_ex.argtypes = lib.ret_chunkwise_msr_fwd.argtypes + [op]
    lib.ret_chunkwise_msr_fwd_ex.restype = i32
    lib.ret_chunkwise_bwd_ex.argtypes = lib.ret_chunkwise_bwd.argtypes + [op]
    lib.ret_chunkwise_bwd_ex.restype = i32
    lib.ret_chunkwise_bwd_saved_ex.argtypes = lib.ret_chunkwise_bwd.argtypes[:18] + [vp, sz] + \
        lib.ret_chunkwise_bwd.argtypes[18:] + [op]
    lib.ret_chunkwise_bwd_saved_ex.restype = i32
    lib.ret_recurrent_step_ex.argtypes = lib.ret_recurrent_step.argtypes + [op]
    lib.ret_recurrent_step_ex.restype = i32
    lib.ret_recurrent_step_positions_ex.argtypes = lib.ret_recurrent_step_positions.argtypes + [op]
    lib.ret_recurrent_step_positions_ex.restype = i32
    lib.ret_chunkwise_normalized_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, op]
    lib.ret_chunkwise_normalized_workspace_bytes.restype = sz
    lib.ret_chunkwise_normalized_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, fp, dp, i64, i32,
                                                 i32, vp, vp, vp, vp, vp, sz, vp, op]
    lib.ret_chunkwise_normalized_fwd.restype = i32
    lib.ret_recurrent_step_normalized.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, fp, dp, i64,
                                                  i32, vp, op]
    lib.ret_recurrent_step_normalized.restype = i32
    lib.ret_chunkwise_fwd_noalloc.argtypes = lib.ret_chunkwise_fwd.argtypes[:17] + [vp]
    lib.ret_chunkwise_fwd_noalloc.restype = i32
    lib.ret_options_default.argtypes = [op]
    lib.ret_options_default.restype = None
    lib.ret_timer_create.restype = vp
    lib.ret_timer_destroy.argtypes = [vp]
    lib.ret_timer_destroy.restype = None
    lib.ret_timer_reset.argtypes = [vp]
    lib.ret_timer_reset.restype = None
    lib.ret_timer_query.argtypes = [vp, ctypes.c_char_p, dp, ctypes.POINTER(i64)]
    lib.ret_timer_query.restype = i32
    _lib = lib
    return lib


def _built_digest():
    """The source digest recorded in the built library (None if it cannot be read)."""
    try:
        lib = ctypes.CDLL(_build.LIB_PATH)
        lib.ret_source_digest.restype = ctypes.c_char_p
        return lib.ret_source_digest().decode()
    except (OSError, AttributeError):
        return None


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RET_F32
    if t.dtype == torch.bfloat16:
        return RET_BF16
    raise TypeError("tensors must be float32 or bfloat16, got %s" % t.dtype)


def _dev(t, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, name, shape, dtypes=None):
    """t must be a tensor of the given shape (and one of `dtypes`, if given); None passes."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError("%s must be %s, got %s" % (name, " or ".join(str(d) for d in dtypes), t.dtype))


def _same_device(*ts):
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError("all tensors must be on one device, got %s" % sorted(str(d) for d in devs))


_IO = (torch.float32, torch.bfloat16)


def _qkv(q, k, v, step=False):
    """Shapes of q, k, v ([B, N, H, d] or, for a decode step, [B, H, d]) and one dtype among them."""
    nd = 3 if step else 4
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != nd:
            raise ValueError("%s must be a %d-d tensor" % (name, nd))
    _shape(k, "k", q.shape, _IO)
    _shape(v, "v", tuple(q.shape[:-1]) + (v.shape[-1],), (q.dtype,))
    if q.dtype not in _IO or k.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype (float32 or bfloat16)")


def _gamma(gamma, H):
    g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float32).reshape(-1))
    if g.shape[0] != H:
        raise ValueError("gamma must have H=%d entries" % H)
    return g, g.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _theta(theta, dk):
    if theta is None:
        return None, None
    th = np.ascontiguousarray(np.asarray(theta, dtype=np.float64).reshape(-1))
    if th.shape[0] != dk // 2:
        raise ValueError("theta must have d_k/2 entries")
    return th, th.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, st):
    if st != 0:
        raise RetentionError(fn, st, load().ret_last_error().decode())


def ret_parallel_fwd(q, k, v, o, gamma, theta=None, pos0=0, stream=None):
    """o <- parallel-form retention of (q, k, v); q,k [B,N,H,dk], v,o [B,N,H,dv]."""
    lib = load()
    _qkv(q, k, v)
    B, N, H, dk = q.shape
    dv = v.shape[3]
    _shape(o, "o", (B, N, H, dv), _IO)
    _same_device(q, k, v, o)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    st = lib.ret_parallel_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, N, H, dk, dv, _dt(q),
                              _dt(o), gp, tp, int(pos0), _stream(stream))
    _check("ret_parallel_fwd", st)
    return o


def ret_chunkwise_workspace_bytes(B, N, H, dk, dv, chunk, in_dtype=torch.bfloat16, options=None) -> int:
    dt = RET_BF16 if in_dtype == torch.bfloat16 else RET_F32
    return int(load().ret_chunkwise_workspace_bytes_ex(B, N, H, dk, dv, chunk, dt, _options(options)))


def chunkwise_workspace(q, v, chunk, options=None):
    """Allocate (with torch) the zero-filled workspace ret_chunkwise_fwd plans for these shapes (and options), or
    None. Calls leave it ready for the next call."""
    B, N, H, dk = q.shape
    nbytes = ret_chunkwise_workspace_bytes(B, N, H, dk, v.shape[3], chunk, q.dtype, options)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=q.device)


def ret_chunkwise_check(workspace, stream=None):
    """Raise if a call that used `workspace` abandoned a segment-chain wait (synchronises the stream)."""
    if workspace is None:
        return
    _check("ret_chunkwise_check", load().ret_chunkwise_check(_dev(workspace, "workspace"), _stream(stream)))


def ret_chunkwise_fwd(q, k, v, o, gamma, chunk, theta=None, pos0=0, state_in=None, state_out=None,
                      workspace=None, stream=None, options=None):
    """o <- chunkwise retention of (q, k, v) starting from state_in; final state to state_out. options: a dict of
    ret_options_t fields (plan choices, a Timer under "timer") or None."""
    lib = load()
    _qkv(q, k, v)
    B, N, H, dk = q.shape
    dv = v.shape[3]
    _shape(o, "o", (B, N, H, dv), _IO)
    for name, s in (("state_in", state_in), ("state_out", state_out)):
        _shape(s, name, (B, H, dk, dv), (torch.float32,))
    _same_device(q, k, v, o, state_in, state_out, workspace)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ret_chunkwise_fwd_ex(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, N, H, dk, dv, _dt(q),
                                  _dt(o), gp, tp, int(pos0), int(chunk), _dev(state_in, "state_in"),
                                  _dev(state_out, "state_out"), _dev(workspace, "workspace"), ws_bytes,
                                  _stream(stream), _options(options))
    _check("ret_chunkwise_fwd", st)
    return o


def ret_recurrent_step(q, k, v, o, state, gamma, pos, theta=None, stream=None, options=None):
    """One decode step at position pos: state <- gamma state + k'^T v (in place), o <- q' state."""
    lib = load()
    _qkv(q, k, v, step=True)
    B, H, dk = q.shape
    dv = v.shape[2]
    _shape(o, "o", (B, H, dv), _IO)
    if state is None:
        raise ValueError("state must be float32 [B,H,dk,dv]")
    _shape(state, "state", (B, H, dk, dv), (torch.float32,))
    _same_device(q, k, v, o, state)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    st = lib.ret_recurrent_step_ex(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(state, "state"), B,
                                   H, dk, dv, _dt(q), _dt(o), gp, tp, int(pos), _stream(stream), _options(options))
    _check("ret_recurrent_step", st)
    return o


def ret_recurrent_step_positions(q, k, v, o, state, gamma, pos, theta=None, stream=None, options=None):
    """One decode step with sequence b at position pos[b] (pos: int64 [B] on the device, read when the kernel
    runs)."""
    lib = load()
    _qkv(q, k, v, step=True)
    B, H, dk = q.shape
    dv = v.shape[2]
    _shape(o, "o", (B, H, dv), _IO)
    if state is None:
        raise ValueError("state must be float32 [B,H,dk,dv]")
    _shape(state, "state", (B, H, dk, dv), (torch.float32,))
    if not isinstance(pos, torch.Tensor) or pos.dtype != torch.int64 or tuple(pos.shape) != (B,) \
            or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int64 tensor [B]")
    _same_device(q, k, v, o, state, pos)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    st = lib.ret_recurrent_step_positions_ex(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
                                             _dev(state, "state"), B, H, dk, dv, _dt(q), _dt(o), gp, tp,
                                             _dev(pos, "pos"), _stream(stream), _options(options))
    _check("ret_recurrent_step_positions", st)
    return o


def ret_msr_epilogue(o, y, gate=None, gn_weight=None, gn_bias=None, eps=1e-5, stream=None):
    """y = swish(gate) (.) GroupNorm_h(o), one GroupNorm group per head: o, gate, y [..., H, d_v] (the leading
    dims are the rows); gn_weight, gn_bias float32 [H * d_v] or None. y may be o or gate (in place)."""
    lib = load()
    if o.dim() < 2 or tuple(y.shape) != tuple(o.shape) or (gate is not None and tuple(gate.shape) != tuple(o.shape)):
        raise ValueError("o, y (and gate) must share one shape [..., H, d_v]")
    H, dv = o.shape[-2], o.shape[-1]
    rows = o.numel() // (H * dv) if H * dv else 0
    for name, t in (("gn_weight", gn_weight), ("gn_bias", gn_bias)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != H * dv):
            raise ValueError("%s must be float32 with H*d_v entries" % name)
    _same_device(o, y, gate, gn_weight, gn_bias)
    st = lib.ret_msr_epilogue(_dev(o, "o"), _dev(gate, "gate"), _dev(gn_weight, "gn_weight"),
                              _dev(gn_bias, "gn_bias"), _dev(y, "y"), rows, H, dv, _dt(o),
                              _dt(gate) if gate is not None else RET_BF16, _dt(y), float(eps), _stream(stream))
    _check("ret_msr_epilogue", st)
    return y


def ret_chunkwise_msr_fwd(q, k, v, y, gamma, chunk, gate=None, gn_weight=None, gn_bias=None, eps=1e-5, theta=None,
                          pos0=0, state_in=None, state_out=None, workspace=None, stream=None, options=None):
    """Chunkwise retention, then y = swish(gate) (.) GroupNorm_h(O), fused into the output stores where the
    kernel holds whole head rows. Arguments as ret_chunkwise_fwd (y in the place of o) and ret_msr_epilogue."""
    lib = load()
    _qkv(q, k, v)
    B, N, H, dk = q.shape
    dv = v.shape[3]
    _shape(y, "y", (B, N, H, dv), _IO)
    _shape(gate, "gate", (B, N, H, dv), _IO)
    for name, t in (("gn_weight", gn_weight), ("gn_bias", gn_bias)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != H * dv):
            raise ValueError("%s must be float32 with H*d_v entries" % name)
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (B, H, dk, dv)):
            raise ValueError("%s must be float32 [B,H,dk,dv]" % name)
    _same_device(q, k, v, y, gate, gn_weight, gn_bias, state_in, state_out, workspace)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ret_chunkwise_msr_fwd_ex(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(gate, "gate"), _dev(y, "y"), B,
                                      N, H, dk, dv, _dt(q), _dt(y), _dt(gate) if gate is not None else RET_BF16, gp,
                                      tp, int(pos0), int(chunk), _dev(state_in, "state_in"),
                                      _dev(state_out, "state_out"), _dev(gn_weight, "gn_weight"),
                                      _dev(gn_bias, "gn_bias"), float(eps), _dev(workspace, "workspace"), wsb,
                                      _stream(stream), _options(options))
    _check("ret_chunkwise_msr_fwd", st)
    return y


def chunkwise_bwd_workspace(q, v, chunk, options=None):
    """A zero-filled workspace of ret_chunkwise_bwd_workspace_bytes for these shapes (ret_chunkwise_check reports
    on it after the gradients' calls)."""
    B, N, H, dk = q.shape
    nbytes = load().ret_chunkwise_bwd_workspace_bytes_ex(B, N, H, dk, v.shape[3], int(chunk), _dt(q),
                                                         _options(options))
    if nbytes == 0:
        raise ValueError("gradients: unsupported shape")
    return torch.zeros((nbytes,), dtype=torch.uint8, device=q.device)


def ret_chunkwise_bwd(q, k, v, dout, dq, dk, dv, gamma, chunk, theta=None, pos0=0, workspace=None, stream=None,
                      options=None, check=False, fwd_workspace=None):
    """dq, dk, dv <- gradients of sum(dout (.) O), O = chunkwise retention of (q, k, v) from a zero state. Without a
    workspace one is allocated for the call; check=True then synchronises and raises if a segment-chain wait gave
    up (the affected gradients are NaN either way). fwd_workspace: the workspace of the ret_chunkwise_fwd call that
    made O (same inputs and options, no state_in), whose rotated q, k and segment states are then reused where its
    kernels left them (ret_chunkwise_bwd_saved_ex)."""
    lib = load()
    _qkv(q, k, v)
    B, N, H, d_k = q.shape
    d_v = v.shape[3]
    _shape(dout, "dout", (B, N, H, d_v), (q.dtype,))
    _shape(dq, "dq", (B, N, H, d_k), _IO)
    _shape(dk, "dk", (B, N, H, d_k), (dq.dtype,))
    _shape(dv, "dv", (B, N, H, d_v), (dq.dtype,))
    _same_device(q, k, v, dout, dq, dk, dv, workspace, fwd_workspace)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, d_k)
    if workspace is None:
        workspace = chunkwise_bwd_workspace(q, v, chunk, options)
    wsb = workspace.numel() * workspace.element_size()
    fwp = _dev(fwd_workspace, "fwd_workspace") if fwd_workspace is not None else None
    fwb = fwd_workspace.numel() * fwd_workspace.element_size() if fwd_workspace is not None else 0
    st = lib.ret_chunkwise_bwd_saved_ex(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(dout, "dout"), _dev(dq, "dq"),
                                        _dev(dk, "dk"), _dev(dv, "dv"), B, N, H, d_k, d_v, _dt(q), _dt(dq), gp, tp,
                                        int(pos0), int(chunk), fwp, fwb, _dev(workspace, "workspace"), wsb,
                                        _stream(stream), _options(options))
    _check("ret_chunkwise_bwd", st)
    if check:
        ret_chunkwise_check(workspace, stream)
    return dq, dk, dv


def norm_flags(scale=False, decay=False, scores=False) -> int:
    """RET_NORM_* flags: scores / sqrt(d_k), decay rows divided by the root of their sums, scores rows divided by
    max(|row sum|, 1)."""
    return (RET_NORM_SCALE if scale else 0) | (RET_NORM_DECAY if decay else 0) | (RET_NORM_SCORES if scores else 0)


def chunkwise_normalized_workspace(q, v, chunk, options=None):
    """A zero-filled workspace of ret_chunkwise_normalized_workspace_bytes for these shapes."""
    B, N, H, dk = q.shape
    nbytes = load().ret_chunkwise_normalized_workspace_bytes(B, N, H, dk, v.shape[3], int(chunk), _dt(q),
                                                             _options(options))
    if nbytes == 0:
        raise ValueError("normalized chunkwise form: unsupported shape")
    return torch.zeros((nbytes,), dtype=torch.uint8, device=q.device)


def ret_chunkwise_normalized_fwd(q, k, v, o, gamma, chunk, norm, theta=None, pos0=0, state_in=None, state_out=None,
                                 z_in=None, z_out=None, workspace=None, stream=None, options=None):
    """o <- chunkwise retention with the score normalizations `norm` (RET_NORM_* flags); the state and the key
    sum z [B,H,dk] are carried in and out."""
    lib = load()
    _qkv(q, k, v)
    B, N, H, dk = q.shape
    dv = v.shape[3]
    _shape(o, "o", (B, N, H, dv), _IO)
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        _shape(t, name, (B, H, dk, dv), (torch.float32,))
    for name, t in (("z_in", z_in), ("z_out", z_out)):
        _shape(t, name, (B, H, dk), (torch.float32,))
    _same_device(q, k, v, o, state_in, state_out, z_in, z_out, workspace)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    if workspace is None:
        workspace = chunkwise_normalized_workspace(q, v, chunk, options)
    wsb = workspace.numel() * workspace.element_size()
    st = lib.ret_chunkwise_normalized_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, N, H, dk, dv,
                                          _dt(q), _dt(o), gp, tp, int(pos0), int(chunk), int(norm),
                                          _dev(state_in, "state_in"), _dev(state_out, "state_out"),
                                          _dev(z_in, "z_in"), _dev(z_out, "z_out"), _dev(workspace, "workspace"), wsb,
                                          _stream(stream), _options(options))
    _check("ret_chunkwise_normalized_fwd", st)
    return o


def ret_recurrent_step_normalized(q, k, v, o, state, z, gamma, pos, norm, theta=None, stream=None, options=None):
    """One decode step with the score normalizations: state and z [B,H,dk] updated in place, o <- normalized
    q' state."""
    lib = load()
    _qkv(q, k, v, step=True)
    B, H, dk = q.shape
    dv = v.shape[2]
    _shape(o, "o", (B, H, dv), _IO)
    if state is None or z is None:
        raise ValueError("state [B,H,dk,dv] and z [B,H,dk] (float32) are required")
    _shape(state, "state", (B, H, dk, dv), (torch.float32,))
    _shape(z, "z", (B, H, dk), (torch.float32,))
    _same_device(q, k, v, o, state, z)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    st = lib.ret_recurrent_step_normalized(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
                                           _dev(state, "state"), _dev(z, "z"), B, H, dk, dv, _dt(q), _dt(o), gp, tp,
                                           int(pos), int(norm), _stream(stream), _options(options))
    _check("ret_recurrent_step_normalized", st)
    return o


def ret_chunkwise_fwd_noalloc(q, k, v, o, gamma, chunk, theta=None, pos0=0, state_in=None, state_out=None,
                              stream=None):
    """ret_chunkwise_fwd with the library's own device scratch array as the workspace: allocates nothing (for
    callers that cannot). Calls that overlap in time on one GPU must not be made."""
    lib = load()
    _qkv(q, k, v)
    B, N, H, dk = q.shape
    dv = v.shape[3]
    _shape(o, "o", (B, N, H, dv), _IO)
    for name, s in (("state_in", state_in), ("state_out", state_out)):
        _shape(s, name, (B, H, dk, dv), (torch.float32,))
    _same_device(q, k, v, o, state_in, state_out)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    st = lib.ret_chunkwise_fwd_noalloc(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, N, H, dk, dv,
                                       _dt(q), _dt(o), gp, tp, int(pos0), int(chunk), _dev(state_in, "state_in"),
                                       _dev(state_out, "state_out"), _stream(stream))
    _check("ret_chunkwise_fwd_noalloc", st)
    return o
