"""Thin ctypes binding of libretention.so (C ABI in include/retention.h).

Argument marshalling only: tensors are checked for device, dtype, shape and contiguity, and their data
pointers, gamma/theta host arrays and torch's current HIP stream are passed to the C entry points of the
same names. Every step of the computation runs in the HIP kernels. If the library is missing this module
raises; there is no CPU path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import build as _build

RET_F32, RET_BF16 = 0, 1
_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace", -4: "hip error"}

_lib = None


class RetentionError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__("%s failed: %s (%d): %s" % (fn, _STATUS.get(status, "?"), status, detail))
        self.status = status


def library_path() -> str:
    return _build.LIB_PATH


def load(build_if_missing: bool = True):
    """Load libretention.so (building it in-tree first if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB_PATH):
        if not build_if_missing:
            raise RuntimeError("libretention.so is not built: run linear_recurrent_sequence_amd.build.build()")
        _build.build()
    lib = ctypes.CDLL(_build.LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    fp, dp = ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)
    lib.ret_abi_version.restype = i32
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
    lib.ret_timing_enable.argtypes = [i32]
    lib.ret_timing_enable.restype = i32
    lib.ret_timing_query.argtypes = [ctypes.c_char_p, dp, ctypes.POINTER(i64)]
    lib.ret_timing_query.restype = i32
    lib.ret_timing_reset.restype = None
    _lib = lib
    return lib


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
    B, N, H, dk = q.shape
    dv = v.shape[3]
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    st = lib.ret_parallel_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, N, H, dk, dv, _dt(q),
                              _dt(o), gp, tp, int(pos0), _stream(stream))
    _check("ret_parallel_fwd", st)
    return o


def ret_chunkwise_workspace_bytes(B, N, H, dk, dv, chunk, in_dtype=torch.bfloat16) -> int:
    dt = RET_BF16 if in_dtype == torch.bfloat16 else RET_F32
    return int(load().ret_chunkwise_workspace_bytes(B, N, H, dk, dv, chunk, dt))


def chunkwise_workspace(q, v, chunk):
    """Allocate (with torch) the zero-filled workspace ret_chunkwise_fwd plans for these shapes, or None. Calls
    leave it ready for the next call."""
    B, N, H, dk = q.shape
    nbytes = ret_chunkwise_workspace_bytes(B, N, H, dk, v.shape[3], chunk, q.dtype)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=q.device)


def ret_chunkwise_check(workspace, stream=None):
    """Raise if a call that used `workspace` abandoned a segment-chain wait (synchronises the stream)."""
    if workspace is None:
        return
    _check("ret_chunkwise_check", load().ret_chunkwise_check(_dev(workspace, "workspace"), _stream(stream)))


def ret_chunkwise_fwd(q, k, v, o, gamma, chunk, theta=None, pos0=0, state_in=None, state_out=None,
                      workspace=None, stream=None):
    """o <- chunkwise retention of (q, k, v) starting from state_in; final state to state_out."""
    lib = load()
    B, N, H, dk = q.shape
    dv = v.shape[3]
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    for name, s in (("state_in", state_in), ("state_out", state_out)):
        if s is not None and (s.dtype != torch.float32 or tuple(s.shape) != (B, H, dk, dv)):
            raise ValueError("%s must be float32 [B,H,dk,dv]" % name)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ret_chunkwise_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, N, H, dk, dv, _dt(q),
                               _dt(o), gp, tp, int(pos0), int(chunk), _dev(state_in, "state_in"),
                               _dev(state_out, "state_out"), _dev(workspace, "workspace"), ws_bytes,
                               _stream(stream))
    _check("ret_chunkwise_fwd", st)
    return o


def ret_recurrent_step(q, k, v, o, state, gamma, pos, theta=None, stream=None):
    """One decode step at position pos: state <- gamma state + k'^T v (in place), o <- q' state."""
    lib = load()
    B, H, dk = q.shape
    dv = v.shape[2]
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv):
        raise ValueError("state must be float32 [B,H,dk,dv]")
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    st = lib.ret_recurrent_step(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(state, "state"), B, H,
                                dk, dv, _dt(q), _dt(o), gp, tp, int(pos), _stream(stream))
    _check("ret_recurrent_step", st)
    return o


def ret_recurrent_step_positions(q, k, v, o, state, gamma, pos, theta=None, stream=None):
    """One decode step with sequence b at position pos[b] (pos: int64 [B] on the device, read when the kernel
    runs)."""
    lib = load()
    B, H, dk = q.shape
    dv = v.shape[2]
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv):
        raise ValueError("state must be float32 [B,H,dk,dv]")
    if pos.dtype != torch.int64 or tuple(pos.shape) != (B,) or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int64 tensor [B]")
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    st = lib.ret_recurrent_step_positions(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
                                          _dev(state, "state"), B, H, dk, dv, _dt(q), _dt(o), gp, tp,
                                          _dev(pos, "pos"), _stream(stream))
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
    st = lib.ret_msr_epilogue(_dev(o, "o"), _dev(gate, "gate"), _dev(gn_weight, "gn_weight"),
                              _dev(gn_bias, "gn_bias"), _dev(y, "y"), rows, H, dv, _dt(o),
                              _dt(gate) if gate is not None else RET_BF16, _dt(y), float(eps), _stream(stream))
    _check("ret_msr_epilogue", st)
    return y


def ret_chunkwise_msr_fwd(q, k, v, y, gamma, chunk, gate=None, gn_weight=None, gn_bias=None, eps=1e-5, theta=None,
                          pos0=0, state_in=None, state_out=None, workspace=None, stream=None):
    """Chunkwise retention, then y = swish(gate) (.) GroupNorm_h(O), fused into the output stores where the
    kernel holds whole head rows. Arguments as ret_chunkwise_fwd (y in the place of o) and ret_msr_epilogue."""
    lib = load()
    B, N, H, dk = q.shape
    dv = v.shape[3]
    if tuple(y.shape) != (B, N, H, dv) or (gate is not None and tuple(gate.shape) != (B, N, H, dv)):
        raise ValueError("y (and gate) must be [B,N,H,d_v]")
    for name, t in (("gn_weight", gn_weight), ("gn_bias", gn_bias)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != H * dv):
            raise ValueError("%s must be float32 with H*d_v entries" % name)
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (B, H, dk, dv)):
            raise ValueError("%s must be float32 [B,H,dk,dv]" % name)
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, dk)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ret_chunkwise_msr_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(gate, "gate"), _dev(y, "y"), B, N,
                                   H, dk, dv, _dt(q), _dt(y), _dt(gate) if gate is not None else RET_BF16, gp, tp,
                                   int(pos0), int(chunk), _dev(state_in, "state_in"), _dev(state_out, "state_out"),
                                   _dev(gn_weight, "gn_weight"), _dev(gn_bias, "gn_bias"), float(eps),
                                   _dev(workspace, "workspace"), wsb, _stream(stream))
    _check("ret_chunkwise_msr_fwd", st)
    return y


def chunkwise_bwd_workspace(q, v, chunk):
    """A zero-filled workspace of ret_chunkwise_bwd_workspace_bytes for these shapes."""
    B, N, H, dk = q.shape
    nbytes = load().ret_chunkwise_bwd_workspace_bytes(B, N, H, dk, v.shape[3], int(chunk), _dt(q))
    if nbytes == 0:
        raise ValueError("gradients: unsupported shape")
    return torch.zeros((nbytes,), dtype=torch.uint8, device=q.device)


def ret_chunkwise_bwd(q, k, v, dout, dq, dk, dv, gamma, chunk, theta=None, pos0=0, workspace=None, stream=None):
    """dq, dk, dv <- gradients of sum(dout (.) O), O = chunkwise retention of (q, k, v) from a zero state."""
    lib = load()
    B, N, H, d_k = q.shape
    d_v = v.shape[3]
    if tuple(dout.shape) != (B, N, H, d_v) or tuple(dq.shape) != tuple(q.shape) or tuple(dk.shape) != tuple(k.shape) \
            or tuple(dv.shape) != tuple(v.shape):
        raise ValueError("dout/dv must be [B,N,H,d_v] and dq/dk [B,N,H,d_k]")
    if dout.dtype != q.dtype or dq.dtype != dk.dtype or dq.dtype != dv.dtype:
        raise ValueError("dout must have the inputs' dtype and dq, dk, dv one dtype")
    g, gp = _gamma(gamma, H)
    th, tp = _theta(theta, d_k)
    if workspace is None:
        workspace = chunkwise_bwd_workspace(q, v, chunk)
    wsb = workspace.numel() * workspace.element_size()
    st = lib.ret_chunkwise_bwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(dout, "dout"), _dev(dq, "dq"),
                               _dev(dk, "dk"), _dev(dv, "dv"), B, N, H, d_k, d_v, _dt(q), _dt(dq), gp, tp, int(pos0),
                               int(chunk), _dev(workspace, "workspace"), wsb, _stream(stream))
    _check("ret_chunkwise_bwd", st)
    return dq, dk, dv


def timing_enable(on: bool) -> bool:
    return bool(load().ret_timing_enable(1 if on else 0))


def timing_query(kernel: str = ""):
    """(total milliseconds, launches) recorded for `kernel` ('' = all kernels)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    st = load().ret_timing_query(kernel.encode(), ctypes.byref(ms), ctypes.byref(n))
    if st != 0:
        raise RetentionError("ret_timing_query", st, "")
    return ms.value, n.value


def timing_reset():
    load().ret_timing_reset()
