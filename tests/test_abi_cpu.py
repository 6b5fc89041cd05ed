"""The C-ABI library loads, exports every entry point include/retention.h declares, and rejects invalid
arguments on the host before touching a GPU (no GPU needed; no compute call is made)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "retention.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ret_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from linear_recurrent_sequence_amd import retention
    return retention.load()


def test_header_declares_the_three_operations():
    names = _declared()
    for fn in ("ret_chunkwise_fwd", "ret_recurrent_step", "ret_parallel_fwd", "ret_chunkwise_workspace_bytes"):
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), "libretention.so does not export %s" % name


def test_version_and_status_strings(lib):
    declared = int(re.search(r"#define RET_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.ret_abi_version() == declared
    assert lib.ret_status_string(0) == b"ok"
    assert lib.ret_status_string(-2) == b"unsupported shape or dtype"


def _call_chunk(lib, **kw):
    a = dict(q=16, k=32, v=48, o=64, B=1, N=64, H=2, dk=64, dv=64, ind=1, outd=1, gamma=[0.9, 0.99], theta=None,
             pos0=0, chunk=64, sin=None, sout=None, ws=None, wsb=0)
    a.update(kw)
    g = np.asarray(a["gamma"], np.float32)
    th = None if a["theta"] is None else np.asarray(a["theta"], np.float64)
    return lib.ret_chunkwise_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["N"], a["H"], a["dk"], a["dv"],
                                 a["ind"], a["outd"], g.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                 None if th is None else th.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                 a["pos0"], a["chunk"], a["sin"], a["sout"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1),                 # null pointer
    (dict(N=0), -1),                    # empty sequence
    (dict(gamma=[0.9, 1.5]), -1),       # gamma outside (0, 1]
    (dict(gamma=[0.9, 0.0]), -1),
    (dict(gamma=[0.9, float("nan")]), -1),
    (dict(q=8), -1),                    # misaligned
    (dict(o=16), -1),                   # o aliases q
    (dict(ind=0, outd=1), -1),          # F32 input with BF16 output
    (dict(chunk=0), -1),
    (dict(dk=63, theta=[0.1] * 31), -1),  # odd d_k with rotation
    (dict(dk=48), -2),                  # no instance for d_k = 48
    (dict(dv=96), -2),                  # bf16 d_v must be a multiple of 64
    (dict(chunk=48), -2),
    (dict(wsb=1024), -3),               # workspace bytes without a workspace
])
def test_chunkwise_rejects_invalid_arguments(lib, kw, status):
    assert _call_chunk(lib, **kw) == status
    assert lib.ret_last_error() != b""


def test_workspace_query(lib):
    # one (b, h) with a long sequence is split into segments; many short sequences are not
    n_long = lib.ret_chunkwise_workspace_bytes(1, 65536, 8, 128, 128, 128, 1)
    # 8 units (8 heads x 1 d_v tile of 128) x 32 segments of 2048 tokens in three launches (local passes, scan,
    # full passes): the first 64 KB (header, untouched), then one 128x128 fp32 state slot per (unit, segment)
    assert n_long == 64 * 1024 + 8 * 32 * 128 * 128 * 4
    # fp32 input runs the split kernels: the header, then one d_k x d_v state per (b, h, segment)
    n_f32 = lib.ret_chunkwise_workspace_bytes(1, 4096, 2, 64, 64, 64, 0)
    assert n_f32 > 256 and (n_f32 - 256) % (2 * 64 * 64 * 4) == 0
    # 8 d_v tiles of 64 per head: q and k are rotated once into the workspace (two bf16 copies) beside the
    # segment chain
    n_wide = lib.ret_chunkwise_workspace_bytes(1, 8192, 16, 256, 512, 128, 1)
    rot = 2 * 1 * 8192 * 16 * 256 * 2
    assert n_wide > rot and (n_wide - rot) % 256 == 0
    assert lib.ret_chunkwise_workspace_bytes(128, 512, 8, 64, 64, 64, 1) == 0
    assert lib.ret_chunkwise_workspace_bytes(1, 64, 8, 48, 64, 64, 1) == 0  # unsupported shape: 0


def test_step_and_parallel_reject_invalid_arguments(lib):
    g = np.asarray([0.9], np.float32).ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    assert lib.ret_recurrent_step(16, 32, 48, 64, None, 1, 1, 64, 64, 1, 1, g, None, 0, None) == -1
    assert lib.ret_recurrent_step(16, 32, 48, 64, 80, 1, 1, 64, 66, 1, 1, g, None, 0, None) == -2
    assert lib.ret_recurrent_step(16, 32, 48, 64, 80, 1, 1, 48, 64, 1, 1, g, None, 0, None) == -2
    assert lib.ret_parallel_fwd(16, 32, 48, 64, 1, 8, 1, 48, 64, 1, 1, g, None, 0, None) == -2
    assert lib.ret_parallel_fwd(16, 32, 48, 64, 1, -1, 1, 64, 64, 1, 1, g, None, 0, None) == -1


def test_step_positions_rejects_invalid_arguments(lib):
    g = np.asarray([0.9], np.float32).ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    call = lambda pos=96, dk=64: lib.ret_recurrent_step_positions(16, 32, 48, 64, 80, 1, 1, dk, 64, 1, 1, g, None,
                                                                  pos, None)
    assert call(pos=None) == -1         # positions are required
    assert call(pos=100) == -1          # misaligned positions
    assert call(dk=48) == -2            # no decode tile for d_k = 48


def test_epilogue_rejects_invalid_arguments(lib):
    """ret_msr_epilogue validates on the host; rows = 0 returns OK without a launch."""
    e = lambda *a: lib.ret_msr_epilogue(*a)
    assert e(None, None, None, None, 32, 4, 2, 64, 1, 1, 1, 1e-5, None) == -1           # null o
    assert e(16, None, None, None, None, 4, 2, 64, 1, 1, 1, 1e-5, None) == -1           # null y
    assert e(16, None, None, None, 32, -1, 2, 64, 1, 1, 1, 1e-5, None) == -1            # negative rows
    assert e(16, None, None, None, 32, 4, 0, 64, 1, 1, 1, 1e-5, None) == -1             # no heads
    assert e(16, None, None, None, 32, 4, 2, 64, 1, 1, 1, -1.0, None) == -1             # eps < 0
    assert e(16, None, None, None, 32, 4, 2, 64, 1, 1, 1, float("nan"), None) == -1     # eps NaN
    assert e(16, None, None, None, 32, 4, 2, 64, 1, 1, 7, 1e-5, None) == -1             # bad dtype
    assert e(8, None, None, None, 32, 4, 2, 64, 1, 1, 1, 1e-5, None) == -1              # misaligned o
    assert e(16, 40, None, None, 32, 4, 2, 64, 1, 1, 1, 1e-5, None) == -1               # misaligned gate
    assert e(16, None, None, None, 32, 4, 2, 48, 1, 1, 1, 1e-5, None) == -2             # d_v not supported
    assert e(16, None, None, None, 32, 0, 2, 64, 1, 1, 1, 1e-5, None) == 0              # empty: no launch


def test_chunkwise_msr_rejects_invalid_arguments(lib):
    """ret_chunkwise_msr_fwd checks the epilogue's arguments before anything is launched."""
    g = np.asarray([0.9, 0.99], np.float32).ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    call = lambda gate=None, y=64, dv=64, gdt=1, eps=1e-5, gw=None: lib.ret_chunkwise_msr_fwd(
        16, 32, 48, gate, y, 1, 64, 2, 64, dv, 1, 1, gdt, g, None, 0, 64, None, None, gw, None, eps, None, 0, None)
    assert call(gdt=5) == -1            # bad gate dtype
    assert call(eps=-1.0) == -1         # eps < 0
    assert call(gate=72) == -1          # misaligned gate
    assert call(gw=8) == -1             # misaligned weight
    assert call(gate=64) == -1          # gate aliases y
    assert call(dv=96) == -2            # no epilogue for d_v = 96


def test_gradients_workspace_and_rejections(lib):
    """ret_chunkwise_bwd: workspace size from the shapes, host-side rejections before any launch."""
    wsq = lambda *a, dt=1: lib.ret_chunkwise_bwd_workspace_bytes(*a, dt)
    # d = 64 in short segments (the reversed traversal, rotating while staging): the segment chain alone, no
    # rotated copies of q and k
    n = 8 * 2048 * 8 * 64
    assert 0 < wsq(8, 2048, 8, 64, 64, 64) < 2 * n * 2
    assert wsq(8, 2048, 8, 64, 64, 64) % 256 == 0
    # d_k = 128, N a multiple of 32: the streaming kernel in place, rotating while staging and writing dq and dk
    # itself (the segment states alone: 4 units x 16 segments x 64 KB after the 64 KB of chain metadata);
    # otherwise five reordered bf16 copies (K' twice, Q', V, dO) and three fp32 outputs
    n2 = 1 * 4096 * 4 * 128
    assert wsq(1, 4096, 4, 128, 128, 64) == 65536 + 4 * 16 * 128 * 128 * 4
    n2r = 1 * 4090 * 4 * 128
    assert wsq(1, 4090, 4, 128, 128, 64) >= 5 * n2r * 2 + 3 * n2r * 4
    assert wsq(1, 100, 2, 32, 64, 64) == 0      # d_k = 32: no bf16 kernel
    # d_v = 512 is wider than any retention's d_k: dq' and dk' are sums over two halves of 256. With N a multiple
    # of 32 every retention runs on the three-launch kernels, which read the halves and reversed rows in place:
    # the segment states, Q', K' (bf16) and two fp32 outputs per half
    n4k, n4v = 8192 * 16 * 256, 8192 * 16 * 512
    assert 2 * n4k * 2 + 4 * n4k * 4 <= wsq(1, 8192, 16, 256, 512, 128) < 2 * n4k * 2 + 4 * n4k * 4 + n4v * 4
    # otherwise copies of each half of V and dO, natural and reversed, and two fp32 outputs per half
    n5k, n5v = 8190 * 16 * 256, 8190 * 16 * 512
    assert wsq(1, 8190, 16, 256, 512, 128) >= 3 * n5k * 2 + n5v * 2 + 8 * n5k * 2 + 4 * n5k * 4 + n5v * 4
    assert wsq(1, 100, 2, 64, 1024, 64) == 0     # halves of 512 are still too wide
    assert wsq(1, 0, 2, 64, 64, 64) == 0
    g = np.asarray([0.9, 0.99], np.float32).ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    need = wsq(1, 64, 2, 64, 64, 64)

    def call(q=16, k=32, v=48, do=64, dq=80, dk=96, dv=112, ind=1, outd=0, ws=4096, wsb=None, chunk=64, dkk=64):
        return lib.ret_chunkwise_bwd(q, k, v, do, dq, dk, dv, 1, 64, 2, dkk, 64, ind, outd, g, None, 0, chunk, ws,
                                     need if wsb is None else wsb, None)
    assert call(ind=0, dkk=128) == -2   # fp32 inputs: no fp32 kernel for d_k = 128
    # fp32: five fp32 copies and three fp32 outputs; no fp32 kernel for d_k = 128
    n3 = 2 * 300 * 2 * 32
    assert wsq(2, 300, 2, 32, 32, 32, dt=0) >= 8 * n3 * 4
    assert wsq(2, 300, 2, 128, 64, 64, dt=0) == 0
    assert call(do=None) == -1          # null dout
    assert call(dk=16) == -1            # dk aliases q
    assert call(dv=80) == -1            # dv aliases dq
    assert call(do=72) == -1            # misaligned dout
    assert call(chunk=0) == -1
    assert call(dkk=48) == -2           # no kernel for d_k = 48
    assert call(wsb=need - 256) == -3   # workspace too small
    assert call(ws=None) == -3


def test_library_matches_its_sources(lib):
    """The loaded library was built from the sources in the tree (a stale build is rebuilt or refused)."""
    from linear_recurrent_sequence_amd import build
    lib.ret_source_digest.restype = ctypes.c_char_p
    assert lib.ret_source_digest().decode() == build.source_digest()


def test_options_and_timer_objects(lib):
    """ret_options_default fills the documented defaults; a timer is a caller-owned object that starts empty
    (no GPU call is made)."""
    from linear_recurrent_sequence_amd import retention as R
    o = R.Options()
    lib.ret_options_default(ctypes.byref(o))
    assert (o.segments, o.target_wgs, o.prerotate, o.onchip, o.variant, o.bwd_direct, o.step_cache, o.chain_spin) == \
        (0, 0, -1, 1, 0, 1, 0, 0)
    assert o.timer is None
    t = R.Timer()
    assert t.query("") == (0.0, 0)
    t.reset()
    t.close()
    with pytest.raises(ValueError):
        R._options({"no_such_option": 1})


def test_options_change_the_plan_on_the_host(lib):
    """A forced segment count changes the chunkwise workspace the plan wants (host-side planning only)."""
    from linear_recurrent_sequence_amd import retention as R
    import torch
    n_default = R.ret_chunkwise_workspace_bytes(1, 4096, 2, 64, 64, 64, torch.bfloat16)
    n_one = R.ret_chunkwise_workspace_bytes(1, 4096, 2, 64, 64, 64, torch.bfloat16, options={"segments": 1})
    n_many = R.ret_chunkwise_workspace_bytes(1, 4096, 2, 64, 64, 64, torch.bfloat16, options={"segments": 32})
    assert n_one == 0 and n_many > n_default > 0


# The binding checks shapes and dtypes before it forms any device pointer, so mismatches are caught on CPU
# tensors here (the device check would only come after).
def _cpu_qkv(B=1, N=8, H=2, dk=16, dv=16, dt=None):
    import torch
    dt = dt or torch.float32
    return (torch.zeros(B, N, H, dk, dtype=dt), torch.zeros(B, N, H, dk, dtype=dt), torch.zeros(B, N, H, dv, dtype=dt))


@pytest.mark.parametrize("bad", ["k_shape", "v_heads", "o_shape", "mixed_dtype", "state_shape", "o_dtype"])
def test_binding_rejects_mismatched_tensors(lib, bad):
    import torch
    from linear_recurrent_sequence_amd import retention as R
    q, k, v = _cpu_qkv()
    o = torch.zeros(1, 8, 2, 16)
    state = None
    if bad == "k_shape":
        k = torch.zeros(1, 8, 2, 32)
    elif bad == "v_heads":
        v = torch.zeros(1, 8, 3, 16)
    elif bad == "o_shape":
        o = torch.zeros(1, 4, 2, 16)
    elif bad == "mixed_dtype":
        k = k.to(torch.bfloat16)
    elif bad == "state_shape":
        state = torch.zeros(1, 2, 16, 8)
    elif bad == "o_dtype":
        o = torch.zeros(1, 8, 2, 16, dtype=torch.float64)
    with pytest.raises(ValueError):
        R.ret_chunkwise_fwd(q, k, v, o, [0.9, 0.9], 16, state_out=state)


def test_binding_rejects_mismatched_step_and_gradients(lib):
    import torch
    from linear_recurrent_sequence_amd import retention as R
    q, k, v = (torch.zeros(2, 3, 16) for _ in range(3))
    with pytest.raises(ValueError):  # o of a step is [B, H, d_v]
        R.ret_recurrent_step(q, k, v, torch.zeros(2, 3, 8), torch.zeros(2, 3, 16, 16), [0.9] * 3, pos=0)
    with pytest.raises(ValueError):  # missing state
        R.ret_recurrent_step(q, k, v, torch.zeros(2, 3, 16), None, [0.9] * 3, pos=0)
    q, k, v = _cpu_qkv()
    with pytest.raises(ValueError):  # dv of the wrong shape
        R.ret_chunkwise_bwd(q, k, v, torch.zeros_like(v), torch.zeros_like(q), torch.zeros_like(k),
                            torch.zeros(1, 8, 2, 8), [0.9, 0.9], 16)
