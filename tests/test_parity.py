"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on the same seeded inputs.

Bar (max|gpu - oracle| / max|oracle| over the whole tensor): 1e-5 for fp32 inputs, 2e-2 for bf16 inputs
with fp32 accumulation. Outputs and final states are both checked.
"""
import os

import numpy as np
import pytest

import oracle
from linear_recurrent_sequence_amd import workloads as W
from tests.conftest import print_case
from tests.helpers import empty_out, rel_err, rel_err_per_head, to_dev, to_host, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from linear_recurrent_sequence_amd import retention
    retention.load(build_if_missing=True)
    return retention


def _gpu_chunkwise(R, q, k, v, w_dtype, gamma, chunk, theta=None, pos0=0, s_in=None, dv=None, out_dtype=None,
                   options=None):
    import torch
    qd, kd, vd = to_dev(q, w_dtype), to_dev(k, w_dtype), to_dev(v, w_dtype)
    B, N, H, dk = q.shape
    dv = v.shape[3]
    o = empty_out((B, N, H, dv), out_dtype or w_dtype)
    sin = None if s_in is None else torch.from_numpy(np.ascontiguousarray(s_in, np.float32)).cuda()
    sout = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = R.chunkwise_workspace(qd, vd, chunk, options)
    R.ret_chunkwise_fwd(qd, kd, vd, o, gamma, chunk, theta=theta, pos0=pos0, state_in=sin, state_out=sout,
                        workspace=ws, options=options)
    torch.cuda.synchronize()
    R.ret_chunkwise_check(ws)
    return to_host(o), to_host(sout)


# ---------------------------------------------------------------------------------------------------
# Workload 1: fp32, B=1 N=64 H=8 d=16, no rotation; parallel, recurrent and chunkwise (chunk 16).
# ---------------------------------------------------------------------------------------------------
def test_workload1_all_three_forms(R):
    import torch
    w = W.WORKLOADS[1]
    q, k, v, _ = W.make_qkv(w)
    print_case("workload1", w)
    o_ref, s_ref = oracle.recurrent(q, k, v, w.gamma)
    # chunkwise
    o, s = _gpu_chunkwise(R, q, k, v, "f32", w.gamma, w.chunk)
    assert rel_err(o, o_ref) <= 1e-5 and rel_err(s, s_ref) <= 1e-5, (rel_err(o, o_ref), rel_err(s, s_ref))
    # parallel
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    op = empty_out(v.shape, "f32")
    R.ret_parallel_fwd(qd, kd, vd, op, w.gamma)
    torch.cuda.synchronize()
    assert rel_err(to_host(op), o_ref) <= 1e-5
    # recurrent: 64 single-token steps
    state = torch.zeros((1, 8, 16, 16), dtype=torch.float32, device="cuda")
    outs = []
    for n in range(w.N):
        on = empty_out((1, 8, 16), "f32")
        R.ret_recurrent_step(qd[:, n].contiguous(), kd[:, n].contiguous(), vd[:, n].contiguous(), on, state,
                             w.gamma, pos=n)
        outs.append(on)
    torch.cuda.synchronize()
    orr = np.stack([to_host(x) for x in outs], axis=1)
    assert rel_err(orr, o_ref) <= 1e-5 and rel_err(to_host(state), s_ref) <= 1e-5


# ---------------------------------------------------------------------------------------------------
# Multi-tile shapes with ragged tails, rotation, pos0 and an initial state.
# ---------------------------------------------------------------------------------------------------
SMALL = [
    # dtype, B, N, H, dk, dv, chunk, rotate, pos0, state_in, segments (None = planner)
    ("f32", 2, 200, 3, 32, 48, 32, True, 5, True, None),
    ("f32", 1, 77, 2, 64, 16, 64, True, 0, False, None),
    ("f32", 1, 150, 2, 16, 32, 16, False, 0, True, 3),
    ("bf16", 2, 333, 3, 64, 128, 64, True, 11, True, None),
    ("bf16", 1, 700, 2, 128, 64, 128, True, 0, True, 3),
    ("bf16", 1, 300, 2, 32, 64, 32, True, 3, False, 4),
    ("bf16", 1, 260, 1, 256, 128, 128, True, 0, True, 2),
    ("bf16", 3, 1, 2, 64, 64, 64, True, 9, True, None),      # one token
    ("bf16", 1, 45, 2, 64, 64, 64, False, 0, False, None),   # shorter than one chunk
    ("bf16", 1, 1100, 1, 64, 64, 64, True, 7, False, 1),     # 18 chunks in one segment
    ("bf16", 2, 300, 2, 64, 256, 64, True, 3, True, 3),      # 4 d_v tiles: q, k rotated once up front
    ("bf16", 1, 333, 1, 256, 512, 128, True, 0, True, 2),    # 8 d_v tiles, d_k 256
    # segments of at most 256 tokens with d_k <= 64 run on chip (the whole segment held in LDS and registers)
    ("bf16", 2, 1000, 2, 64, 64, 128, False, 0, True, None),  # chunk 128 as two 64s, ragged last segment
    ("bf16", 1, 2500, 2, 32, 64, 64, True, 0, True, 10),     # 10 segments: two look-back groups
    ("bf16", 1, 530, 3, 64, 192, 32, True, 2, True, 3),      # chunk 32, 3 d_v tiles, 6 chunks per segment
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "%s-B%d-N%d-H%d-dk%d-dv%d-C%d" % c[:7])
def test_chunkwise_small(R, case):
    dt, B, N, H, dk, dv, C, rot, pos0, with_state, segs = case
    print_case("chunkwise_small", case)
    opts = {"segments": segs} if segs is not None else None
    rng = np.random.default_rng(100 + N)
    scale = 1.0 if dt == "f32" else 8.0
    q = W.normal(rng, (B, N, H, dk), scale, dt)
    k = W.normal(rng, (B, N, H, dk), scale, dt)
    v = W.normal(rng, (B, N, H, dv), scale, dt)
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) if with_state else None
    gamma = W.gamma_schedule(H)
    theta = W.theta_schedule(dk) if rot else None
    o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=pos0, state_in=s0)
    o, s = _gpu_chunkwise(R, q, k, v, dt, gamma, C, theta=theta, pos0=pos0, s_in=s0, options=opts)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print("  err o=%.3g state=%.3g" % (eo, es))
    assert eo <= tol(dt) and es <= tol(dt), (eo, es)


@pytest.mark.parametrize("threads", ["wide", "256x2", "512", "256", "dma"])
def test_chunkwise_dk256_workgroup_sizes(R, threads):
    """d_k 256 with d_v tiles of 128 (the wide-head kernel: the default where d_v is not a multiple of 256; the
    chained kernel with 512 threads whose waves own 16 columns, or 256 threads of 32 columns), the 256-thread
    kernels with d_v tiles of 64, and the LDS-loading kernels with d_v tiles of 256 (d_v 512). All match the
    oracle, with two segments."""
    opts = {"variant": {"wide": 0, "512": 4, "256x2": 1, "256": 2, "dma": 5}[threads], "segments": 2}
    B, N, H, dk, dv, C = 1, 300, 2, 256, 384 if threads != "dma" else 512, 64
    print_case("dk256 threads=%s" % threads, (B, N, H, dk, dv, C))
    rng = np.random.default_rng(71)
    q = W.normal(rng, (B, N, H, dk), 16.0, "bf16")
    k = W.normal(rng, (B, N, H, dk), 16.0, "bf16")
    v = W.normal(rng, (B, N, H, dv), 16.0, "bf16")
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
    o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=9, state_in=s0)
    o, s = _gpu_chunkwise(R, q, k, v, "bf16", gamma, C, theta=theta, pos0=9, s_in=s0, options=opts)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print("  err o=%.3g state=%.3g" % (eo, es))
    assert eo <= tol("bf16") and es <= tol("bf16"), (eo, es)


@pytest.mark.parametrize("variant", ["0", "1", "2", "4"])
def test_chunkwise_dk128_tiles(R, variant):
    """d_k 128: d_v tiles of 128 (512 threads x 16 columns: the default; 256 threads x 32 columns) and of 64, with
    rotation while staging, state in and out and three segments, all matching the oracle."""
    opts = {"variant": int(variant), "segments": 3}
    B, N, H, dk, dv, C = 2, 333, 2, 128, 256, 128
    print_case("dk128 variant=%s" % variant, (B, N, H, dk, dv, C))
    rng = np.random.default_rng(73)
    q = W.normal(rng, (B, N, H, dk), 11.0, "bf16")
    k = W.normal(rng, (B, N, H, dk), 11.0, "bf16")
    v = W.normal(rng, (B, N, H, dv), 11.0, "bf16")
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
    o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=4, state_in=s0)
    o, s = _gpu_chunkwise(R, q, k, v, "bf16", gamma, C, theta=theta, pos0=4, s_in=s0, options=opts)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print("  err o=%.3g state=%.3g" % (eo, es))
    assert eo <= tol("bf16") and es <= tol("bf16"), (eo, es)


WIDE = [  # (d_k, B, N, H, d_v, chunk, rotation, state_in, segments)
    (256, 1, 333, 2, 256, 64, True, True, 3),
    (256, 2, 37, 1, 128, 64, True, False, None),
    (256, 1, 1, 2, 128, 32, True, True, None),
    (256, 1, 200, 2, 128, 32, False, True, 2),
    (256, 1, 300, 1, 384, 128, True, False, 2),
    (256, 1, 129, 3, 128, 512, True, True, 1),
    (128, 1, 333, 2, 256, 64, True, True, 3),
    (128, 2, 100, 2, 128, 32, False, False, None),
    (128, 1, 65, 1, 128, 128, True, True, 1),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "dk%d-B%d-N%d-H%d-dv%d-C%d-rot%d-s%d-seg%s" % c)
def test_chunkwise_wide_kernel(R, case):
    """The wide-head kernel (32-token steps, q and k rotated once up front): d_k 128 and 256, chunks of 32 to
    512 tokens, ragged tails shorter than one step, with and without rotation and an incoming state, one or several
    chained segments. Matches the oracle's output and final state."""
    dk, B, N, H, dv, C, rot, with_state, segs = case
    print_case("wide", case)
    opts = {"variant": 3}
    if segs is not None:
        opts["segments"] = segs
    rng = np.random.default_rng(400 + N + dk)
    q = W.normal(rng, (B, N, H, dk), 16.0, "bf16")
    k = W.normal(rng, (B, N, H, dk), 16.0, "bf16")
    v = W.normal(rng, (B, N, H, dv), 16.0, "bf16")
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) if with_state else None
    gamma = W.gamma_schedule(H)
    theta = W.theta_schedule(dk) if rot else None
    o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=5, state_in=s0)
    o, s = _gpu_chunkwise(R, q, k, v, "bf16", gamma, C, theta=theta, pos0=5, s_in=s0, options=opts)
    for h in range(H):
        eo, es = rel_err(o[:, :, h], o_ref[:, :, h]), rel_err(s[:, h], s_ref[:, h])
        print("  head %d err o=%.3g state=%.3g" % (h, eo, es))
        assert eo <= tol("bf16") and es <= tol("bf16"), (h, eo, es)


DMA = [  # (B, N, H, d_v, chunk, rotation, state_in, segments, options)
    (1, 333, 2, 256, 64, True, True, 3, {}),
    (2, 37, 1, 256, 64, True, False, None, {}),
    (1, 1, 2, 512, 32, True, True, None, {}),
    (1, 200, 2, 256, 32, False, True, 2, {}),
    (1, 300, 1, 512, 128, True, False, 2, {}),
    (1, 129, 3, 256, 512, True, True, 1, {}),
    (1, 1000, 2, 256, 128, True, True, 9, {}),
    (1, 333, 2, 256, 64, True, True, 3, {"prerotate": 0}),  # no rotated copies: the 512-thread kernel instead
]


@pytest.mark.parametrize("case", DMA, ids=lambda c: "B%d-N%d-H%d-dv%d-C%d-rot%d-s%d-seg%s-%s" % (
    c[:8] + ("".join("%s%s" % kv for kv in c[8].items()) or "default",)))
def test_chunkwise_dma_kernel(R, case):
    """The LDS-loading wide-head kernel (d_k 256, d_v tiles of 256, variant 5): ragged tails shorter than
    one step, with and without rotation and an incoming state, one to nine chained segments, chunks of 32 to 512
    tokens; and the same call without room for rotated copies, which takes the 512-thread kernel. Matches the
    oracle's output and final state per head."""
    B, N, H, dv, C, rot, with_state, segs, extra = case
    dk = 256
    print_case("dma", case)
    opts = dict(extra, variant=5)
    if segs is not None:
        opts["segments"] = segs
    rng = np.random.default_rng(700 + N + dv)
    q = W.normal(rng, (B, N, H, dk), 16.0, "bf16")
    k = W.normal(rng, (B, N, H, dk), 16.0, "bf16")
    v = W.normal(rng, (B, N, H, dv), 16.0, "bf16")
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) if with_state else None
    gamma = W.gamma_schedule(H)
    theta = W.theta_schedule(dk) if rot else None
    o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=3, state_in=s0)
    o, s = _gpu_chunkwise(R, q, k, v, "bf16", gamma, C, theta=theta, pos0=3, s_in=s0, options=opts)
    for h in range(H):
        eo, es = rel_err(o[:, :, h], o_ref[:, :, h]), rel_err(s[:, h], s_ref[:, h])
        print("  head %d err o=%.3g state=%.3g" % (h, eo, es))
        assert eo <= tol("bf16") and es <= tol("bf16"), (h, eo, es)


def test_chunkwise_dma_kernel_is_launched(R):
    """d_k 256 with d_v 512 and variant 5: the plan launches the LDS-loading kernel (timer name ret_chunk_dma),
    after the up-front rotation."""
    import torch
    B, N, H, dk, dv, C = 1, 256, 2, 256, 512, 128
    rng = np.random.default_rng(5)
    q = to_dev(W.normal(rng, (B, N, H, dk), 8.0, "bf16"), "bf16")
    k = to_dev(W.normal(rng, (B, N, H, dk), 8.0, "bf16"), "bf16")
    v = to_dev(W.normal(rng, (B, N, H, dv), 8.0, "bf16"), "bf16")
    o = empty_out((B, N, H, dv), "bf16")
    timer = R.Timer()
    R.ret_chunkwise_fwd(q, k, v, o, W.gamma_schedule(H), C, theta=W.theta_schedule(dk),
                        workspace=R.chunkwise_workspace(q, v, C, {"variant": 5}), options={"timer": timer, "variant": 5})
    torch.cuda.synchronize()
    assert timer.query("ret_chunk_dma")[1] == 1 and timer.query("ret_rotate_qk")[1] == 1
    timer.close()


@pytest.mark.parametrize("onchip", ["1", "0"])
@pytest.mark.parametrize("pre", ["1", "0"])
def test_chunkwise_prerotation_either_way(R, pre, onchip):
    """q and k rotated once into the workspace (prerotate 1) or while staging (0), on a shape with 4 d_v tiles
    and two segments, in the on-chip and the streaming kernel: all match the oracle."""
    opts = {"prerotate": int(pre), "onchip": int(onchip), "segments": 2}
    B, N, H, dk, dv, C = 1, 333, 2, 64, 256, 64
    print_case("prerotation=%s onchip=%s" % (pre, onchip), (B, N, H, dk, dv, C))
    rng = np.random.default_rng(83)
    q = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
    k = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
    v = W.normal(rng, (B, N, H, dv), 8.0, "bf16")
    gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
    o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=21)
    o, s = _gpu_chunkwise(R, q, k, v, "bf16", gamma, C, theta=theta, pos0=21, options=opts)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print("  err o=%.3g state=%.3g" % (eo, es))
    assert eo <= tol("bf16") and es <= tol("bf16"), (eo, es)


@pytest.mark.parametrize("onchip", ["1", "0"])
def test_chunkwise_short_segments_either_kernel(R, onchip):
    """Segments of at most 256 tokens: the on-chip kernel (default) and the streaming single-pass kernel
    (onchip 0) give the oracle's result on the same inputs, with a state handed in and out."""
    opts = {"onchip": int(onchip)}
    B, N, H, dk, dv, C = 2, 1234, 2, 64, 128, 64
    print_case("short_segments onchip=%s" % onchip, (B, N, H, dk, dv, C))
    rng = np.random.default_rng(57)
    q = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
    k = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
    v = W.normal(rng, (B, N, H, dv), 8.0, "bf16")
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
    o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=40, state_in=s0)
    o, s = _gpu_chunkwise(R, q, k, v, "bf16", gamma, C, theta=theta, pos0=40, s_in=s0, options=opts)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print("  err o=%.3g state=%.3g" % (eo, es))
    assert eo <= tol("bf16") and es <= tol("bf16"), (eo, es)


@pytest.mark.parametrize("dk", [128, 256])
def test_chunkwise_wide_dv_without_workspace(R, dk):
    """Without a workspace a call runs one segment per (b, h) and rotates q and k while staging, also where a
    full workspace would hold rotated copies (8 or 4 d_v tiles)."""
    B, N, H, dv, C = 1, 200, 2, 512, 64
    print_case("wide_dv_no_workspace", (B, N, H, dk, dv, C))
    rng = np.random.default_rng(31)
    q = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
    k = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
    v = W.normal(rng, (B, N, H, dv), 8.0, "bf16")
    gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
    o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=17)
    import torch
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o = empty_out((B, N, H, dv), "bf16")
    sout = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    R.ret_chunkwise_fwd(qd, kd, vd, o, gamma, C, theta=theta, pos0=17, state_out=sout, workspace=None)
    torch.cuda.synchronize()
    assert rel_err(to_host(o), o_ref) <= tol("bf16") and rel_err(to_host(sout), s_ref) <= tol("bf16")


def test_chunkwise_workspace_reuse_and_repeatability(R):
    """One workspace serves repeated calls and a call of another shape: every call leaves it ready for the
    next. 11 and 9 segments span two look-back groups, so the prefix handed across a group boundary is
    used. The segment states are summed in a fixed order, so repeated calls give identical bits."""
    import torch
    cases = [(2, 1400, 2, 64, 128, 64, 11), (1, 1150, 2, 128, 64, 128, 9)]
    ws_bytes = 0
    for B, N, H, dk, dv, C, segs in cases:
        ws_bytes = max(ws_bytes, R.ret_chunkwise_workspace_bytes(B, N, H, dk, dv, C, options={"segments": segs}))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    for B, N, H, dk, dv, C, segs in cases:
        print_case("workspace_reuse", (B, N, H, dk, dv, C, segs))
        opts = {"segments": segs}
        rng = np.random.default_rng(7 + N)
        q = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
        k = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
        v = W.normal(rng, (B, N, H, dv), 8.0, "bf16")
        s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
        gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
        o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=5, state_in=s0)
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        sin = torch.from_numpy(s0).cuda()
        runs = []
        for _ in range(3):
            o = empty_out((B, N, H, dv), "bf16")
            sout = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
            R.ret_chunkwise_fwd(qd, kd, vd, o, gamma, C, theta=theta, pos0=5, state_in=sin, state_out=sout,
                                workspace=ws, options=opts)
            torch.cuda.synchronize()
            R.ret_chunkwise_check(ws)
            runs.append((to_host(o), to_host(sout)))
        for o, sout in runs:
            assert rel_err(o, o_ref) <= tol("bf16") and rel_err(sout, s_ref) <= tol("bf16")
        for o, sout in runs[1:]:
            assert np.array_equal(o, runs[0][0]) and np.array_equal(sout, runs[0][1])
        units = B * H * (dv // 64)
        up = lambda n: (n + 255) // 256 * 256
        hdr = ws[:256 + up(units * 8) + up(units * segs * 4)].cpu().numpy().view(np.int32)
        assert (hdr == 0).all(), hdr[:4]  # error word, per-unit tickets and counters, slot flags back at zero


@pytest.mark.parametrize("dt,dk,dv", [("f32", 32, 32), ("bf16", 64, 64), ("bf16", 256, 128)])
def test_parallel_small(R, dt, dk, dv):
    import torch
    print_case("parallel_small", dt, dk, dv)
    rng = np.random.default_rng(7)
    B, N, H = 2, 150, 2
    scale = 1.0 if dt == "f32" else 8.0
    q = W.normal(rng, (B, N, H, dk), scale, dt)
    k = W.normal(rng, (B, N, H, dk), scale, dt)
    v = W.normal(rng, (B, N, H, dv), scale, dt)
    gamma = np.array([0.9, 0.999], np.float32)
    theta = W.theta_schedule(dk)
    ref = oracle.parallel(q, k, v, gamma, theta=theta, pos0=3)
    o = empty_out((B, N, H, dv), dt)
    R.ret_parallel_fwd(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), o, gamma, theta=theta, pos0=3)
    torch.cuda.synchronize()
    assert rel_err(to_host(o), ref) <= tol(dt)


# decode tiles: state columns and rows per wave (the library widens tiles too small for a shape); pairs "2"
# forces workgroups of several (b, h) pairs, here with a partial last workgroup (6 pairs); cache "1" the state's
# accesses without the non-temporal hint
@pytest.mark.parametrize("cache", ["0", "1"])
@pytest.mark.parametrize("pairs", ["0", "2"])
@pytest.mark.parametrize("cw,wr", [("16", "64"), ("32", "64"), ("64", "64"), ("32", "32"), ("32", "16"),
                                   ("64", "16")])
@pytest.mark.parametrize("dt,dk,dv", [("f32", 16, 16), ("f32", 64, 36), ("bf16", 64, 64), ("bf16", 128, 128),
                                      ("bf16", 256, 200)])
def test_recurrent_steps_small(R, dt, dk, dv, cw, wr, pairs, cache):
    import torch
    print_case("recurrent_small", dt, dk, dv, cw, wr, pairs, cache)
    opts = {"step_cw": int(cw), "step_wr": int(wr), "step_pairs": int(pairs), "step_cache": int(cache)}
    rng = np.random.default_rng(9)
    B, H, n = 3, 2, 20
    scale = 1.0 if dt == "f32" else 8.0
    q = W.normal(rng, (B, n, H, dk), scale, dt)
    k = W.normal(rng, (B, n, H, dk), scale, dt)
    v = W.normal(rng, (B, n, H, dv), scale, dt)
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    gamma = np.array([0.95, 1.0], np.float32)
    theta = W.theta_schedule(dk)
    o_ref, s_ref = oracle.recurrent(q, k, v, gamma, theta=theta, pos0=1000, state_in=s0)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    state = torch.from_numpy(s0).cuda()
    outs = []
    for t in range(n):
        o = empty_out((B, H, dv), dt)
        R.ret_recurrent_step(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), o, state, gamma,
                             pos=1000 + t, theta=theta, options=opts)
        outs.append(o)
    torch.cuda.synchronize()
    got = np.stack([to_host(x) for x in outs], axis=1)
    assert rel_err(got, o_ref) <= tol(dt) and rel_err(to_host(state), s_ref) <= tol(dt)


# ---------------------------------------------------------------------------------------------------
# Multi-scale retention epilogue: y = swish(gate) (.) GroupNorm_h(o).
# ---------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("affine,gated", [(True, True), (False, True), (True, False), (False, False)])
@pytest.mark.parametrize("dts", [("bf16", "bf16", "bf16"), ("f32", "f32", "f32"), ("f32", "bf16", "bf16"),
                                 ("bf16", "f32", "f32")])
@pytest.mark.parametrize("dv", [16, 64, 128, 512])
def test_msr_epilogue(R, dv, dts, affine, gated):
    """Rows of 3 heads, 37 tokens (a partial last workgroup), every dtype mix, with and without the
    per-channel affine and the gate."""
    import torch
    o_dt, g_dt, y_dt = dts
    print_case("msr_epilogue", dv, dts, affine, gated)
    rng = np.random.default_rng(300 + dv)
    rows, H = 37, 3
    # rows of very different scales and offsets, held exactly in the input dtype
    o = W.round_to(rng.standard_normal((rows, H, dv)) * rng.uniform(0.05, 20.0, size=(rows, H, 1))
                   + rng.uniform(-3.0, 3.0, size=(rows, H, 1)), o_dt)
    g = W.normal(rng, (rows, H, dv), 0.5, g_dt) if gated else None
    w = rng.standard_normal(H * dv).astype(np.float32) if affine else None
    b = rng.standard_normal(H * dv).astype(np.float32) if affine else None
    ref = oracle.msr_epilogue(o, g, w, b, eps=1e-5)
    y = empty_out((rows, H, dv), y_dt)
    td = lambda a: None if a is None else torch.from_numpy(a).cuda()
    R.ret_msr_epilogue(to_dev(o, o_dt), y, gate=None if g is None else to_dev(g, g_dt), gn_weight=td(w),
                       gn_bias=td(b), eps=1e-5)
    torch.cuda.synchronize()
    err = rel_err(to_host(y), ref)
    print("  err %.3g" % err)
    assert err <= tol(y_dt), err


def test_msr_epilogue_in_place_and_decode_rows(R):
    """y = o in place, on the rows of one decode step ([B, H, d_v]), eps 0.1."""
    import torch
    rng = np.random.default_rng(41)
    B, H, dv = 5, 4, 64
    o = W.normal(rng, (B, H, dv), 1.0, "f32")
    g = W.normal(rng, (B, H, dv), 1.0, "f32")
    ref = oracle.msr_epilogue(o, g, eps=0.1)
    od = to_dev(o, "f32")
    R.ret_msr_epilogue(od, od, gate=to_dev(g, "f32"), eps=0.1)
    torch.cuda.synchronize()
    assert rel_err(to_host(od), ref) <= 1e-5


def test_msr_layer_chunkwise_then_epilogue(R):
    """retention-layer-d512 in full: the chunkwise forward, then the epilogue with a gate and per-channel
    affine, against the oracle's chunkwise form and epilogue."""
    import torch
    w = W.WORKLOADS[2]
    print_case("msr_layer", w)
    q, k, v, rng = W.make_qkv(w)
    gate = W.normal(rng, (w.B, w.N, w.H, w.dv), 1.0, "bf16")
    gw = rng.uniform(0.5, 1.5, w.H * w.dv).astype(np.float32)
    gb = (0.1 * rng.standard_normal(w.H * w.dv)).astype(np.float32)
    o_ref, _ = oracle.chunkwise(q, k, v, w.gamma, w.chunk, theta=w.theta)
    y_ref = oracle.msr_epilogue(o_ref, gate, gw, gb, eps=1e-5)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o = empty_out((w.B, w.N, w.H, w.dv), "bf16")
    R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, w.chunk, theta=w.theta, workspace=R.chunkwise_workspace(qd, vd, w.chunk))
    y = empty_out((w.B, w.N, w.H, w.dv), "bf16")
    R.ret_msr_epilogue(o, y, gate=to_dev(gate, "bf16"), gn_weight=torch.from_numpy(gw).cuda(),
                       gn_bias=torch.from_numpy(gb).cuda(), eps=1e-5)
    torch.cuda.synchronize()
    err = rel_err(to_host(y), y_ref)
    print("  err %.3g" % err)
    assert err <= 2e-2, err


@pytest.mark.parametrize("gate_dt,affine", [("bf16", True), ("f32", True), (None, True), ("bf16", False)])
def test_chunkwise_msr_fused(R, gate_dt, affine):
    """retention-layer-d512 through ret_chunkwise_msr_fwd: the on-chip kernel applies the epilogue before its
    stores. Against the oracle, and bit for bit against the chunkwise call followed by ret_msr_epilogue (the
    same bf16 outputs, the same reduction order over 8 lanes of 8 values)."""
    import torch
    w = W.WORKLOADS[2]
    print_case("chunkwise_msr_fused", gate_dt, affine)
    q, k, v, rng = W.make_qkv(w)
    gate = None if gate_dt is None else W.normal(rng, (w.B, w.N, w.H, w.dv), 1.0, gate_dt)
    gw = rng.uniform(0.5, 1.5, w.H * w.dv).astype(np.float32) if affine else None
    gb = (0.1 * rng.standard_normal(w.H * w.dv)).astype(np.float32) if affine else None
    o_ref, _ = oracle.chunkwise(q, k, v, w.gamma, w.chunk, theta=w.theta)
    y_ref = oracle.msr_epilogue(o_ref, gate, gw, gb, eps=1e-5)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    gd = None if gate is None else to_dev(gate, gate_dt)
    td = lambda a: None if a is None else torch.from_numpy(a).cuda()
    ws = R.chunkwise_workspace(qd, vd, w.chunk)
    y = empty_out((w.B, w.N, w.H, w.dv), "bf16")
    R.ret_chunkwise_msr_fwd(qd, kd, vd, y, w.gamma, w.chunk, gate=gd, gn_weight=td(gw), gn_bias=td(gb), eps=1e-5,
                            theta=w.theta, workspace=ws)
    o = empty_out((w.B, w.N, w.H, w.dv), "bf16")
    R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, w.chunk, theta=w.theta, workspace=ws)
    y2 = empty_out((w.B, w.N, w.H, w.dv), "bf16")
    R.ret_msr_epilogue(o, y2, gate=gd, gn_weight=td(gw), gn_bias=td(gb), eps=1e-5)
    torch.cuda.synchronize()
    R.ret_chunkwise_check(ws)
    err = rel_err(to_host(y), y_ref)
    print("  err %.3g" % err)
    assert err <= 2e-2, err
    assert torch.equal(y, y2)


@pytest.mark.parametrize("case", ["dv128", "f32_out", "streaming_kernel", "f32_in"])
def test_chunkwise_msr_unfused(R, case):
    """Shapes the kernels cannot fuse (two d_v tiles per head, fp32 output, the streaming kernel, fp32 input):
    the chunkwise call, then the epilogue over y in place, against the oracle."""
    import torch
    B, N, H, dk, dv, C, dt, odt = 2, 300, 2, 64, 64, 64, "bf16", "bf16"
    opts = None
    if case == "dv128":
        dv = 128
    elif case == "f32_out":
        odt = "f32"
    elif case == "streaming_kernel":
        opts = {"onchip": 0, "segments": 2}
    else:
        dt, odt, dk, C = "f32", "f32", 32, 32
    print_case("chunkwise_msr_unfused", case)
    rng = np.random.default_rng(61)
    q = W.normal(rng, (B, N, H, dk), 8.0, dt)
    k = W.normal(rng, (B, N, H, dk), 8.0, dt)
    v = W.normal(rng, (B, N, H, dv), 8.0, dt)
    gate = W.normal(rng, (B, N, H, dv), 1.0, "bf16")
    gw = rng.uniform(0.5, 1.5, H * dv).astype(np.float32)
    gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=4, state_in=s0)
    # the epilogue reads O as rounded to the output dtype
    y_ref = oracle.msr_epilogue(W.round_to(o_ref, odt) if odt == "bf16" else o_ref, gate, gw, None, eps=1e-5)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    y = empty_out((B, N, H, dv), odt)
    sout = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = R.chunkwise_workspace(qd, vd, C, opts)
    R.ret_chunkwise_msr_fwd(qd, kd, vd, y, gamma, C, gate=to_dev(gate, "bf16"), gn_weight=torch.from_numpy(gw).cuda(),
                            eps=1e-5, theta=theta, pos0=4, state_in=torch.from_numpy(s0).cuda(), state_out=sout,
                            workspace=ws, options=opts)
    torch.cuda.synchronize()
    err, es = rel_err(to_host(y), y_ref), rel_err(to_host(sout), s_ref)
    print("  err %.3g state %.3g" % (err, es))
    assert err <= tol(dt) and es <= tol(dt), (err, es)  # the bar of the input dtype, as for the chunkwise form


# ---------------------------------------------------------------------------------------------------
# Full-size workloads 2-5.
# ---------------------------------------------------------------------------------------------------
def test_workload2_chunkwise_full(R):
    w = W.WORKLOADS[2]
    print_case("workload2", w)
    q, k, v, _ = W.make_qkv(w)
    o_ref, s_ref = oracle.chunkwise(q, k, v, w.gamma, w.chunk, theta=w.theta)
    o, s = _gpu_chunkwise(R, q, k, v, w.dtype, w.gamma, w.chunk, theta=w.theta)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    ph = rel_err_per_head(o, o_ref)
    print("  err o=%.3g state=%.3g" % (eo, es))
    print("  per head:", " ".join("%.2e" % e for e in ph))
    assert eo <= 2e-2 and es <= 2e-2
    assert max(ph) <= 2e-2, ph  # each head at the bar on its own scale


def test_workload3_prefill_then_1024_decode_steps(R):
    import torch
    w = W.WORKLOADS[3]
    print_case("workload3", w)
    q, k, v, rng = W.make_qkv(w)
    steps = [W.make_step(w, rng) for _ in range(w.steps)]
    sq = np.stack([s[0] for s in steps], axis=1)
    sk = np.stack([s[1] for s in steps], axis=1)
    sv = np.stack([s[2] for s in steps], axis=1)
    _, s_pre = oracle.chunkwise(q, k, v, w.gamma, w.chunk, theta=w.theta)
    o_ref, s_ref = oracle.recurrent(sq, sk, sv, w.gamma, theta=w.theta, pos0=w.prefill, state_in=s_pre)
    # GPU: chunkwise prefill, then the decode steps from the GPU's own state
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o = empty_out(v.shape, "bf16")
    state = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, w.chunk, theta=w.theta, state_out=state,
                        workspace=R.chunkwise_workspace(qd, vd, w.chunk))
    torch.cuda.synchronize()
    assert rel_err(to_host(state), s_pre) <= 2e-2
    sqd = to_dev(np.ascontiguousarray(sq.transpose(1, 0, 2, 3)), "bf16")
    skd = to_dev(np.ascontiguousarray(sk.transpose(1, 0, 2, 3)), "bf16")
    svd = to_dev(np.ascontiguousarray(sv.transpose(1, 0, 2, 3)), "bf16")
    outs = torch.empty((w.steps, w.B, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    for t in range(w.steps):
        R.ret_recurrent_step(sqd[t], skd[t], svd[t], outs[t], state, w.gamma, pos=w.prefill + t, theta=w.theta)
    torch.cuda.synchronize()
    got = to_host(outs).transpose(1, 0, 2, 3)
    eo, es = rel_err(got, o_ref), rel_err(to_host(state), s_ref)
    print("  err o=%.3g state=%.3g" % (eo, es))
    assert eo <= 2e-2 and es <= 2e-2


def test_workload4_chunkwise_full(R):
    w = W.WORKLOADS[4]
    print_case("workload4", w)
    q, k, v, _ = W.make_qkv(w)
    o_ref, s_ref = oracle.chunkwise(q, k, v, w.gamma, w.chunk, theta=w.theta)
    o, s = _gpu_chunkwise(R, q, k, v, w.dtype, w.gamma, w.chunk, theta=w.theta)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    ph = rel_err_per_head(o, o_ref)
    print("  err o=%.3g state=%.3g" % (eo, es))
    print("  per head:", " ".join("%.2e" % e for e in ph))
    assert eo <= 2e-2 and es <= 2e-2
    assert max(ph) <= 2e-2, ph  # each head at the bar on its own scale


def test_workload5_long_sequence_then_256_decode_steps(R):
    import torch
    w = W.WORKLOADS[5]
    print_case("workload5", w)
    q, k, v, rng = W.make_qkv(w)
    steps = [W.make_step(w, rng) for _ in range(w.steps)]
    o_ref, s_ref = oracle.chunkwise(q, k, v, w.gamma, w.chunk, theta=w.theta)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    del q, k, v
    o = empty_out(o_ref.shape, "bf16")
    state = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, w.chunk, theta=w.theta, state_out=state,
                        workspace=R.chunkwise_workspace(qd, vd, w.chunk))
    torch.cuda.synchronize()
    oh = to_host(o)
    eo, es = rel_err(oh, o_ref), rel_err(to_host(state), s_ref)
    ph = rel_err_per_head(oh, o_ref)
    print("  chunkwise err o=%.3g state=%.3g" % (eo, es))
    print("  per head:", " ".join("%.2e" % e for e in ph))
    assert eo <= 2e-2 and es <= 2e-2
    assert max(ph) <= 2e-2, ph
    del o_ref, oh
    sq = np.stack([s[0] for s in steps], axis=1)
    sk = np.stack([s[1] for s in steps], axis=1)
    sv = np.stack([s[2] for s in steps], axis=1)
    od_ref, sd_ref = oracle.recurrent(sq, sk, sv, w.gamma, theta=w.theta, pos0=w.N, state_in=s_ref)
    outs = []
    for t in range(w.steps):
        ot = empty_out((w.B, w.H, w.dv), "bf16")
        R.ret_recurrent_step(to_dev(sq[:, t], "bf16"), to_dev(sk[:, t], "bf16"), to_dev(sv[:, t], "bf16"), ot, state,
                             w.gamma, pos=w.N + t, theta=w.theta)
        outs.append(ot)
    torch.cuda.synchronize()
    got = np.stack([to_host(x) for x in outs], axis=1)
    ed, esd = rel_err(got, od_ref), rel_err(to_host(state), sd_ref)
    print("  decode err o=%.3g state=%.3g" % (ed, esd))
    assert ed <= 2e-2 and esd <= 2e-2


def test_workspace_shared_by_calls_of_different_shapes(R):
    """One workspace for calls of different shapes in turn: a small chain layout (2 units), a large one (64
    units, whose counters and flags would lie over the small layout's state slots if these were not kept
    apart), then the small one again; each against the oracle."""
    import torch
    print_case("workspace_shared")
    rng = np.random.default_rng(71)
    shapes = [(1, 2048, 2, 64, 64), (8, 2048, 8, 64, 64), (1, 2048, 2, 64, 64)]
    need = max(R.load().ret_chunkwise_workspace_bytes(b, n, h, dk, dv, 64, R.RET_BF16) for b, n, h, dk, dv in shapes)
    ws = torch.zeros((need,), dtype=torch.uint8, device="cuda")
    for i, (B, N, H, dk, dv) in enumerate(shapes):
        q = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
        k = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
        v = W.normal(rng, (B, N, H, dv), 8.0, "bf16")
        gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        o = empty_out((B, N, H, dv), "bf16")
        R.ret_chunkwise_fwd(qd, kd, vd, o, gamma, 64, theta=theta, workspace=ws)
        torch.cuda.synchronize()
        R.ret_chunkwise_check(ws)
        o_ref, _ = oracle.chunkwise(q, k, v, gamma, 64, theta=theta)
        e = rel_err(to_host(o), o_ref)
        print("  call %d %s: err %.3g" % (i, (B, N, H, dk, dv), e))
        assert e <= tol("bf16"), (i, e)
