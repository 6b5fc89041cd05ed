"""GPU parity of the gradients of chunkwise retention (ret_chunkwise_bwd, through the C ABI) against the fp64
oracle's adjoint scan on the same seeded inputs.

Bar: max|gpu - oracle| / max|oracle| <= 2e-2 for each of dq, dk, dv (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest

import oracle
from linear_recurrent_sequence_amd import workloads as W
from tests.conftest import print_case
from tests.helpers import empty_out, rel_err, to_dev, to_host, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from linear_recurrent_sequence_amd import retention
    retention.load(build_if_missing=True)
    return retention


def _gpu_grad(R, q, k, v, do, gamma, chunk, theta, pos0, out_dt, workspace=None, in_dt="bf16", options=None):
    import torch
    qd, kd, vd, dod = (to_dev(x, in_dt) for x in (q, k, v, do))
    dq, dk, dv = empty_out(q.shape, out_dt), empty_out(k.shape, out_dt), empty_out(v.shape, out_dt)
    R.ret_chunkwise_bwd(qd, kd, vd, dod, dq, dk, dv, gamma, chunk, theta=theta, pos0=pos0, workspace=workspace,
                        options=options, check=workspace is None)
    torch.cuda.synchronize()
    return to_host(dq), to_host(dk), to_host(dv)


def _check(got, ref, bar):
    errs = [rel_err(g, r) for g, r in zip(got, ref)]
    print("  err dq=%.3g dk=%.3g dv=%.3g" % tuple(errs))
    assert max(errs) <= bar, errs


GRAD_SMALL = [
    # B, N, H, dk, dv, chunk, rotate, pos0, out dtype
    (2, 200, 3, 64, 64, 64, True, 7, "f32"),    # ragged last chunk, rotation from position 7
    (1, 333, 2, 128, 64, 64, True, 0, "f32"),   # d_k > d_v: the dq and dk retentions run with d_k, d_v swapped
    (1, 130, 2, 64, 128, 32, False, 0, "f32"),  # d_v > d_k, chunk 32
    (1, 300, 1, 256, 256, 128, True, 3, "f32"),
    (2, 150, 2, 64, 64, 64, True, 11, "bf16"),  # bf16 gradients
    (1, 1, 2, 64, 64, 64, True, 5, "f32"),      # one token
    (3, 64, 2, 64, 64, 64, True, 0, "f32"),     # exactly one chunk
    # d = 64 in several short segments: the reversed traversal (no reordered copies)
    (2, 700, 4, 64, 64, 64, True, 9, "f32"),
    (1, 1000, 3, 64, 64, 32, True, 0, "bf16"),  # chunk 32
    (2, 600, 2, 64, 64, 64, False, 0, "bf16"),  # no rotation: dq and dk written by the retentions themselves
    (1, 777, 2, 64, 64, 128, True, 4, "f32"),   # chunk 128 as 64-token sub-chunks
    # d_v = 512 (the paper's head: d_k 256, d_v 512): dq' and dk' as sums over two halves of d_v
    (1, 700, 2, 256, 512, 128, True, 5, "bf16"),
    (2, 300, 1, 128, 512, 64, False, 0, "f32"),
]


@pytest.mark.parametrize("case", GRAD_SMALL, ids=lambda c: "B%d-N%d-H%d-dk%d-dv%d-C%d" % c[:6] + "-" + c[8])
def test_gradients_small(R, case):
    B, N, H, dk, dv, chunk, rot, pos0, out_dt = case
    w = W.Workload("grad", B=B, N=N, H=H, dk=dk, dv=dv, dtype="bf16", scale=float(np.sqrt(dk)), seed=31 + N,
                   chunk=chunk, rotate=rot)
    print_case("gradients", w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=pos0)
    got = _gpu_grad(R, q, k, v, do, w.gamma, chunk, w.theta, pos0, out_dt)
    _check(got, ref, tol("bf16"))


GRAD_IN_PLACE = [
    # B, N, H, dk, dv, chunk, rotate, pos0, out dtype, kernel, several segments, final reordering launches. N a
    # multiple of 32: every retention runs over the reversed sequence in place on the kernel named, with no
    # reordered copies. d_k 256 with d_v a multiple of 256: the three-launch kernels, which also read the d_v blocks
    # of dO and V in place, and with several segments dq' and dk' of every block each in one launch from transposed
    # states (of a local pass and scan over K' and V, and of the dv retention); otherwise (one block) the
    # single-pass kernels' reversed instances: the streaming kernel with d_v tiles of 128 for d_k = 128, the
    # wide-head kernel for d_k = 256. Where the dq' and dk' retentions run on the streaming kernel, it writes dq and
    # dk itself, turned back by the transpose rotation: no final reordering launch; and where the dv retention runs
    # on it too, every retention rotates its operands while staging: no up-front rotation either.
    (1, 640, 2, 256, 512, 128, True, 5, "bf16", "ret_chunk_dma", True, 1),   # 5 segments, two d_v blocks
    (2, 512, 2, 256, 256, 64, True, 0, "f32", "ret_chunk_dma", True, 1),     # one block
    (1, 1024, 1, 256, 512, 32, False, 0, "f32", "ret_chunk_dma", True, 1),   # no rotation, chunk 32
    (1, 32, 2, 256, 512, 128, True, 9, "f32", "ret_chunk_dma", False, 1),    # one step
    (1, 640, 2, 128, 128, 128, True, 5, "bf16", "ret_chunk_fused", True, 0),  # the long-sequence head
    (1, 512, 2, 128, 256, 64, True, 0, "f32", "ret_chunk_fused", True, 1),    # d_k < d_v (d_k 256 runs: wide)
    (2, 384, 1, 256, 128, 32, False, 0, "f32", "ret_chunk_fused", True, 0),   # d_k > d_v, chunk 32
]


@pytest.mark.parametrize("case", GRAD_IN_PLACE, ids=lambda c: "B%d-N%d-H%d-dk%d-dv%d-C%d" % c[:6] + "-" + c[8])
def test_gradients_in_place(R, case):
    """Gradients with no reordered copies: the only reordering launch left is the one that sums the d_v blocks'
    dq' and dk' and turns them back by the transpose rotation, and none where the retentions' kernel does that."""
    B, N, H, dk, dv, chunk, rot, pos0, out_dt, kernel, multi, nperm = case
    w = W.Workload("grad", B=B, N=N, H=H, dk=dk, dv=dv, dtype="bf16", scale=float(np.sqrt(dk)), seed=61 + N,
                   chunk=chunk, rotate=rot)
    print_case("gradients-in-place", kernel, w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=pos0)
    timer = R.Timer()
    got = _gpu_grad(R, q, k, v, do, w.gamma, chunk, w.theta, pos0, out_dt, options={"timer": timer})
    assert timer.query("ret_permute_rotate")[1] == nperm
    assert timer.query("ret_rotate_qk")[1] == (1 if rot and nperm else 0)
    if kernel == "ret_chunk_dma":
        nb = dv // 256
        # dq' per block, dv, then dk' per block; or (several segments) the states of (K', V), dq' of all blocks,
        # dv, dk' of all blocks
        assert timer.query(kernel)[1] == (3 if multi else 2 * nb + 1)
        assert timer.query("ret_chunk_dma_local")[1] == (2 if multi else 0)
        assert timer.query("ret_chunk_dma_scan")[1] == (2 if multi else 0)
    else:
        assert timer.query(kernel)[1] >= 1
        assert timer.query("ret_chunk_fused")[1] + timer.query("ret_chunk_wide")[1] == 3
    timer.close()
    _check(got, ref, tol("bf16"))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gradients_streaming_seeded_shapes(R, seed):
    """The streaming kernel's gradient path (rotation while staging, outputs turned back in the kernel, dk' from
    the dv retention's states) on seeded shapes: N a multiple of 64 from 1024 to 6144, 1 or 2 heads, 2 to 5
    segments (segments of 3 to 48 chunks, so the rotation factors are carried across groups of 8 and re-evaluated
    mid-segment), a position offset up to 2^20, bf16 or fp32 gradients."""
    rng0 = np.random.default_rng(1000 + seed)
    N = int(rng0.integers(16, 97)) * 64
    H = int(rng0.integers(1, 3))
    nseg = int(rng0.integers(2, 6))
    pos0 = int(rng0.integers(0, 1 << 20))
    out_dt = ["bf16", "f32"][seed % 2]
    w = W.Workload("grad", B=1, N=N, H=H, dk=128, dv=128, dtype="bf16", scale=float(np.sqrt(128)), seed=91 + seed,
                   chunk=128, rotate=True)
    print_case("gradients-streaming-seeded", (N, H, nseg, pos0, out_dt), w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=pos0)
    timer = R.Timer()
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, pos0, out_dt, options={"timer": timer, "segments": nseg})
    assert timer.query("ret_permute_rotate")[1] == 0 and timer.query("ret_rotate_qk")[1] == 0
    timer.close()
    _check(got, ref, tol("bf16"))


@pytest.mark.parametrize("N", [1000, 1056])
def test_gradients_dk128_other_lengths(R, N):
    """d_k = d_v = 128 where the streaming kernel's reversed instances do not apply (N not a multiple of its 64-token
    step): 1056, a multiple of 32, runs in place on the wide-head kernels with the final reordering launch; 1000
    through reordered copies. Both match the oracle."""
    w = W.Workload("grad", B=1, N=N, H=2, dk=128, dv=128, dtype="bf16", scale=float(np.sqrt(128)), seed=83 + N,
                   chunk=128, rotate=True)
    print_case("gradients-dk128-length", N, w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=11)
    timer = R.Timer()
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 11, "bf16", options={"timer": timer})
    assert timer.query("ret_permute_rotate")[1] == (1 if N % 32 == 0 else 2)
    timer.close()
    _check(got, ref, tol("bf16"))


@pytest.mark.parametrize("case", [(2, 700, 4, 64, 9), (1, 1024, 2, 64, 70001)], ids=["ragged", "far-positions"])
def test_gradients_on_chip_rotate_while_staging(R, case):
    """d = 64 in short segments (the on-chip kernel's reversed traversal): no rotation launch and no rotated
    copies; the dq' and dk' runs turn their v rows (K, Q) while staging and their outputs back, the dv run rotates
    its q and k (K, Q) while staging over the reversed sequence, a ragged last chunk included."""
    B, N, H, d, pos0 = case
    w = W.Workload("grad", B=B, N=N, H=H, dk=d, dv=d, dtype="bf16", scale=float(np.sqrt(d)), seed=79 + N, chunk=64,
                   rotate=True)
    print_case("gradients-on-chip-rotation", pos0, w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=pos0)
    timer = R.Timer()
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, pos0, "f32", options={"timer": timer})
    assert timer.query("ret_rotate_qk")[1] == 0
    assert timer.query("ret_chunk_seg")[1] == 3
    timer.close()
    _check(got, ref, tol("bf16"))


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_gradients_rotated_by_their_kernel(R, out_dt):
    """d_k = d_v = 128 in two segments of 2048 tokens (32 chunks of 64 each, the rotation factors carried from chunk
    to chunk and evaluated exactly every 8) at positions past 70000: the streaming kernel rotates K and Q while
    staging them (as v of the dq' and dk' retentions, as q and k of the dv retention over the reversed sequence)
    and turns dq and dk back by the transpose rotation itself: no rotation or reordering launch."""
    w = W.Workload("grad", B=1, N=4096, H=2, dk=128, dv=128, dtype="bf16", scale=float(np.sqrt(128)), seed=73,
                   chunk=128, rotate=True)
    print_case("gradients-own-outputs", out_dt, w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=70001)
    timer = R.Timer()
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 70001, out_dt,
                    options={"timer": timer, "segments": 2})
    assert timer.query("ret_permute_rotate")[1] == 0
    assert timer.query("ret_rotate_qk")[1] == 0
    assert timer.query("ret_chunk_fused")[1] == 3
    # local passes and scans of dq' and dv only: dk' enters its segments with the dv retention's states, transposed
    assert timer.query("ret_chunk_fused_local")[1] == 2 and timer.query("ret_chunk_fused_scan")[1] == 2
    timer.close()
    _check(got, ref, tol("bf16"))


@pytest.mark.parametrize("direct", ["1", "0"])
@pytest.mark.parametrize("dk,dv,variant", [(256, 512, 0), (128, 128, 0), (128, 128, 3)])
def test_gradients_in_place_or_copied(R, direct, dk, dv, variant):
    """d_k 256, d_v 512 (the three-launch kernels) and d_k = d_v = 128 (the streaming kernel, or the wide-head
    kernel with variant 3) in place (bwd_direct 1) and through reordered copies (0)."""
    w = W.Workload("grad", B=1, N=768, H=2, dk=dk, dv=dv, dtype="bf16", scale=float(np.sqrt(dk)), seed=47,
                   chunk=128, rotate=True)
    print_case("gradients-path", direct, w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=1)
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 1, "f32",
                    options={"bwd_direct": int(direct), "variant": variant})
    _check(got, ref, tol("bf16"))


@pytest.mark.parametrize("direct", ["1", "0"])
def test_gradients_both_paths(R, direct):
    """The reversed-traversal path and the reordered-copies path (bwd_direct 0) on one shape."""
    w = W.Workload("grad", B=3, N=900, H=2, dk=64, dv=64, dtype="bf16", scale=8.0, seed=43, chunk=64, rotate=True)
    print_case("gradients-path", direct, w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=2)
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 2, "bf16", options={"bwd_direct": int(direct)})
    _check(got, ref, tol("bf16"))


F32_CASES = [
    # B, N, H, dk, dv, chunk, rotate, pos0
    (2, 150, 2, 32, 32, 32, True, 3),
    (1, 200, 2, 64, 128, 32, True, 7),   # d_v = 128: two halves of 64 (the fp32 kernels' widest d_k)
    (1, 300, 3, 64, 16, 64, True, 0),
    (2, 77, 2, 16, 64, 16, False, 0),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "B%d-N%d-H%d-dk%d-dv%d-C%d" % c[:6])
def test_gradients_f32(R, case):
    """fp32 inputs and gradients (the reordered-copies path on the fp32 kernels) at the fp32 bar of 1e-5."""
    B, N, H, dk, dv, chunk, rot, pos0 = case
    w = W.Workload("grad32", B=B, N=N, H=H, dk=dk, dv=dv, dtype="f32", scale=1.0, seed=51 + N, chunk=chunk,
                   rotate=rot)
    print_case("gradients-f32", w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=pos0)
    got = _gpu_grad(R, q, k, v, do, w.gamma, chunk, w.theta, pos0, "f32", in_dt="f32")
    _check(got, ref, tol("f32"))


def test_gradients_workspace_reused(R):
    """Two calls on one workspace (the chain part is left zeroed by each call) give the same gradients."""
    import torch
    w = W.Workload("grad", B=2, N=700, H=4, dk=64, dv=64, dtype="bf16", scale=8.0, seed=41, chunk=64, rotate=True)
    print_case("gradients-reuse", w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ws = R.chunkwise_bwd_workspace(to_dev(q, "bf16"), to_dev(v, "bf16"), w.chunk)
    first = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 0, "f32", workspace=ws)
    second = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 0, "f32", workspace=ws)
    R.ret_chunkwise_check(ws)  # no segment-chain wait gave up
    for a, b in zip(first, second):
        assert np.array_equal(a, b)
    _check(first, oracle.grad(q, k, v, do, w.gamma, theta=w.theta), tol("bf16"))
    torch.cuda.synchronize()


def test_gradients_workload2_full(R):
    """The retention-layer-d512 workload (B=8, N=2048, H=8, d=64, chunk 64, rotation) at full size."""
    w = W.WORKLOADS[2]
    print_case("gradients-workload2", w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta)
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 0, "f32")
    _check(got, ref, tol("bf16"))


def test_gradients_long_sequence_full(R):
    """The long-sequence workload (B=1, N=65536, H=8, d=128, chunk 128) at full size: the streaming kernels over
    the reversed sequence in place, many segments per head."""
    w = W.WORKLOADS[5]
    print_case("gradients-workload5", w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta)
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 0, "bf16")
    _check(got, ref, tol("bf16"))


def test_gradients_7b_class_layer_full(R):
    """The 7b-class-layer workload (B=1, N=8192, H=16, d_k=256, d_v=512, chunk 128) at full size: the paper's
    head shape, dq' and dk' as sums over the two halves of d_v, read in place; and the same gradients, bit for bit,
    from the forward call's saved rotated q, k and segment states."""
    import torch
    w = W.WORKLOADS[4]
    print_case("gradients-workload4", w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta)
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 0, "bf16")
    _check(got, ref, tol("bf16"))
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    fws = R.chunkwise_workspace(qd, vd, w.chunk)
    R.ret_chunkwise_fwd(qd, kd, vd, empty_out(v.shape, "bf16"), w.gamma, w.chunk, theta=w.theta, workspace=fws)
    dq, dk_, dv_ = empty_out(q.shape, "bf16"), empty_out(k.shape, "bf16"), empty_out(v.shape, "bf16")
    R.ret_chunkwise_bwd(qd, kd, vd, dod, dq, dk_, dv_, w.gamma, w.chunk, theta=w.theta, fwd_workspace=fws, check=True)
    torch.cuda.synchronize()
    for a, b in zip(got, (to_host(dq), to_host(dk_), to_host(dv_))):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("case", [
    # B, N, H, dk, dv, chunk, rotate, pos0, forward options: the forward's rotated q, k and segment states reused
    (1, 640, 2, 256, 512, 128, True, 5, None),
    (2, 512, 2, 256, 256, 64, False, 0, None),
    # nothing to reuse: a forward with another segment plan, or another kernel family
    (1, 640, 2, 256, 512, 128, True, 5, {"segments": 2}),
    (1, 300, 2, 64, 64, 64, True, 3, None),
    # the streaming kernel's split launches (d_k = d_v = 128): dq' enters its segments with the forward's states
    (1, 2048, 2, 128, 128, 128, True, 7, None),
], ids=["dk256-dv512", "dk256-dv256-norot", "other-plan", "dk64", "dk128"])
def test_gradients_after_forward(R, case):
    """ret_chunkwise_bwd_saved_ex with the forward call's workspace gives the same gradients as the gradients
    computed on their own, and skips the rotation and the (K', V) states where it reuses them: bit for bit where
    the forward ran the same kernels on the same values (d_k 256), to rounding where dq' enters its segments with
    the forward's states (d_k 128: those sums are formed in another order of products and roundings)."""
    import torch
    B, N, H, dk, dv, chunk, rot, pos0, fopts = case
    w = W.Workload("grad", B=B, N=N, H=H, dk=dk, dv=dv, dtype="bf16", scale=float(np.sqrt(dk)), seed=71 + N,
                   chunk=chunk, rotate=rot)
    print_case("gradients-after-forward", fopts, w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    o = empty_out(v.shape, "bf16")
    fws = R.chunkwise_workspace(qd, vd, chunk, fopts)
    R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, chunk, theta=w.theta, pos0=pos0, workspace=fws, options=fopts)
    grads = []
    for saved in (False, True):
        dq, dk_, dv_ = empty_out(q.shape, "f32"), empty_out(k.shape, "f32"), empty_out(v.shape, "f32")
        timer = R.Timer()
        R.ret_chunkwise_bwd(qd, kd, vd, dod, dq, dk_, dv_, w.gamma, chunk, theta=w.theta, pos0=pos0,
                            options={"timer": timer}, fwd_workspace=fws if saved else None, check=True)
        torch.cuda.synchronize()
        grads.append((to_host(dq), to_host(dk_), to_host(dv_)))
        if saved and fopts is None and dk == 256:
            assert timer.query("ret_rotate_qk")[1] == 0
            assert timer.query("ret_chunk_dma_local")[1] == 1 and timer.query("ret_chunk_dma_scan")[1] == 1
        if dk == 128:  # local passes and scan of the dv retention only (and of dq' on its own)
            assert timer.query("ret_chunk_fused_local")[1] == (1 if saved else 2)
            assert timer.query("ret_chunk_fused_scan")[1] == (1 if saved else 2)
        timer.close()
    for a, b in zip(*grads):
        if dk == 128:
            assert rel_err(a, b) <= 1e-3, rel_err(a, b)
        else:
            assert np.array_equal(a, b)
    _check(grads[1], oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=pos0), tol("bf16"))
