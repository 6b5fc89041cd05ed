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


def _gpu_grad(R, q, k, v, do, gamma, chunk, theta, pos0, out_dt, workspace=None, in_dt="bf16"):
    import torch
    qd, kd, vd, dod = (to_dev(x, in_dt) for x in (q, k, v, do))
    dq, dk, dv = empty_out(q.shape, out_dt), empty_out(k.shape, out_dt), empty_out(v.shape, out_dt)
    R.ret_chunkwise_bwd(qd, kd, vd, dod, dq, dk, dv, gamma, chunk, theta=theta, pos0=pos0, workspace=workspace)
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


@pytest.mark.parametrize("direct", ["1", "0"])
def test_gradients_both_paths(R, direct, monkeypatch):
    """The reversed-traversal path and the reordered-copies path (RET_BWD_DIRECT=0) on one shape."""
    monkeypatch.setenv("RET_BWD_DIRECT", direct)
    w = W.Workload("grad", B=3, N=900, H=2, dk=64, dv=64, dtype="bf16", scale=8.0, seed=43, chunk=64, rotate=True)
    print_case("gradients-path", direct, w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta, pos0=2)
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 2, "bf16")
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
    """The long-sequence workload (B=1, N=65536, H=8, d=128, chunk 128) at full size: the streaming kernels on
    reordered copies, 64 segments per head."""
    w = W.WORKLOADS[5]
    print_case("gradients-workload5", w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta)
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 0, "bf16")
    _check(got, ref, tol("bf16"))


def test_gradients_7b_class_layer_full(R):
    """The 7b-class-layer workload (B=1, N=8192, H=16, d_k=256, d_v=512, chunk 128) at full size: the paper's
    head shape, dq' and dk' as sums over the two halves of d_v."""
    w = W.WORKLOADS[4]
    print_case("gradients-workload4", w)
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    ref = oracle.grad(q, k, v, do, w.gamma, theta=w.theta)
    got = _gpu_grad(R, q, k, v, do, w.gamma, w.chunk, w.theta, 0, "bf16")
    _check(got, ref, tol("bf16"))
