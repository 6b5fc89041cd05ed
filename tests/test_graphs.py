"""HIP graph capture: the chunkwise forward, the fused layer and the gradients captured once and replayed with
new inputs copied in between (eager work and synchronizations between replays), every replay checked against
the fp64 oracle. The library records no memset or host synchronization into a stream, so its calls capture as
plain kernel nodes; the segment chain leaves its workspace ready for the next replay."""
import numpy as np
import pytest

import oracle
from linear_recurrent_sequence_amd import workloads as W
from tests.conftest import print_case
from tests.helpers import rel_err, to_host, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from linear_recurrent_sequence_amd import retention
    retention.load(build_if_missing=True)
    return retention


def _capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _inputs(rng, B, N, H, dk, dv):
    return (W.normal(rng, (B, N, H, dk), 8.0, "bf16"), W.normal(rng, (B, N, H, dk), 8.0, "bf16"),
            W.normal(rng, (B, N, H, dv), 8.0, "bf16"), W.normal(rng, (B, N, H, dv), 8.0, "bf16"))


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 256)])
def test_chunkwise_forward_replays(R, dk, dv):
    import torch
    B, N, H, C = 2, 1000, 4, 64
    print_case("graph_chunkwise", B, N, H, dk, dv)
    rng = np.random.default_rng(61)
    gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
    qd = torch.empty((B, N, H, dk), dtype=torch.bfloat16, device="cuda")
    kd, vd = torch.empty_like(qd), torch.empty((B, N, H, dv), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(vd)
    state = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = R.chunkwise_workspace(qd, vd, C)
    g = _capture(torch, lambda: R.ret_chunkwise_fwd(qd, kd, vd, o, gamma, C, theta=theta, state_out=state,
                                                     workspace=ws))
    for rep in range(3):
        q, k, v, _ = _inputs(rng, B, N, H, dk, dv)
        for dst, src in ((qd, q), (kd, k), (vd, v)):
            dst.copy_(torch.from_numpy(src).to(torch.bfloat16))
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        R.ret_chunkwise_check(ws)
        o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta)
        eo, es = rel_err(to_host(o), o_ref), rel_err(to_host(state), s_ref)
        print("  replay %d: err o=%.3g state=%.3g" % (rep, eo, es))
        assert eo <= tol("bf16") and es <= tol("bf16"), (rep, eo, es)


def test_fused_layer_and_gradients_replay(R):
    """ret_chunkwise_msr_fwd and ret_chunkwise_bwd (reversed traversal) in one graph."""
    import torch
    B, N, H, dk, dv, C = 2, 900, 4, 64, 64, 64
    print_case("graph_layer_grad", B, N, H)
    rng = np.random.default_rng(62)
    gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
    qd = torch.empty((B, N, H, dk), dtype=torch.bfloat16, device="cuda")
    kd, vd, dod, gate = (torch.empty_like(qd) for _ in range(4))
    y, dq, dk_, dv_ = (torch.empty_like(qd) for _ in range(4))
    ws = R.chunkwise_workspace(qd, vd, C)
    wsb = R.chunkwise_bwd_workspace(qd, vd, C)

    def calls():
        R.ret_chunkwise_msr_fwd(qd, kd, vd, y, gamma, C, gate=gate, eps=1e-5, theta=theta, workspace=ws)
        R.ret_chunkwise_bwd(qd, kd, vd, dod, dq, dk_, dv_, gamma, C, theta=theta, workspace=wsb)

    g = _capture(torch, calls)
    for rep in range(2):
        q, k, v, do = _inputs(rng, B, N, H, dk, dv)
        gt = W.normal(rng, (B, N, H, dv), 1.0, "bf16")
        for dst, src in ((qd, q), (kd, k), (vd, v), (dod, do), (gate, gt)):
            dst.copy_(torch.from_numpy(src).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        R.ret_chunkwise_check(ws)
        R.ret_chunkwise_check(wsb)
        o_ref, _ = oracle.chunkwise(q, k, v, gamma, C, theta=theta)
        y_ref = oracle.msr_epilogue(o_ref, gate=gt, eps=1e-5)
        ey = rel_err(to_host(y), y_ref)
        ref = oracle.grad(q, k, v, do, gamma, theta=theta)
        errs = [rel_err(to_host(t), r) for t, r in zip((dq, dk_, dv_), ref)]
        print("  replay %d: err y=%.3g dq=%.3g dk=%.3g dv=%.3g" % (rep, ey, *errs))
        assert ey <= tol("bf16") and max(errs) <= tol("bf16"), (rep, ey, errs)
