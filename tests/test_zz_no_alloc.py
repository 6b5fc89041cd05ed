"""The no-allocation chunkwise entry point (its workspace is the library's own device array) against
ret_chunkwise_fwd with a caller-allocated workspace, called through the C ABI: two calls in a row, the second
with a smaller input, each matching the existing entry point's output and state to the bf16 bar (2e-2) and the
oracle; run alone in a fresh process and after the other tests."""
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


# (B, N, H, dk, dv, chunk): a chained on-chip call, then a smaller one; a d_k 128 chained call, then a smaller;
# the d_k 256 / d_v 512 head (rotated copies beside the chain), then a smaller one.
SEQUENCES = [
    [(2, 1500, 2, 64, 64, 64), (1, 700, 2, 64, 64, 64)],
    [(1, 2000, 2, 128, 128, 128), (1, 900, 1, 128, 128, 128)],
    [(1, 1100, 2, 256, 512, 128), (1, 300, 2, 256, 512, 128)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "dk%d" % s[0][3])
def test_noalloc_matches_the_allocating_call(R, seq):
    import torch
    for i, (B, N, H, dk, dv, C) in enumerate(seq):
        print_case("noalloc call %d" % i, (B, N, H, dk, dv, C))
        rng = np.random.default_rng(1000 + 10 * i + dk)
        q = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
        k = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
        v = W.normal(rng, (B, N, H, dv), 8.0, "bf16")
        s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
        gamma, theta = W.gamma_schedule(H), W.theta_schedule(dk)
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        sin = torch.from_numpy(s0).cuda()
        o_ref_dev = empty_out((B, N, H, dv), "bf16")
        s_ref_dev = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
        ws = R.chunkwise_workspace(qd, vd, C)
        R.ret_chunkwise_fwd(qd, kd, vd, o_ref_dev, gamma, C, theta=theta, pos0=3, state_in=sin, state_out=s_ref_dev,
                            workspace=ws)
        o = empty_out((B, N, H, dv), "bf16")
        sout = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
        R.ret_chunkwise_fwd_noalloc(qd, kd, vd, o, gamma, C, theta=theta, pos0=3, state_in=sin, state_out=sout)
        torch.cuda.synchronize()
        o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=3, state_in=s0)
        e_o, e_s = rel_err(to_host(o), to_host(o_ref_dev)), rel_err(to_host(sout), to_host(s_ref_dev))
        e_or, e_sr = rel_err(to_host(o), o_ref), rel_err(to_host(sout), s_ref)
        print("  vs allocating call: o=%.3g state=%.3g; vs oracle: o=%.3g state=%.3g" % (e_o, e_s, e_or, e_sr))
        assert e_o <= tol("bf16") and e_s <= tol("bf16"), (e_o, e_s)
        assert e_or <= tol("bf16") and e_sr <= tol("bf16"), (e_or, e_sr)
