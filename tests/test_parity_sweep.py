"""GPU parity over seeded random shapes: the chunkwise forward, its gradients and the decode step against the fp64
oracle, with shapes, chunk sizes, positions, initial states and plan options drawn per case. Every bf16 kernel
family is reached this way: the on-chip d_k <= 64 kernel and the streaming one, the d_k = 128 and 256 kernels
(chained, three launches, wide and LDS-loading variants, with and without rotated copies), segment counts from 1
to 9, ragged sequences, positions past 2^20, and the gradients on the reversed traversal or reordered copies,
with and without the forward call's workspace.

Bar (max|gpu - oracle| / max|oracle|): 2e-2 for bf16 inputs. The gradients of bf16 heads with d_k = 32 have no
kernels (their dq and dk retentions would need d_v = 32); such cases must report an unsupported shape.
"""
import numpy as np
import pytest

import oracle
from linear_recurrent_sequence_amd import workloads as W
from tests.conftest import print_case
from tests.helpers import empty_out, rel_err, to_dev, to_host, tol

pytestmark = pytest.mark.gpu

DV_OF = {32: [64, 128], 64: [64, 128, 256], 128: [128, 256], 256: [128, 256, 512]}


@pytest.fixture(scope="module")
def R():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from linear_recurrent_sequence_amd import retention
    retention.load(build_if_missing=True)
    return retention


def _draw(rng):
    """One case: shape, chunk, rotation and position, initial state, plan options."""
    dk = int(rng.choice([32, 64, 128, 256]))
    dv = int(rng.choice(DV_OF[dk]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    N = int(rng.integers(1, 900)) if rng.random() < 0.7 else int(rng.choice([32, 64, 96, 128, 256, 512, 640]))
    C = int(rng.choice([32, 64, 128, 256]))
    rot = bool(rng.random() < 0.8)
    pos0 = int(rng.choice([0, 3, 1000, 65536, 2 ** 20 + 7]))
    has_s = bool(rng.random() < 0.4)
    opts = {}
    if rng.random() < 0.5:
        opts["segments"] = int(rng.integers(1, 10))
    if dk == 256 and rng.random() < 0.3:
        opts["variant"] = int(rng.choice([3, 5]))
    if dk <= 64 and rng.random() < 0.3:
        opts["onchip"] = 0
    if rng.random() < 0.2:
        opts["prerotate"] = int(rng.integers(0, 2))
    return B, N, H, dk, dv, C, rot, pos0, has_s, opts


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_forward_and_gradients(R, seed):
    import torch
    rng = np.random.default_rng(9100 + seed)
    for case in range(16):
        B, N, H, dk, dv, C, rot, pos0, has_s, opts = _draw(rng)
        print_case("sweep", seed, case, (B, N, H, dk, dv, C, rot, pos0, has_s, opts))
        q = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
        k = W.normal(rng, (B, N, H, dk), 8.0, "bf16")
        v = W.normal(rng, (B, N, H, dv), 8.0, "bf16")
        s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) if has_s else None
        gamma, theta = W.gamma_schedule(H), (W.theta_schedule(dk) if rot else None)
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        o = empty_out((B, N, H, dv), "bf16")
        sin = torch.from_numpy(s0).cuda() if has_s else None
        sout = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
        ws = R.chunkwise_workspace(qd, vd, C, opts)
        R.ret_chunkwise_fwd(qd, kd, vd, o, gamma, C, theta=theta, pos0=pos0, state_in=sin, state_out=sout,
                            workspace=ws, options=opts)
        torch.cuda.synchronize()
        R.ret_chunkwise_check(ws)
        o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=pos0, state_in=s0)
        eo, es = rel_err(to_host(o), o_ref), rel_err(to_host(sout), s_ref)
        print("  err o=%.3g state=%.3g" % (eo, es))
        assert eo <= tol("bf16") and es <= tol("bf16"), (eo, es)

        if rng.random() >= 0.6:
            continue
        gopts = dict(opts)
        if rng.random() < 0.3:
            gopts["bwd_direct"] = int(rng.integers(0, 2))
        odt = str(rng.choice(["bf16", "f32"]))
        reuse = (not has_s) and gopts == opts and rng.random() < 0.5
        do = W.normal(rng, (B, N, H, dv), 8.0, "bf16")
        print_case("sweep grad", odt, gopts, "after the forward" if reuse else "")
        dq, dkg, dvg = empty_out(q.shape, odt), empty_out(k.shape, odt), empty_out(v.shape, odt)
        if dk == 32:
            with pytest.raises(ValueError, match="unsupported"):
                R.ret_chunkwise_bwd(qd, kd, vd, to_dev(do, "bf16"), dq, dkg, dvg, gamma, C, theta=theta, pos0=pos0,
                                    options=gopts, check=True)
            continue
        R.ret_chunkwise_bwd(qd, kd, vd, to_dev(do, "bf16"), dq, dkg, dvg, gamma, C, theta=theta, pos0=pos0,
                            options=gopts, check=True, fwd_workspace=ws if reuse else None)
        torch.cuda.synchronize()
        ref = oracle.grad(q, k, v, do, gamma, theta=theta, pos0=pos0)
        errs = [rel_err(to_host(g), r) for g, r in zip((dq, dkg, dvg), ref)]
        print("  err dq=%.3g dk=%.3g dv=%.3g" % tuple(errs))
        assert max(errs) <= tol("bf16"), errs


@pytest.mark.parametrize("seed", range(4))
def test_random_shapes_fp32(R, seed):
    """fp32 inputs (d_k in {16, 32, 64}, chunks of 16 to 64): the chunkwise and parallel forms and the gradients
    over seeded random shapes, positions and initial states, at the fp32 bar."""
    import torch
    rng = np.random.default_rng(9300 + seed)
    for case in range(12):
        dk = int(rng.choice([16, 32, 64]))
        dv = int(rng.choice([16, 32, 48, 64, 80, 128]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 400))
        C = int(rng.choice([16, 32, 64]))
        rot = bool(rng.random() < 0.7)
        pos0 = int(rng.choice([0, 5, 4096, 2 ** 20 + 3]))
        has_s = bool(rng.random() < 0.5)
        opts = {"segments": int(rng.integers(1, 6))} if rng.random() < 0.5 else {}
        print_case("sweep fp32", seed, case, (B, N, H, dk, dv, C, rot, pos0, has_s, opts))
        q = rng.standard_normal((B, N, H, dk)).astype(np.float32)
        k = rng.standard_normal((B, N, H, dk)).astype(np.float32)
        v = rng.standard_normal((B, N, H, dv)).astype(np.float32)
        s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) if has_s else None
        gamma, theta = W.gamma_schedule(H), (W.theta_schedule(dk) if rot else None)
        qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
        o = empty_out((B, N, H, dv), "f32")
        sin = torch.from_numpy(s0).cuda() if has_s else None
        sout = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
        ws = R.chunkwise_workspace(qd, vd, C, opts)
        R.ret_chunkwise_fwd(qd, kd, vd, o, gamma, C, theta=theta, pos0=pos0, state_in=sin, state_out=sout,
                            workspace=ws, options=opts)
        op = empty_out((B, N, H, dv), "f32")
        R.ret_parallel_fwd(qd, kd, vd, op, gamma, theta=theta, pos0=pos0)
        torch.cuda.synchronize()
        R.ret_chunkwise_check(ws)
        o_ref, s_ref = oracle.chunkwise(q, k, v, gamma, C, theta=theta, pos0=pos0, state_in=s0)
        p_ref = oracle.parallel(q, k, v, gamma, theta=theta, pos0=pos0)
        errs = rel_err(to_host(o), o_ref), rel_err(to_host(sout), s_ref), rel_err(to_host(op), p_ref)
        print("  err o=%.3g state=%.3g parallel=%.3g" % errs)
        assert max(errs) <= tol("f32"), errs
        if dv in (48, 80):  # the gradients' dq and dk retentions take d_v as their d_k: 16, 32, 64 or twice 64
            continue
        do = rng.standard_normal((B, N, H, dv)).astype(np.float32)
        dq, dkg, dvg = empty_out(q.shape, "f32"), empty_out(k.shape, "f32"), empty_out(v.shape, "f32")
        R.ret_chunkwise_bwd(qd, kd, vd, to_dev(do, "f32"), dq, dkg, dvg, gamma, C, theta=theta, pos0=pos0,
                            options=opts, check=True)
        torch.cuda.synchronize()
        ref = oracle.grad(q, k, v, do, gamma, theta=theta, pos0=pos0)
        gerrs = [rel_err(to_host(g), r) for g, r in zip((dq, dkg, dvg), ref)]
        print("  err dq=%.3g dk=%.3g dv=%.3g" % tuple(gerrs))
        assert max(gerrs) <= tol("f32"), gerrs


@pytest.mark.parametrize("seed", range(4))
def test_random_shapes_decode(R, seed):
    """Decode steps over seeded random shapes (bf16 d_k 32 to 256, fp32 d_k 16 to 64; batch and heads from 1 up to
    40 and 8), positions and states: three consecutive steps, each output and state against the oracle's step."""
    import torch
    rng = np.random.default_rng(9500 + seed)
    for case in range(10):
        bf = bool(rng.random() < 0.6)
        dk = int(rng.choice([32, 64, 128, 256] if bf else [16, 32, 64]))
        dv = int(rng.choice([64, 128, 256] if bf else [16, 32, 64, 128]))
        B, H = int(rng.integers(1, 41)), int(rng.integers(1, 9))
        rot = bool(rng.random() < 0.8)
        pos = int(rng.choice([0, 7, 70000, 2 ** 20 + 1]))
        dt = "bf16" if bf else "f32"
        print_case("sweep decode", seed, case, (dt, B, H, dk, dv, rot, pos))
        gamma, theta = W.gamma_schedule(H), (W.theta_schedule(dk) if rot else None)
        s_ref = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
        state = torch.from_numpy(s_ref.copy()).cuda()
        for t in range(3):
            scale = 8.0 if bf else 1.0
            q = W.normal(rng, (B, H, dk), scale, dt)
            k = W.normal(rng, (B, H, dk), scale, dt)
            v = W.normal(rng, (B, H, dv), scale, dt)
            o = empty_out((B, H, dv), dt)
            R.ret_recurrent_step(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), o, state, gamma, pos + t, theta=theta)
            torch.cuda.synchronize()
            o_ref, s_ref = oracle.recurrent_step(q, k, v, gamma, s_ref, pos + t, theta=theta)
            eo, es = rel_err(to_host(o), o_ref), rel_err(to_host(state), s_ref)
            print("  step %d err o=%.3g state=%.3g" % (t, eo, es))
            assert eo <= tol(dt) and es <= tol(dt), (t, eo, es)
