"""Pins for the oracle's multi-scale retention epilogue and score normalizations (no GPU).

Sources: "Hybrid Architectures: RetNet and the Three Computation Paradigms", sections 8.4 (GroupNorm with one
group per head), 8.5 (retention score normalization) and 9.1 (the swish gate); the paper summary, "Gating
mechanism" and "Retention Score Normalization". The checks rest on what fixes the result independently of
the oracle's code: library routines of the same definitions (torch's group_norm and silu, in float64),
closed forms, and the pages' statement that GroupNorm cancels any per-head scale.
"""
import numpy as np
import pytest

import oracle


def _torch():
    torch = pytest.importorskip("torch")
    return torch


@pytest.mark.parametrize("H,dv,eps", [(1, 4, 1e-5), (3, 16, 1e-5), (4, 64, 0.1), (2, 8, 0.0)])
def test_groupnorm_matches_library_routine(H, dv, eps):
    """GroupNorm_h with per-channel weight and bias equals torch's group_norm with H groups, per token."""
    torch = _torch()
    rng = np.random.default_rng(101)
    o = rng.standard_normal((3, 7, H, dv)) * rng.uniform(0.1, 10.0, size=(1, 1, H, 1))
    w = rng.standard_normal(H * dv)
    b = rng.standard_normal(H * dv)
    y = oracle.msr_epilogue(o, weight=w, bias=b, eps=eps)
    ref = torch.nn.functional.group_norm(torch.from_numpy(o.reshape(-1, H * dv)), H, torch.from_numpy(w),
                                         torch.from_numpy(b), eps=eps).numpy().reshape(o.shape)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_swish_gate_matches_library_routine_and_its_symmetry():
    """With constant head rows GroupNorm gives 0 exactly, so a bias of 1 leaves y = swish(g): it equals torch's
    silu, vanishes at 0, tends to x and to 0 at the two ends, and satisfies swish(-x) = swish(x) - x."""
    torch = _torch()
    H, dv = 2, 8
    g = np.concatenate([np.linspace(-6, 6, 15), [0.0, 40.0, -40.0]])
    g = np.resize(g, (5, H, dv))
    o = np.ones_like(g) * 3.5
    y = oracle.msr_epilogue(o, gate=g, bias=np.ones(H * dv), eps=1e-5)
    assert np.abs(y - torch.nn.functional.silu(torch.from_numpy(g)).numpy()).max() <= 1e-15
    y0 = oracle.msr_epilogue(np.ones((1, 1, 3)), gate=np.array([[[0.0, 40.0, -40.0]]]), bias=np.ones(3))
    assert y0[0, 0, 0] == 0.0 and abs(y0[0, 0, 1] - 40.0) < 1e-12 and abs(y0[0, 0, 2]) < 1e-15
    x = np.linspace(-5, 5, 11).reshape(1, 1, 11)
    yp = oracle.msr_epilogue(np.ones_like(x), gate=x, bias=np.ones(11))
    yn = oracle.msr_epilogue(np.ones_like(x), gate=-x, bias=np.ones(11))
    assert np.abs(yn - (yp - x)).max() <= 1e-14


def test_groupnorm_standardizes_each_head_separately():
    """Each (token, head) row comes out with mean 0 and variance var / (var + eps), whatever the other heads'
    scales (a norm over all heads together would mix them)."""
    rng = np.random.default_rng(5)
    H, dv, eps = 3, 32, 1e-3
    o = rng.standard_normal((4, 6, H, dv)) * np.array([0.01, 1.0, 100.0]).reshape(1, 1, H, 1) + 7.0
    y = oracle.msr_epilogue(o, eps=eps)
    var = o.var(axis=-1)
    assert np.abs(y.mean(axis=-1)).max() <= 1e-12
    assert np.abs(y.var(axis=-1) - var / (var + eps)).max() <= 1e-12


@pytest.mark.parametrize("alpha", [1e-3, 3.0, 1e4])
def test_groupnorm_scale_invariance(alpha):
    """GroupNorm(alpha * head) = GroupNorm(head) for alpha > 0 (exact with eps = 0)."""
    rng = np.random.default_rng(9)
    o = rng.standard_normal((2, 5, 4, 16))
    g = rng.standard_normal(o.shape)
    a = oracle.msr_epilogue(o, gate=g, eps=0.0)
    b = oracle.msr_epilogue(alpha * o, gate=g, eps=0.0)
    assert np.abs(a - b).max() <= 1e-12


def _qkv(rng, N=24, H=2, dk=8, dv=4):
    q = rng.standard_normal((2, N, H, dk))
    k = rng.standard_normal((2, N, H, dk))
    v = rng.standard_normal((2, N, H, dv))
    return q, k, v


def test_no_normalization_is_the_parallel_form():
    rng = np.random.default_rng(11)
    q, k, v = _qkv(rng)
    gamma = np.array([0.9, 0.99])
    theta = 10000.0 ** (-np.arange(4) / 4.0)
    assert np.array_equal(oracle.parallel_normalized(q, k, v, gamma, theta=theta, pos0=3),
                          oracle.parallel(q, k, v, gamma, theta=theta, pos0=3))


def test_scale_divides_scores_by_sqrt_dk():
    """Scaling QK^T by 1/sqrt(d_k) is the parallel form with q scaled (the form is linear in q)."""
    rng = np.random.default_rng(12)
    q, k, v = _qkv(rng)
    gamma = np.array([0.8, 1.0])
    a = oracle.parallel_normalized(q, k, v, gamma, scale=True)
    b = oracle.parallel(q / np.sqrt(q.shape[-1]), k, v, gamma)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


@pytest.mark.parametrize("gamma", [1.0, 0.9, 0.5])
def test_decay_normalization_closed_form(gamma):
    """Row n of D sums to the geometric series (1 - gamma^(n+1)) / (1 - gamma) (n + 1 at gamma = 1); D~ divides
    row n of the output by its square root."""
    rng = np.random.default_rng(13)
    q, k, v = _qkv(rng)
    g = np.array([gamma, gamma])
    a = oracle.parallel_normalized(q, k, v, g, decay=True)
    b = oracle.parallel(q, k, v, g)
    n = np.arange(q.shape[1])
    s = n + 1.0 if gamma == 1.0 else (1.0 - gamma ** (n + 1)) / (1.0 - gamma)
    assert np.abs(a - b / np.sqrt(s).reshape(1, -1, 1, 1)).max() <= 1e-12 * max(1.0, np.abs(b).max())


def test_score_normalization_divides_rows_by_clamped_row_sum():
    """R~ divides row n by max(|sum_m R[n][m]|, 1); the row sums are the parallel form over values of ones."""
    rng = np.random.default_rng(14)
    q, k, v = _qkv(rng)
    q *= np.linspace(0.05, 2.0, q.shape[1]).reshape(1, -1, 1, 1)  # rows with |sum| both below and above 1
    gamma = np.array([0.7, 0.97])
    a = oracle.parallel_normalized(q, k, v, gamma, scores=True)
    b = oracle.parallel(q, k, v, gamma)
    rs = oracle.parallel(q, k, np.ones(v.shape[:3] + (1,)), gamma)  # [B, N, H, 1]
    den = np.maximum(np.abs(rs), 1.0)
    assert (np.abs(rs) < 1.0).any() and (np.abs(rs) > 1.0).any()
    assert np.abs(a - b / den).max() <= 1e-12 * max(1.0, np.abs(b).max())


def test_normalizations_cancel_under_groupnorm():
    """The three normalizations are scalars per (token, head), so GroupNorm (eps = 0) gives the same output
    with and without them, as the pages state."""
    rng = np.random.default_rng(15)
    q, k, v = _qkv(rng, N=30, dv=8)
    gamma = np.array([0.9, 0.999])
    theta = 10000.0 ** (-np.arange(4) / 4.0)
    gate = rng.standard_normal(v.shape)
    plain = oracle.msr_epilogue(oracle.parallel(q, k, v, gamma, theta=theta), gate=gate, eps=0.0)
    normed = oracle.msr_epilogue(
        oracle.parallel_normalized(q, k, v, gamma, theta=theta, scale=True, decay=True, scores=True), gate=gate,
        eps=0.0)
    assert np.abs(plain - normed).max() <= 1e-10
