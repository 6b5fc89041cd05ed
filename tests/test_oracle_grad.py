"""Pins for the oracle's gradients of retention (no GPU).

The oracle computes dq, dk, dv of L = sum(dO (.) O) by the adjoint of the recurrent scan. The pins rest on what
fixes a gradient independently of that algorithm: central finite differences of the oracle's parallel form
(the definition, with rotation and per-head decay), Euler's identity for a function linear in each argument
(<dq, q> = <dk, k> = <dv, v> = L), and, for gamma = 1 without rotation, the textbook gradient of causal linear
attention written with numpy matrix products.
"""
import numpy as np
import pytest

import oracle


def _inputs(rng, B=1, N=9, H=2, dk=6, dv=4):
    q = rng.standard_normal((B, N, H, dk))
    k = rng.standard_normal((B, N, H, dk))
    v = rng.standard_normal((B, N, H, dv))
    do = rng.standard_normal((B, N, H, dv))
    return q, k, v, do


@pytest.mark.parametrize("rotate,pos0", [(True, 5), (False, 0), (True, 1000)])
def test_gradients_match_finite_differences(rotate, pos0):
    rng = np.random.default_rng(21)
    q, k, v, do = _inputs(rng)
    gamma = np.array([0.8, 0.97])
    theta = np.array([0.3, 1.1, 0.05]) if rotate else None
    loss = lambda q, k, v: float((oracle.parallel(q, k, v, gamma, theta=theta, pos0=pos0) * do).sum())
    dq, dk, dv = oracle.grad(q, k, v, do, gamma, theta=theta, pos0=pos0)
    eps = 1e-6
    for name, an, x in (("q", dq, q), ("k", dk, k), ("v", dv, v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(**args)
            args[name] = xm
            fd[idx] = (lp - loss(**args)) / (2 * eps)
        assert np.abs(an - fd).max() <= 1e-7 * max(1.0, np.abs(fd).max()), name


def test_euler_identities():
    """O is linear in q, in k and in v, so each gradient dotted with its argument gives L."""
    rng = np.random.default_rng(22)
    q, k, v, do = _inputs(rng, B=2, N=50, H=3, dk=8, dv=6)
    gamma = np.array([0.9, 0.99, 1.0])
    theta = 10000.0 ** (-np.arange(4) / 4.0)
    L = float((oracle.parallel(q, k, v, gamma, theta=theta, pos0=7) * do).sum())
    dq, dk, dv = oracle.grad(q, k, v, do, gamma, theta=theta, pos0=7)
    for g, x in ((dq, q), (dk, k), (dv, v)):
        assert abs(float((g * x).sum()) - L) <= 1e-10 * max(1.0, abs(L))


def test_gamma_one_is_causal_linear_attention_gradient():
    """gamma = 1, no rotation: O = tril(Q K^T) V per head, so dV = A^T dO, dQ = tril(dO V^T) K and
    dK = tril(dO V^T)^T Q."""
    rng = np.random.default_rng(23)
    q, k, v, do = _inputs(rng, B=1, N=12, H=1, dk=5, dv=3)
    dq, dk, dv = oracle.grad(q, k, v, do, np.array([1.0]))
    Q, K, V, dO = q[0, :, 0], k[0, :, 0], v[0, :, 0], do[0, :, 0]
    A = np.tril(Q @ K.T)
    M = np.tril(dO @ V.T)
    assert np.abs(dv[0, :, 0] - A.T @ dO).max() <= 1e-12
    assert np.abs(dq[0, :, 0] - M @ K).max() <= 1e-12
    assert np.abs(dk[0, :, 0] - M.T @ Q).max() <= 1e-12
