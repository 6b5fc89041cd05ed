"""Pins of the fp64 oracle against values and facts the pages fix (no GPU).

Sources: "Hybrid Architectures: RetNet and the Three Computation Paradigms" (the worked example of
sections 3, 4 and 7, the linear-attention trace of section 1.1, the rotation table of section 6.9 and the
gamma table of section 8.2), and the RetNet paper summary (unrolled equation with the conjugate transpose).
Values are read from tests/golden/worked_example.json, which cites each one.
"""
import math

import numpy as np
import pytest

import oracle
from linear_recurrent_sequence_amd import workloads

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _example(golden):
    ex = golden["running_example"]
    q = np.array(ex["Q"], float)[None, :, None, :]   # [B=1, N=4, H=1, d=2]
    k = np.array(ex["K"], float)[None, :, None, :]
    v = np.array(ex["V"], float)[None, :, None, :]
    return q, k, v, np.array([ex["gamma"]])


def test_recurrent_trace_matches_worked_example(golden):
    q, k, v, g = _example(golden)
    tr = golden["recurrent_trace"]
    o, _ = oracle.recurrent(q, k, v, g)
    np.testing.assert_allclose(o[0, :, 0, :], np.array(tr["o"]), atol=1e-12)
    for n in range(1, 5):
        _, s = oracle.recurrent(q[:, :n], k[:, :n], v[:, :n], g)
        np.testing.assert_allclose(s[0, 0], np.array(tr["S"][n - 1]), atol=1e-12)


def test_state_norms(golden):
    q, k, v, g = _example(golden)
    want = golden["state_norms"]
    for n in range(1, 5):
        _, s = oracle.recurrent(q[:, :n], k[:, :n], v[:, :n], g)
        assert abs(np.linalg.norm(s[0, 0]) - want["frobenius"][n - 1]) <= want["tolerance"]


def test_parallel_output_matches_worked_example(golden):
    q, k, v, g = _example(golden)
    o = oracle.parallel(q, k, v, g)
    np.testing.assert_allclose(o[0, :, 0, :], np.array(golden["parallel_form"]["output"]), atol=1e-12)


def test_parallel_intermediates_via_one_hot_values(golden):
    """With v_m = e_m (d_v = n), row n of the output is row n of the masked score matrix."""
    q, k, _, g = _example(golden)
    pf = golden["parallel_form"]
    eye = np.eye(4)[None, :, None, :]
    # masked scores QK^T (.) D
    o = oracle.parallel(q, k, eye, g)
    np.testing.assert_allclose(o[0, :, 0, :], np.array(pf["QKt_masked"]), atol=1e-12)
    # D itself: every score q_n . k_m = 1
    ones = np.zeros((1, 4, 1, 2))
    ones[..., 0] = 1.0
    o = oracle.parallel(ones, ones, eye, g)
    np.testing.assert_allclose(o[0, :, 0, :], np.array(pf["D"]), atol=1e-12)
    # QK^T on and below the diagonal: gamma = 1 turns the mask into the plain causal mask
    o = oracle.parallel(q, k, eye, np.array([1.0]))
    np.testing.assert_allclose(o[0, :, 0, :], np.tril(np.array(pf["QKt"])), atol=1e-12)


def test_chunkwise_B2_matches_worked_example(golden):
    q, k, v, g = _example(golden)
    cw = golden["chunkwise_B2"]
    C = cw["chunk"]
    o, r2 = oracle.chunkwise(q, k, v, g, C)
    np.testing.assert_allclose(o[0, :2, 0], np.array(cw["inner_1"]), atol=1e-12)
    np.testing.assert_allclose(o[0, 2:, 0], np.array(cw["output_2"]), atol=1e-12)
    np.testing.assert_allclose(r2[0, 0], np.array(cw["R_2"]), atol=1e-12)
    _, r1 = oracle.chunkwise(q[:, :2], k[:, :2], v[:, :2], g, C)
    np.testing.assert_allclose(r1[0, 0], np.array(cw["R_1"]), atol=1e-12)
    # chunk 2 from a zero state is its inner part alone; from R_1 it adds the cross part
    inner2, _ = oracle.chunkwise(q[:, 2:], k[:, 2:], v[:, 2:], g, C)
    np.testing.assert_allclose(inner2[0, :, 0], np.array(cw["inner_2"]), atol=1e-12)
    full2, _ = oracle.chunkwise(q[:, 2:], k[:, 2:], v[:, 2:], g, C, state_in=r1)
    np.testing.assert_allclose((full2 - inner2)[0, :, 0], np.array(cw["cross_2"]), atol=1e-12)


def test_gamma_one_reproduces_linear_attention_trace(golden):
    """gamma = 1 with keys phi(K) is the accumulate-only state of the linear-attention section."""
    la = golden["linear_attention_trace"]
    K = np.array(golden["running_example"]["K"], float)
    phi = np.where(K > 0, K + 1.0, np.exp(K))  # elu(x) + 1
    np.testing.assert_allclose(phi, np.array(la["phi_K"]), atol=0)
    q, _, v, _ = _example(golden)
    kk = phi[None, :, None, :]
    for n in range(1, 5):
        _, s = oracle.recurrent(q[:, :n], kk[:, :n], v[:, :n], np.array([1.0]))
        np.testing.assert_allclose(s[0, 0], np.array(la["S"][n - 1]), atol=1e-12)
        assert abs(np.linalg.norm(s[0, 0]) - la["frobenius"][n - 1]) <= la["tolerance"]


def test_rotation_table(golden):
    """One pair, theta = pi/4, query at position 4 and keys at 1..4: scores are cos / sin of distance."""
    rt = golden["rotation_table"]
    theta = np.array([rt["theta"]])
    eye = np.eye(4)[None, :, None, :]
    q = np.zeros((1, 4, 1, 2))
    q[..., 0] = 1.0
    kc = np.zeros((1, 4, 1, 2))
    kc[..., 0] = 1.0
    ks = np.zeros((1, 4, 1, 2))
    ks[..., 1] = 1.0
    g1 = np.array([1.0])
    for pos0 in (1, 1000):  # the table is indexed by distance only
        oc = oracle.parallel(q, kc, eye, g1, theta=theta, pos0=pos0)[0, 3, 0]
        os_ = oracle.parallel(q, ks, eye, g1, theta=theta, pos0=pos0)[0, 3, 0]
        np.testing.assert_allclose(oc, rt["cos"], atol=rt["tolerance"])
        # k = (0, 1): Re(1 * conj(i) * e^{i d theta}) = sin(d theta) in the conjugate-transpose form
        np.testing.assert_allclose(os_, rt["sin"], atol=rt["tolerance"])


def test_gamma_schedule_table(golden):
    gt = golden["gamma_table"]
    g = workloads.gamma_schedule(8).astype(np.float64)
    np.testing.assert_allclose(g, gt["gamma_printed"], atol=gt["tolerance"])
    assert g[0] == 0.96875 and g[7] == 0.999755859375
    win = np.log(0.01) / np.log(g[:4])
    np.testing.assert_array_equal(np.round(win).astype(int), gt["effective_window_printed"][:4])


def test_gamma_schedule_loglinear():
    """The larger models' schedule: endpoints 1 - 1/32 and 1 - 1/512 (exact in fp32), 1 - gamma in geometric
    progression between them, decays strictly slower head by head."""
    g = workloads.gamma_schedule_loglinear(16).astype(np.float64)
    assert g[0] == 1 - 1 / 32 and g[-1] == 1 - 1 / 512
    ratios = (1 - g[1:]) / (1 - g[:-1])
    np.testing.assert_allclose(ratios, (1 / 16) ** (1 / 15), rtol=1e-5)
    assert np.all(np.diff(g) > 0)


def _complex_unrolled(q, k, v, g, theta, pos0):
    """Paper summary's unrolled form in complex numbers, pure Python, for tiny inputs:
    o_n = sum_{m<=n} gamma^(n-m) Re[(Qc_n e^{i p_n theta}) (Kc_m e^{i p_m theta})^dagger] v_m."""
    B, N, H, dk = q.shape
    dv = v.shape[3]
    out = np.zeros((B, N, H, dv))
    for b in range(B):
        for h in range(H):
            for n in range(N):
                for m in range(n + 1):
                    s = 0j
                    for i in range(dk // 2):
                        qc = complex(q[b, n, h, 2 * i], q[b, n, h, 2 * i + 1])
                        kc = complex(k[b, m, h, 2 * i], k[b, m, h, 2 * i + 1])
                        a = qc * complex(math.cos((pos0 + n) * theta[i]), math.sin((pos0 + n) * theta[i]))
                        c = kc * complex(math.cos((pos0 + m) * theta[i]), math.sin((pos0 + m) * theta[i]))
                        s += a * c.conjugate()
                    w = (g[h] ** (n - m)) * s.real
                    out[b, n, h, :] += w * v[b, m, h, :]
    return out


def test_rotation_matches_complex_form():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 9, 2, 6))
    k = rng.standard_normal((1, 9, 2, 6))
    v = rng.standard_normal((1, 9, 2, 3))
    g = np.array([0.9, 0.75])
    theta = np.array([0.3, 1.1, 2.9])
    want = _complex_unrolled(q, k, v, g, theta, pos0=5)
    for got in (oracle.parallel(q, k, v, g, theta=theta, pos0=5),
                oracle.recurrent(q, k, v, g, theta=theta, pos0=5)[0],
                oracle.chunkwise(q, k, v, g, 4, theta=theta, pos0=5)[0]):
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_gamma_one_no_rotation_is_causal_linear_attention():
    """gamma = 1, theta = 0: o_n = q_n sum_{m<=n} k_m^T v_m (numpy cumsum of outer products)."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 13, 3, 4))
    k = rng.standard_normal((2, 13, 3, 4))
    v = rng.standard_normal((2, 13, 3, 5))
    g = np.ones(3)
    outer = np.einsum("bnhi,bnhj->bnhij", k, v)
    S = np.cumsum(outer, axis=1)
    want = np.einsum("bnhi,bnhij->bnhj", q, S)
    for got in (oracle.parallel(q, k, v, g),
                oracle.recurrent(q, k, v, g)[0],
                oracle.chunkwise(q, k, v, g, 5)[0]):
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    _, s = oracle.recurrent(q, k, v, g)
    np.testing.assert_allclose(s, S[:, -1], rtol=1e-12, atol=1e-12)


def test_single_token_decay_closed_form():
    """One key/value pair followed by zero keys: o_n = gamma^(n-m) (q_n . k_m) v_m exactly."""
    N, g = 40, 0.96875
    q = np.zeros((1, N, 1, 2))
    k = np.zeros((1, N, 1, 2))
    v = np.zeros((1, N, 1, 1))
    q[0, :, 0, 0] = 1.0
    k[0, 3, 0, 0] = 2.0
    v[0, 3, 0, 0] = 1.5
    want = np.zeros(N)
    want[3:] = 3.0 * g ** np.arange(N - 3)
    for got in (oracle.parallel(q, k, v, [g]),
                oracle.recurrent(q, k, v, [g])[0],
                oracle.chunkwise(q, k, v, [g], 16)[0]):
        np.testing.assert_allclose(got[0, :, 0, 0], want, rtol=1e-13, atol=0)
