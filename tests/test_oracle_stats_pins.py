"""Pins of the oracle's per-row statistics (kappa, wmax, sabs) against
closed forms, special cases and a Monte Carlo evaluation of what kappa means,
none of which reuses the oracle's formulas.

kappa_i is the factor by which independent relative errors of a row's
probabilities (RMS e) become a relative error of the row (RMS e * kappa_i)
to first order; the GPU parity tests bound each FP8 row by it.  wmax_i is
the softmax mass at the row maximum, sabs_i the magnitude scale of the
largest score's terms.
"""
import numpy as np
import pytest
import torch

from causal_prefill_attention_attn_amd.synth import to_bf16_bits


def _bf16(x):
    return to_bf16_bits(np.asarray(x, np.float32))


def _dec(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_query_zero_and_constant_v(oracle):
    rng = np.random.default_rng(1)
    q = _bf16(rng.standard_normal((2, 40, 3, 16)))
    k = _bf16(rng.standard_normal((2, 40, 3, 16)))
    v = _bf16(rng.standard_normal((2, 40, 3, 8)))
    _, _, st = oracle.attention(q, k, v, oracle.BF16, 0.5, True, stats=True)
    # query 0 sees one key: o = v0, so every term of kappa vanishes, and all
    # of the mass sits at the maximum
    assert np.all(st["kappa"][:, :, 0] == 0.0)
    assert np.all(st["wmax"][:, :, 0] == 1.0)
    assert np.all(st["kappa"][:, :, 1:] > 0.0)
    # equal value rows: o = v for every row, whatever the weights
    vc = np.broadcast_to(v[:, :1], v.shape).copy()
    _, _, st = oracle.attention(q, k, vc, oracle.BF16, 0.5, True, stats=True)
    assert np.all(st["kappa"] <= 1e-14)  # o equals v up to the rounding of the weighted sum


def test_two_keys_closed_form(oracle):
    """S = 2, row 1: with weights w0, w1 (w0 + w1 = 1) the row is
    o = w0 v0 + w1 v1, so v0 - o = w1 (v0 - v1) and v1 - o = w0 (v1 - v0):
    kappa = sqrt(2) w0 w1 |v0 - v1| / |o|; wmax = max(w0, w1)."""
    rng = np.random.default_rng(2)
    for trial in range(20):
        q = _bf16(rng.standard_normal((1, 2, 1, 8)))
        k = _bf16(rng.standard_normal((1, 2, 1, 8)))
        v = _bf16(rng.standard_normal((1, 2, 1, 6)))
        tau = 0.9
        _, _, st = oracle.attention(q, k, v, oracle.BF16, tau, True, stats=True)
        qd, kd, vd = _dec(q)[0, :, 0], _dec(k)[0, :, 0], _dec(v)[0, :, 0]
        s0, s1 = tau * qd[1] @ kd[0], tau * qd[1] @ kd[1]
        w1 = 1.0 / (1.0 + np.exp(s0 - s1))
        w0 = 1.0 - w1
        o = w0 * vd[0] + w1 * vd[1]
        kap = np.sqrt(2.0) * w0 * w1 * np.linalg.norm(vd[0] - vd[1]) / np.linalg.norm(o)
        np.testing.assert_allclose(st["kappa"][0, 0, 1], kap, rtol=1e-12)
        np.testing.assert_allclose(st["wmax"][0, 0, 1], max(w0, w1), rtol=1e-12)


def test_kappa_is_the_first_order_error_gain(oracle):
    """Monte Carlo: perturb each softmax weight by an independent relative
    error of RMS sigma, renormalise, and compare the mean squared relative
    change of the row with (sigma * kappa)^2.  The weights come from torch's
    float64 softmax, not from the oracle."""
    rng = np.random.default_rng(3)
    S, d = 24, 8
    q = _bf16(rng.standard_normal((1, S, 1, d)))
    k = _bf16(rng.standard_normal((1, S, 1, d)))
    v = _bf16(rng.standard_normal((1, S, 1, d)) + 0.5)
    tau = 0.8
    _, _, st = oracle.attention(q, k, v, oracle.BF16, tau, True, stats=True)
    qd, kd, vd = (torch.from_numpy(_dec(x)[0, :, 0]) for x in (q, k, v))
    sigma, n = 1e-5, 20000
    g = torch.Generator().manual_seed(4)
    for i in (3, 11, 23):
        w = torch.softmax(tau * (kd[: i + 1] @ qd[i]), dim=0)
        o = w @ vd[: i + 1]
        e = torch.randn((n, i + 1), generator=g, dtype=torch.float64) * sigma
        wp = w * (1 + e)
        op = (wp @ vd[: i + 1]) / wp.sum(dim=1, keepdim=True)
        ms = float(((op - o).norm(dim=1) ** 2).mean() / o.norm() ** 2)
        np.testing.assert_allclose(np.sqrt(ms) / sigma, st["kappa"][0, 0, i], rtol=0.03)


def test_wmax_with_ties_and_uniform_scores(oracle):
    rng = np.random.default_rng(5)
    S, d = 9, 4
    q = _bf16(rng.standard_normal((1, S, 1, d)))
    k = _bf16(rng.standard_normal((1, S, 1, d)))
    v = _bf16(rng.standard_normal((1, S, 1, d)))
    # all scores equal (Q = 0): every key is at the maximum
    _, _, st = oracle.attention(np.zeros_like(q), k, v, oracle.BF16, 1.0, True, stats=True)
    np.testing.assert_allclose(st["wmax"][0, 0], 1.0, rtol=1e-15)
    # keys 2 and 5 equal and far ahead of the rest for query 8: two keys share
    # the maximum, each with weight 1 / (2 + sum of the others' exp(s - m))
    kd = _dec(k)[0, :, 0].copy()
    qd = _dec(q)[0, 8, 0]
    big = np.sign(qd) * 4
    k2 = k.copy()
    k2[0, 2, 0] = k2[0, 5, 0] = _bf16(big)
    _, _, st = oracle.attention(q, k2, v, oracle.BF16, 1.0, True, stats=True)
    s = kd @ qd
    s[2] = s[5] = big @ qd
    e = np.exp(s - s.max())
    np.testing.assert_allclose(st["wmax"][0, 0, 8], 2.0 / e.sum(), rtol=1e-12)


def test_sabs_counts_magnitudes_not_the_cancelled_score(oracle):
    """q = all ones; k0 alternates +2, -2 (its score cancels to 0 while the
    sum of |q_c k_c| is 2 d), k1 = k2 = all ones (score and magnitude d).
    Query 0 sees key 0 only; query 2 weighs the magnitudes 2 d, d, d by
    its softmax weights 1, e^(tau d), e^(tau d) (normalised)."""
    d = 16
    q = np.ones((1, 3, 1, d), np.float32)
    k = np.ones((1, 3, 1, d), np.float32)
    k[0, 0, 0] = np.where(np.arange(d) % 2 == 0, 2.0, -2.0)
    v = np.ones((1, 3, 1, d), np.float32)
    tau = 0.25
    _, lse, st = oracle.attention(_bf16(q), _bf16(k), _bf16(v), oracle.BF16, tau, True, stats=True)
    assert lse[0, 0, 0] == 0.0
    assert st["sabs"][0, 0, 0] == tau * 2 * d
    e = np.exp(tau * d)
    np.testing.assert_allclose(st["sabs"][0, 0, 2], tau * (2 * d + 2 * e * d) / (1 + 2 * e),
                               rtol=1e-14)


def test_fp8_stats_use_descales(oracle):
    """Descales scale the scores (sabs by dq*dk) and leave kappa, which is
    invariant to a common scale of V, unchanged."""
    rng = np.random.default_rng(6)
    codes = [rng.integers(0, 0x7E, size=(1, 30, 2, 16), dtype=np.uint8) for _ in range(3)]
    _, _, a = oracle.attention(*codes, oracle.FP8, 0.3, True, stats=True)
    _, _, b = oracle.attention(*codes, oracle.FP8, 0.3, True, q_descale=1.0, k_descale=1.0,
                               v_descale=4.0, stats=True)
    np.testing.assert_allclose(a["kappa"], b["kappa"], rtol=1e-12)
    _, _, c = oracle.attention(*codes, oracle.FP8, 0.15, True, q_descale=2.0, k_descale=1.0,
                               stats=True)
    np.testing.assert_allclose(c["sabs"], a["sabs"], rtol=1e-12)
    np.testing.assert_allclose(c["wmax"], a["wmax"], rtol=1e-12)
