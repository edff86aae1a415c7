"""Pins of the CPU fp64 oracle against things other than itself.

Each test fixes the oracle to an independent fact: a library routine
(torch's scaled_dot_product_attention in float64), a brute-force evaluation
in 40-digit arithmetic with a different formulation, closed forms of special
cases, and invariants of the definition.  Together they catch a dropped term,
a wrong sign, a wrong index, a transposed operand or a wrong mask.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

from causal_prefill_attention_attn_amd.synth import to_bf16_bits



def _bf16(x):
    return to_bf16_bits(np.asarray(x, np.float32))


def _dec_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def _small_int_tensor(rng, shape, lo=-3, hi=4):
    # small integers are exact in bf16 and sums of them stay exact
    return rng.integers(lo, hi, size=shape).astype(np.float32)


# ---------------------------------------------------------------- P1 brute force
def _mp_attention(qv, kv, vv, tau, causal):
    """40-digit softmax written without max subtraction:
    w_ij = 1 / sum_j' exp(s_ij' - s_ij);  lse_i = log sum_j exp(s_ij)."""
    mpmath.mp.dps = 40
    B, S, H, dqk = qv.shape
    dv = vv.shape[3]
    o = np.zeros((B, S, H, dv))
    lse = np.zeros((B, H, S))
    for b in range(B):
        for h in range(H):
            for i in range(S):
                js = range(i + 1) if causal else range(S)
                s = {j: mpmath.mpf(tau) * mpmath.fsum(mpmath.mpf(float(qv[b, i, h, c])) * mpmath.mpf(float(kv[b, j, h, c]))
                                                    for c in range(dqk)) for j in js}
                lse[b, h, i] = float(mpmath.log(mpmath.fsum(mpmath.exp(s[j]) for j in js)))
                for c in range(dv):
                    acc = mpmath.mpf(0)
                    for j in js:
                        w = 1 / mpmath.fsum(mpmath.exp(s[jj] - s[j]) for jj in js)
                        acc += w * mpmath.mpf(float(vv[b, j, h, c]))
                    o[b, i, h, c] = float(acc)
    return o, lse


@pytest.mark.parametrize("B,H,S,dqk,dv", [(1, 1, 1, 4, 4), (1, 2, 2, 1, 2), (2, 1, 3, 2, 1), (1, 1, 5, 8, 8),
                                          (2, 2, 8, 4, 2), (1, 1, 17, 8, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_p1_bruteforce_mpmath(oracle, B, H, S, dqk, dv, causal):
    rng = np.random.default_rng(S * 100 + dqk + 7 * causal)
    q = _bf16(rng.standard_normal((B, S, H, dqk)))
    k = _bf16(rng.standard_normal((B, S, H, dqk)))
    v = _bf16(rng.standard_normal((B, S, H, dv)))
    tau = 0.7
    o, lse = oracle.attention(q, k, v, oracle.BF16, tau, causal)
    ro, rl = _mp_attention(_dec_bf16(q), _dec_bf16(k), _dec_bf16(v), tau, causal)
    np.testing.assert_allclose(o, ro, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------- library routine (SDPA)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("B,H,S,dqk,dv", [(2, 3, 37, 128, 128), (1, 2, 64, 192, 128), (1, 1, 130, 16, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_sdpa_fp64(oracle, dtype, B, H, S, dqk, dv, causal):
    rng = np.random.default_rng(11 + S + dqk)
    qf = rng.standard_normal((B, S, H, dqk)).astype(np.float32)
    kf = rng.standard_normal((B, S, H, dqk)).astype(np.float32)
    vf = rng.standard_normal((B, S, H, dv)).astype(np.float32)
    tau = 1.0 / math.sqrt(dqk)
    if dtype == "bf16":
        q, k, v = _bf16(qf), _bf16(kf), _bf16(vf)
        qd = kd = vd = 1.0
        qh, kh, vh = _dec_bf16(q), _dec_bf16(k), _dec_bf16(v)
        dt = oracle.BF16
    else:
        qd, kd, vd = (oracle.descale_amax(x) for x in (qf, kf, vf))
        q, k, v = (oracle.quantize_e4m3(x, d) for x, d in ((qf, qd), (kf, kd), (vf, vd)))
        dec = lambda c, d: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy() * float(np.float32(d))
        qh, kh, vh = dec(q, qd), dec(k, kd), dec(v, vd)
        dt = oracle.FP8
    o, lse = oracle.attention(q, k, v, dt, tau, causal, q_descale=qd, k_descale=kd, v_descale=vd)
    # torch wants [B,H,S,D]
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous() for x in (qh, kh, vh))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=tau)
    ref = ref.permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)
    scores = torch.einsum("bhid,bhjd->bhij", tq, tk) * tau
    if causal:
        scores = scores.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(scores, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


# -------------------------------------------------------- P2 rows sum to one
def test_p2_weights_rows_sum_to_one_and_mask(oracle):
    # V = identity basis (v_j = e_j) makes o_i the weight row w_i.
    S = 24
    rng = np.random.default_rng(3)
    q = _bf16(rng.standard_normal((1, S, 1, 16)))
    k = _bf16(rng.standard_normal((1, S, 1, 16)))
    v = _bf16(np.eye(S, dtype=np.float32).reshape(1, S, 1, S))
    for causal in (True, False):
        w, _ = oracle.attention(q, k, v, oracle.BF16, 0.5, causal)
        w = w[0, :, 0, :]
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert (w >= 0).all()
        if causal:
            assert (w[np.triu_indices(S, 1)] == 0).all()
            assert (w[np.tril_indices(S)] > 0).all()
        else:
            assert (w > 0).all()


# ------------------------------------------------------------- P3 query 0
def test_p3_query_zero_returns_v0(oracle):
    rng = np.random.default_rng(5)
    B, S, H, D = 2, 9, 3, 32
    q = _bf16(rng.standard_normal((B, S, H, D)))
    k = _bf16(rng.standard_normal((B, S, H, D)))
    v = _bf16(rng.standard_normal((B, S, H, D)))
    tau = 0.3
    o, lse = oracle.attention(q, k, v, oracle.BF16, tau, True)
    vh, qh, kh = _dec_bf16(v), _dec_bf16(q), _dec_bf16(k)
    assert np.array_equal(o[:, 0], vh[:, 0])
    s00 = tau * np.einsum("bhc,bhc->bh", qh[:, 0], kh[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], s00, rtol=1e-15, atol=1e-15)


# --------------------------------------------------------- P4 uniform scores
@pytest.mark.parametrize("how", ["q_zero", "tau_zero", "k_equal"])
def test_p4_uniform_scores_prefix_mean(oracle, how):
    rng = np.random.default_rng(8)
    B, S, H, D = 1, 40, 2, 8
    qf = rng.standard_normal((B, S, H, D)).astype(np.float32)
    kf = rng.standard_normal((B, S, H, D)).astype(np.float32)
    tau = 0.9
    if how == "q_zero":
        qf[:] = 0
    elif how == "tau_zero":
        tau = 0.0
    else:
        kf[:] = kf[:, :1]
    q, k = _bf16(qf), _bf16(kf)
    v = _bf16(rng.standard_normal((B, S, H, D)))
    vh = _dec_bf16(v)
    o, lse = oracle.attention(q, k, v, oracle.BF16, tau, True)
    prefix = np.cumsum(vh, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    np.testing.assert_allclose(o, prefix, rtol=1e-13, atol=1e-14)
    s_const = tau * np.einsum("bihc,bhc->bhi", _dec_bf16(q), _dec_bf16(k)[:, 0])
    np.testing.assert_allclose(lse, s_const + np.log(np.arange(1, S + 1))[None, None, :], rtol=1e-13, atol=1e-13)
    on, ln = oracle.attention(q, k, v, oracle.BF16, tau, False)
    np.testing.assert_allclose(on, np.broadcast_to(vh.mean(axis=1, keepdims=True), on.shape), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ln, s_const + np.log(S), rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------- P5 S = 2
def test_p5_two_tokens_closed_form(oracle):
    rng = np.random.default_rng(9)
    q = _bf16(rng.standard_normal((1, 2, 1, 4)))
    k = _bf16(rng.standard_normal((1, 2, 1, 4)))
    v = _bf16(rng.standard_normal((1, 2, 1, 3)))
    tau = 1.3
    o, lse = oracle.attention(q, k, v, oracle.BF16, tau, True)
    qh, kh, vh = _dec_bf16(q)[0, :, 0], _dec_bf16(k)[0, :, 0], _dec_bf16(v)[0, :, 0]
    s10, s11 = tau * qh[1] @ kh[0], tau * qh[1] @ kh[1]
    e0, e1 = math.exp(s10), math.exp(s11)
    np.testing.assert_allclose(o[0, 1, 0], (e0 * vh[0] + e1 * vh[1]) / (e0 + e1), rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0, 1], math.log(e0 + e1), rtol=1e-14)


# ---------------------------------------------------------- P6 one-hot limit
def test_p6_one_hot_limit(oracle):
    rng = np.random.default_rng(10)
    S, D = 30, 16
    q = _bf16(rng.standard_normal((1, S, 1, D)))
    k = _bf16(rng.standard_normal((1, S, 1, D)))
    v = _bf16(rng.standard_normal((1, S, 1, D)))
    qh, kh, vh = _dec_bf16(q)[0, :, 0], _dec_bf16(k)[0, :, 0], _dec_bf16(v)[0, :, 0]
    o, _ = oracle.attention(q, k, v, oracle.BF16, 1e4, True)
    for i in range(S):
        s = qh[i] @ kh[: i + 1].T
        top2 = np.sort(s)[-2:] if i > 0 else None
        if top2 is not None and top2[1] - top2[0] < 1e-2:
            continue  # near tie: the limit is a mixture
        np.testing.assert_allclose(o[0, i, 0], vh[int(np.argmax(s))], rtol=0, atol=1e-12)


# ----------------------------------------------------- P7 shift invariance
def test_p7_key_shift_invariance(oracle):
    rng = np.random.default_rng(12)
    B, S, H, D = 1, 20, 2, 8
    qf = _small_int_tensor(rng, (B, S, H, D))
    kf = _small_int_tensor(rng, (B, S, H, D))
    c = _small_int_tensor(rng, (1, 1, H, D))
    v = _bf16(rng.standard_normal((B, S, H, D)))
    tau = 0.25
    o1, l1 = oracle.attention(_bf16(qf), _bf16(kf), v, oracle.BF16, tau, True)
    o2, l2 = oracle.attention(_bf16(qf), _bf16(kf + c), v, oracle.BF16, tau, True)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-14)
    shift = tau * np.einsum("bihc,bhc->bhi", qf.astype(np.float64), c[:, 0].astype(np.float64))
    np.testing.assert_allclose(l2 - l1, shift, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ P8 structure
def test_p8_linearity_in_v(oracle):
    rng = np.random.default_rng(13)
    B, S, H, D = 1, 16, 2, 8
    q = _bf16(rng.standard_normal((B, S, H, D)))
    k = _bf16(rng.standard_normal((B, S, H, D)))
    v1 = _small_int_tensor(rng, (B, S, H, D))
    v2 = _small_int_tensor(rng, (B, S, H, D))
    oa, _ = oracle.attention(q, k, _bf16(v1), oracle.BF16, 0.5, True)
    ob, _ = oracle.attention(q, k, _bf16(v2), oracle.BF16, 0.5, True)
    oc, _ = oracle.attention(q, k, _bf16(v1 + 2 * v2), oracle.BF16, 0.5, True)
    np.testing.assert_allclose(oc, oa + 2 * ob, rtol=1e-12, atol=1e-12)


def test_p8_head_and_batch_permutation(oracle):
    rng = np.random.default_rng(14)
    B, S, H, D = 3, 11, 4, 8
    q, k, v = (_bf16(rng.standard_normal((B, S, H, D))) for _ in range(3))
    o, l = oracle.attention(q, k, v, oracle.BF16, 0.4, True)
    hp, bp = np.array([2, 0, 3, 1]), np.array([1, 2, 0])
    o2, l2 = oracle.attention(q[bp][:, :, hp], k[bp][:, :, hp], v[bp][:, :, hp], oracle.BF16, 0.4, True)
    assert np.array_equal(o2, o[bp][:, :, hp])
    assert np.array_equal(l2, l[bp][:, hp])


def test_p8_causal_vs_noncausal(oracle):
    rng = np.random.default_rng(15)
    q, k, v = (_bf16(rng.standard_normal((1, 7, 1, 8))) for _ in range(3))
    oc, lc = oracle.attention(q, k, v, oracle.BF16, 0.4, True)
    on, ln = oracle.attention(q, k, v, oracle.BF16, 0.4, False)
    assert np.array_equal(oc[:, -1], on[:, -1]) and np.array_equal(lc[..., -1], ln[..., -1])
    assert not np.allclose(oc[:, :-1], on[:, :-1])
    o1, l1 = oracle.attention(q[:, :1], k[:, :1], v[:, :1], oracle.BF16, 0.4, True)
    o2, l2 = oracle.attention(q[:, :1], k[:, :1], v[:, :1], oracle.BF16, 0.4, False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_row_subset_matches_full(oracle):
    rng = np.random.default_rng(16)
    q, k, v = (_bf16(rng.standard_normal((2, 50, 3, 16))) for _ in range(3))
    of, lf = oracle.attention(q, k, v, oracle.BF16, 0.3, True)
    rows = np.array([0, 7, 31, 49])
    os_, ls = oracle.attention(q, k, v, oracle.BF16, 0.3, True, rows=rows)
    assert np.array_equal(os_, of[:, rows]) and np.array_equal(ls, lf[:, :, rows])


def test_fp8_descales_are_applied(oracle):
    """FP8 path: attention on (codes, descales) equals attention on the
    decoded-and-scaled values fed as exact bf16-representable integers."""
    rng = np.random.default_rng(17)
    B, S, H, D = 1, 12, 1, 8
    codes = [rng.choice(np.array([0x30, 0x38, 0x40, 0xB8, 0xC0, 0x00], np.uint8), size=(B, S, H, D)) for _ in range(3)]
    ds = (2.0, 0.5, 4.0)
    o8, l8 = oracle.attention(*codes, oracle.FP8, 0.3, True, q_descale=ds[0], k_descale=ds[1], v_descale=ds[2])
    vals = [oracle.decode_e4m3(c) * d for c, d in zip(codes, ds)]
    ob, lb = oracle.attention(*(_bf16(x) for x in vals), oracle.BF16, 0.3, True)
    np.testing.assert_allclose(o8, ob, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l8, lb, rtol=1e-14, atol=1e-15)


def test_lse_merge_of_key_halves_is_causal_attention(oracle):
    """Pins the shard merge used by the sequence-parallel test: the oracle's
    own non-causal attention over the first key half and causal attention
    over the second half, merged through their LSE, equal its causal
    attention of the second-half rows over the whole sequence."""
    from merge_util import merge
    rng = np.random.default_rng(5150)
    N, H, D = 40, 2, 16
    q, k, v = (rng.standard_normal((1, 2 * N, H, D)).astype(np.float32) for _ in range(3))
    qb, kb, vb = (to_bf16_bits(x) for x in (q, k, v))
    tau = 0.3
    q2 = np.ascontiguousarray(qb[:, N:])
    oa, la = oracle.attention(q2, np.ascontiguousarray(kb[:, :N]), np.ascontiguousarray(vb[:, :N]),
                              oracle.BF16, tau, False)
    ob, lb = oracle.attention(q2, np.ascontiguousarray(kb[:, N:]), np.ascontiguousarray(vb[:, N:]),
                              oracle.BF16, tau, True)
    mo, ml = merge([(oa, la), (ob, lb)])
    ro, rl = oracle.attention(qb, kb, vb, oracle.BF16, tau, True, rows=np.arange(N, 2 * N))
    np.testing.assert_allclose(mo, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ml, rl, rtol=1e-12, atol=1e-12)


# ---- Hadamard rotation (the step before FP8 quantization)
def test_hadamard_matrix_small_orders_by_hand(oracle):
    s = 1 / math.sqrt(2)
    np.testing.assert_array_equal(oracle.hadamard_matrix(1), [[1.0]])
    np.testing.assert_allclose(oracle.hadamard_matrix(2), [[s, s], [s, -s]], rtol=0, atol=1e-16)
    h4 = 0.5 * np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])
    np.testing.assert_allclose(oracle.hadamard_matrix(4), h4, rtol=0, atol=1e-16)


@pytest.mark.parametrize("n", [64, 128])
def test_hadamard_matrix_orthogonal_symmetric_pm_entries(oracle, n):
    h = oracle.hadamard_matrix(n)
    np.testing.assert_allclose(h @ h.T, np.eye(n), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(h, h.T)
    np.testing.assert_allclose(np.abs(h), np.full((n, n), 1 / math.sqrt(n)), rtol=1e-15)
    # Walsh functions: entry (i, j) has sign (-1)^popcount(i & j)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    sign = np.vectorize(lambda a: -1.0 if bin(a).count("1") % 2 else 1.0)(i & j)
    np.testing.assert_array_equal(np.sign(h), sign)


@pytest.mark.parametrize("d", [128, 192])
def test_hadamard_rows_are_isometric_and_self_inverse(oracle, d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, 3, d))
    y = oracle.hadamard(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(oracle.hadamard(y), x, rtol=0, atol=1e-13)
    # block structure, as read: one block of 128 at d = 128, three blocks of
    # 64 at d = 192.  A unit vector in a block spreads, with equal
    # magnitudes 1/sqrt(block), over that block and nowhere else.
    n = {128: 128, 192: 64}[d]
    assert oracle.hadamard_block(d) == n
    for c in (0, n - 1, d - n, d - 1):
        e = np.zeros(d)
        e[c] = 1.0
        r = oracle.hadamard(e)
        lo = (c // n) * n
        inside = np.zeros(d, bool)
        inside[lo:lo + n] = True
        assert np.all(r[~inside] == 0), c
        np.testing.assert_allclose(np.abs(r[inside]), 1 / math.sqrt(n), rtol=1e-15)


def test_hadamard_spreads_an_outlier_channel(oracle):
    """The reason for the rotation: one dominant channel becomes d equal
    entries, so the per-tensor FP8 scale no longer follows the outlier."""
    x = np.zeros(128)
    x[5] = 100.0
    y = oracle.hadamard(x)
    assert np.max(np.abs(y)) == pytest.approx(100.0 / math.sqrt(128), rel=1e-15)
