"""Pins of the oracle's paged decode step (oracle.decode_paged) against
things other than itself: torch's float64 scaled_dot_product_attention on the
un-paged keys, the last row of the oracle's causal prefill attention (pinned
on its own in test_oracle_pins.py), a 40-digit brute force, and closed forms
(one key, constant values per key/value head, an empty sequence).  The
caches in these tests are built by scattering contiguous keys into randomly
permuted pages, so a wrong page or slot index in the gather fails them."""
import math

import mpmath
import numpy as np
import pytest
import torch

from causal_prefill_attention_attn_amd.synth import to_bf16_bits
from decode_util import scatter as _scatter

BF16, FP8 = 0, 1


def _dec_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def _case(rng, B, lmax, hq, hkv, dqk, dv=128):
    q = to_bf16_bits(rng.standard_normal((B, hq, dqk)).astype(np.float32))
    k = to_bf16_bits(rng.standard_normal((B, lmax, hkv, dqk)).astype(np.float32))
    v = to_bf16_bits(rng.standard_normal((B, lmax, hkv, dv)).astype(np.float32))
    return q, k, v


@pytest.mark.parametrize("hq,hkv,dqk,ps", [(4, 4, 128, 16), (8, 2, 128, 64), (4, 1, 192, 32)])
def test_decode_matches_torch_sdpa_on_unpaged_keys(oracle, hq, hkv, dqk, ps):
    rng = np.random.default_rng(11 + hq + dqk + ps)
    lens = [1, 17, 64, 100]
    q, k, v = _case(rng, len(lens), max(lens), hq, hkv, dqk)
    kp, vp, table = _scatter(rng, k, v, lens, ps)
    tau = 1.0 / math.sqrt(dqk)
    o, lse = oracle.decode_paged(q, kp, vp, table, np.array(lens), BF16, tau)
    g = hq // hkv
    for b, n in enumerate(lens):
        qt = torch.from_numpy(_dec_bf16(q[b]))[:, None, :]                   # [hq, 1, d]
        kt = torch.from_numpy(_dec_bf16(k[b, :n])).permute(1, 0, 2)         # [hkv, n, d]
        vt = torch.from_numpy(_dec_bf16(v[b, :n])).permute(1, 0, 2)
        kt = kt.repeat_interleave(g, 0).contiguous()
        vt = vt.repeat_interleave(g, 0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=tau)[:, 0]
        s = tau * torch.einsum("hd,hnd->hn", qt[:, 0], kt)
        np.testing.assert_allclose(o[b], ref.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, -1).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", [BF16, FP8])
def test_decode_is_last_row_of_causal_prefill(oracle, dtype):
    rng = np.random.default_rng(5 + dtype)
    B, S, H, d = 1, 75, 2, 128
    x = [rng.standard_normal((B, S, H, d)).astype(np.float32) for _ in range(3)]
    if dtype == BF16:
        enc, ds = [to_bf16_bits(t) for t in x], [1.0] * 3
    else:
        ds = [oracle.descale_amax(t) for t in x]
        enc = [oracle.quantize_e4m3(t, s) for t, s in zip(x, ds)]
    tau = 0.09
    ro, rl = oracle.attention(*enc, dtype, tau, True, rows=np.array([S - 1]), q_descale=ds[0],
                              k_descale=ds[1], v_descale=ds[2])
    ps = 16
    kp, vp, table = _scatter(rng, enc[1], enc[2], [S], ps)
    o, lse = oracle.decode_paged(enc[0][:, S - 1], kp, vp, table, np.array([S]), dtype, tau,
                                 q_descale=ds[0], k_descale=ds[1], v_descale=ds[2])
    np.testing.assert_allclose(o[0], ro[0, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0], rl[0, :, 0], rtol=1e-12, atol=1e-13)


def test_decode_brute_force_40_digits_with_groups(oracle):
    """2 query heads per key/value head, 3 sequences, page size 16: every
    output against sum_j v_j / sum_j' exp(s_j' - s_j) in 40 digits."""
    mpmath.mp.dps = 40
    rng = np.random.default_rng(3)
    lens, hq, hkv, d = [5, 16, 23], 4, 2, 128
    q, k, v = _case(rng, 3, 23, hq, hkv, d)
    ps = 16
    kp, vp, table = _scatter(rng, k, v, lens, ps)
    tau = 0.1
    o, lse = oracle.decode_paged(q, kp, vp, table, np.array(lens), BF16, tau)
    qd, kd, vd = _dec_bf16(q), _dec_bf16(k), _dec_bf16(v)
    for b, n in enumerate(lens):
        for h in range(hq):
            hk = h // (hq // hkv)
            s = [tau * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(c))
                                   for a, c in zip(qd[b, h], kd[b, j, hk])) for j in range(n)]
            w = [1 / mpmath.fsum(mpmath.exp(s2 - s1) for s2 in s) for s1 in s]
            for e in range(0, d, 37):
                ref = mpmath.fsum(w[j] * mpmath.mpf(float(vd[b, j, hk, e])) for j in range(n))
                assert abs(o[b, h, e] - float(ref)) <= 1e-13 * (1 + abs(float(ref)))
            ref_lse = mpmath.log(mpmath.fsum(mpmath.exp(x) for x in s))
            assert abs(lse[b, h] - float(ref_lse)) <= 1e-13 * (1 + abs(float(ref_lse)))


def test_decode_single_key_and_empty_sequence(oracle):
    rng = np.random.default_rng(9)
    q, k, v = _case(rng, 2, 1, 2, 2, 128)
    kp, vp, table = _scatter(rng, k, v, [1, 0], 16)
    tau = 0.125
    o, lse = oracle.decode_paged(q, kp, vp, table, np.array([1, 0]), BF16, tau)
    np.testing.assert_array_equal(o[0], _dec_bf16(v[0, 0]))      # softmax of one score is 1
    np.testing.assert_allclose(lse[0], tau * np.einsum("hd,hd->h", _dec_bf16(q[0]), _dec_bf16(k[0, 0])),
                               rtol=1e-14)
    assert (o[1] == 0).all() and np.isneginf(lse[1]).all()


def test_decode_query_head_to_kv_head_mapping(oracle):
    """With 4 query heads per key/value head, query heads 0-3 must read head 0
    and 4-7 head 1: constant values per head make the output that constant."""
    rng = np.random.default_rng(4)
    lens = [40]
    q, k, _ = _case(rng, 1, 40, 8, 2, 128)
    v = np.empty((1, 40, 2, 128), np.uint16)
    v[:, :, 0] = to_bf16_bits(np.float32(1.5))
    v[:, :, 1] = to_bf16_bits(np.float32(-2.0))
    kp, vp, table = _scatter(rng, k, v, lens, 16)
    o, _ = oracle.decode_paged(q, kp, vp, table, np.array(lens), BF16, 0.1)
    np.testing.assert_allclose(o[0, :4], 1.5, rtol=1e-14)
    np.testing.assert_allclose(o[0, 4:], -2.0, rtol=1e-14)


def test_decode_fp8_descales(oracle):
    """Descales multiply the decoded codes: q and k descales scale the logits,
    the v descale scales the output."""
    rng = np.random.default_rng(6)
    q = rng.integers(0, 0x7F, (1, 2, 128), dtype=np.uint8) & 0x3F
    kp = rng.integers(0, 0x7F, (2, 16, 2, 128), dtype=np.uint8) & 0x3F
    vp = rng.integers(0, 0xFF, (2, 16, 2, 128), dtype=np.uint8) & 0xBF
    table, lens = np.array([[1, 0]], np.int32), np.array([20])
    o1, l1 = oracle.decode_paged(q, kp, vp, table, lens, FP8, 0.05)
    o2, l2 = oracle.decode_paged(q, kp, vp, table, lens, FP8, 0.05 / 6.0, q_descale=2.0,
                                 k_descale=3.0, v_descale=0.25)
    np.testing.assert_allclose(o2, 0.25 * o1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)
