"""Hadamard rotation on the GPU against the fp64 oracle, and FP8 attention
of rotated Q, K, V (the step before quantization that "Precisao,
estabilidade e efeito na pratica" on the miraibroadcast.com page credits
with about half of the quantization error).

Parity: the rotation kernels against the oracle's block Sylvester matrix
product; rotated FP8 attention (rotate, quantize, attend, rotate O back)
against the oracle taking the same steps in fp64 from the same fp32 inputs.
Accuracy: plain and rotated FP8 attention against the oracle's attention of
the unquantized inputs (bf16-rounded), on inputs whose Q and K share a few
strong channels.  The gain depends on that: e4m3 is a floating-point format,
so a strong channel costs the other channels of its row no precision, and
the rotation helps by turning the large products of shared strong channels
into many small ones.  When the strong channels of Q and K differ, their
products stay small and the rotation only spreads the strong channels'
energy into every coordinate; the oracle then shows the score error about
2.6 times larger with the rotation than without (a measured fact, not a
test).
"""
import numpy as np
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg
from causal_prefill_attention_attn_amd import synth
from gpu_util import DEV, judge, o_to_f64, u8_to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [128, 192])
@pytest.mark.parametrize("rows", [1, 7, 1000])
def test_hadamard_f32_matches_oracle(oracle, d, rows):
    rng = np.random.default_rng(rows * d)
    x = (rng.standard_normal((rows, d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
    y = pkg.hadamard(torch.from_numpy(x).to(DEV)).cpu().numpy().astype(np.float64)
    ref = oracle.hadamard(x)
    err = np.abs(y - ref).max() / np.abs(ref).max()
    print("hadamard f32 d%d rows %d max rel err %.2e" % (d, rows, err))
    assert err <= 1e-6


@pytest.mark.parametrize("d", [128, 192])
def test_hadamard_in_place_and_self_inverse(oracle, d):
    rng = np.random.default_rng(d + 1)
    x = rng.standard_normal((333, d)).astype(np.float32)
    t = torch.from_numpy(x).to(DEV)
    pkg.hadamard(t, out=t)                       # in place
    np.testing.assert_allclose(t.cpu().numpy(), oracle.hadamard(x), rtol=0, atol=2e-6)
    pkg.hadamard(t, out=t)
    np.testing.assert_allclose(t.cpu().numpy(), x, rtol=0, atol=2e-6)


@pytest.mark.parametrize("d", [128, 192])
def test_hadamard_bf16_rounds_the_fp32_rotation(oracle, d):
    rng = np.random.default_rng(d + 2)
    bits = synth.to_bf16_bits(rng.standard_normal((257, d)).astype(np.float32))
    xb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    y = pkg.hadamard(xb).float().cpu().numpy().astype(np.float64)
    ref = oracle.hadamard(oracle.decode_bf16(bits))
    # one bf16 rounding of a value whose fp32 evaluation differs from fp64 by
    # far less than a bf16 unit: at most one unit (2^-7 relative to the value)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(y - ref) <= ulp * 1.0001), float(np.max(np.abs(y - ref) / ulp))


def _inputs(S, H, d_qk, outliers, seed, shared=True, scale=20.0):
    """Gaussian Q, K, V; Q and K carry a few channels `scale` times stronger,
    the same channels in both when `shared`."""
    rng = np.random.default_rng(seed)
    q, k = (rng.standard_normal((1, S, H, d_qk)).astype(np.float32) for _ in range(2))
    v = rng.standard_normal((1, S, H, 128)).astype(np.float32)
    ch = rng.choice(d_qk, size=outliers, replace=False)
    for x in (q, k):
        if not shared:
            ch = rng.choice(d_qk, size=outliers, replace=False)
        x[..., ch] *= scale
    return q, k, v


def _gpu_fp8(xs, rotate, tau):
    t = [torch.from_numpy(x).to(DEV) for x in xs]
    codes, ds = zip(*[pkg.quantize_fp8(x, rotate=rotate) for x in t])
    o, lse = pkg.flash_attn_func(*codes, softmax_scale=tau, causal=True, q_descale=ds[0],
                                 k_descale=ds[1], v_descale=ds[2])
    if rotate:
        o = pkg.hadamard(o)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def _oracle_fp8(oracle, xs, rotate, tau):
    xs = [oracle.hadamard(x).astype(np.float32) if rotate else x for x in xs]
    ds = [oracle.descale_amax(x) for x in xs]
    enc = [oracle.quantize_e4m3(x, dd) for x, dd in zip(xs, ds)]
    o, lse, st = oracle.attention(*enc, oracle.FP8, tau, True, q_descale=ds[0], k_descale=ds[1],
                                  v_descale=ds[2], stats=True)
    # the rotation back is orthogonal: row norms, hence the per-row
    # statistics, are those of the rotated problem
    return (oracle.hadamard(o) if rotate else o), lse, st


def _pooled(go, ro):
    return float(np.linalg.norm(go - ro) / np.linalg.norm(ro))


@pytest.mark.parametrize("d_qk", [128, 192])
def test_rotated_fp8_attention_matches_oracle(oracle, d_qk):
    S, H = 700, 2
    tau = 1.0 / np.sqrt(d_qk)
    # strong channels (disjoint in Q and K) that keep the logits moderate: the
    # check is the rotate-quantize-attend-rotate pipeline, not FP8 at extreme
    # logit ranges (covered by the unrotated FP8 tests)
    xs = _inputs(S, H, d_qk, 4, 4242 + d_qk, shared=False, scale=5.0)
    go, gl = _gpu_fp8(xs, True, tau)
    ro, rl, st = _oracle_fp8(oracle, xs, True, tau)
    judge("rotated fp8 d%d" % d_qk, synth.FP8, go, gl, ro, rl, st)


@pytest.mark.parametrize("d_qk", [128, 192])
def test_rotation_reduces_fp8_error_with_shared_strong_channels(oracle, d_qk):
    S, H = 700, 2
    tau = 0.05 / np.sqrt(d_qk)        # logit spread ~2: score errors show in O
    xs = _inputs(S, H, d_qk, 4, 777 + d_qk)
    enc = [synth.to_bf16_bits(x) for x in xs]
    ref_o, ref_l = oracle.attention(*enc, oracle.BF16, tau, True)
    res = {}
    for rotate in (False, True):
        go, gl = _gpu_fp8(xs, rotate, tau)
        res[rotate] = (_pooled(go, ref_o), float(np.abs(gl - ref_l).mean()))
    print("d%d error vs unquantized: plain O %.3e lse %.3e | rotated O %.3e lse %.3e" % (
        d_qk, res[False][0], res[False][1], res[True][0], res[True][1]))
    # the pages: about half of the quantization error; the oracle gives
    # 0.38-0.47 of the plain O error on such inputs
    assert res[True][0] < 0.6 * res[False][0]
    assert res[True][1] < res[False][1]


@pytest.mark.parametrize("d", [128, 192])
def test_fused_rotation_quantization(oracle, d):
    """The fused passes equal rotation followed by the plain quantizer (same
    fp32 rotation, bit for bit), and the oracle's quantizer applied to its
    fp64 rotation rounded to fp32 up to codes at rounding ties."""
    rng = np.random.default_rng(d + 3)
    x = (rng.standard_normal((999, d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
    x[:, 7] *= 30.0
    t = torch.from_numpy(x).to(DEV)
    codes_f, ds_f = pkg.quantize_fp8(t, rotate=True)
    codes_u, ds_u = pkg.quantize_fp8(pkg.hadamard(t))
    assert ds_f == ds_u
    assert torch.equal(codes_f, codes_u)
    xr = oracle.hadamard(x).astype(np.float32)
    ds_o = oracle.descale_amax(xr)
    assert abs(ds_o - ds_f) <= 1e-6 * ds_o
    ref = oracle.quantize_e4m3(xr, ds_f).astype(np.int16)
    got = codes_f.cpu().numpy().astype(np.int16)
    diff = np.abs(got - ref)
    print("fused rotate+quantize d%d: %d of %d codes differ from the oracle's" % (d, int((diff > 0).sum()), diff.size))
    assert diff.max() <= 1 and (diff > 0).mean() <= 1e-3


@pytest.mark.parametrize("d", [128, 192])
def test_both_layouts_give_the_same_bits(oracle, d):
    """16-byte-aligned buffers take the 16-elements-per-thread kernels, other
    buffers the row-per-wave ones; both run the same butterflies in the same
    order, so rotation (fp32 and bf16), rotated amax and fused codes agree
    bit for bit between an aligned copy and a copy offset by one element."""
    rng = np.random.default_rng(d + 11)
    rows = 515
    x = (rng.standard_normal((rows, d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
    n = rows * d
    st = torch.cuda.current_stream().cuda_stream
    for esz, dt in ((4, torch.float32), (2, torch.bfloat16)):
        a_in = torch.from_numpy(x.reshape(-1)).to(DEV).to(dt)
        src = torch.zeros((n + 8,), dtype=dt, device=DEV)
        src[1:n + 1] = a_in
        u_in = src[1:n + 1]
        a_out = torch.empty((n,), dtype=dt, device=DEV)
        u_buf = torch.empty((n + 8,), dtype=dt, device=DEV)
        fn = pkg.attn_hadamard_f32 if esz == 4 else pkg.attn_hadamard_bf16
        assert fn(a_in.data_ptr(), rows, d, a_out.data_ptr(), st) == 0
        assert fn(u_in.data_ptr(), rows, d, u_buf.data_ptr() + esz, st) == 0
        torch.cuda.synchronize()
        assert torch.equal(a_out.view(torch.int16 if esz == 2 else torch.int32),
                           u_buf[1:n + 1].view(torch.int16 if esz == 2 else torch.int32)), esz
        if esz == 4:
            ref = oracle.hadamard(x).reshape(-1)
            assert np.abs(a_out.cpu().numpy() - ref).max() <= 1e-6 * np.abs(ref).max()
            am = torch.empty((2,), dtype=torch.float32, device=DEV)
            assert pkg.attn_hadamard_amax_f32(a_in.data_ptr(), rows, d, am.data_ptr(), st) == 0
            assert pkg.attn_hadamard_amax_f32(u_in.data_ptr(), rows, d, am.data_ptr() + 4, st) == 0
            ca = torch.empty((n,), dtype=torch.uint8, device=DEV)
            cu = torch.empty((n + 16,), dtype=torch.uint8, device=DEV)
            assert pkg.attn_hadamard_quantize_e4m3(a_in.data_ptr(), rows, d, 0.01, ca.data_ptr(),
                                                   st) == 0
            assert pkg.attn_hadamard_quantize_e4m3(u_in.data_ptr(), rows, d, 0.01,
                                                   cu.data_ptr() + 3, st) == 0
            torch.cuda.synchronize()
            assert am[0].item() == am[1].item() == float(np.abs(a_out.cpu().numpy()).max())
            assert torch.equal(ca, cu[3:n + 3])
            assert np.array_equal(ca.cpu().numpy(), oracle.quantize_e4m3(a_out.cpu().numpy(), 0.01))


def _gpu_fp8_fused(xs, tau):
    """Rotate and quantize Q, K, V; attention with the O rotation fused into
    the kernel's epilogue (attn_fwd_ex with ATTN_FLAG_HADAMARD_O)."""
    t = [torch.from_numpy(x).to(DEV) for x in xs]
    codes, ds = zip(*[pkg.quantize_fp8(x, rotate=True) for x in t])
    o, lse = pkg.flash_attn_func(*codes, softmax_scale=tau, causal=True, q_descale=ds[0],
                                 k_descale=ds[1], v_descale=ds[2], hadamard_o=True)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d_qk", [128, 192])
def test_fused_o_rotation_matches_oracle(oracle, d_qk):
    S, H = 700, 2
    tau = 1.0 / np.sqrt(d_qk)
    xs = _inputs(S, H, d_qk, 4, 4242 + d_qk, shared=False, scale=5.0)
    go, gl = _gpu_fp8_fused(xs, tau)
    ro, rl, st = _oracle_fp8(oracle, xs, True, tau)
    judge("fused O rotation d%d" % d_qk, synth.FP8, go, gl, ro, rl, st)
    # against the separate bf16 pass over O: the fused path rounds once, the
    # separate one twice, so they agree to a few bf16 units
    so, sl = _gpu_fp8(xs, True, tau)
    assert np.array_equal(sl, gl)
    assert float(np.linalg.norm(so - go) / np.linalg.norm(go)) <= 8e-3


def test_fused_o_rotation_of_constant_values_is_the_hadamard_row(oracle):
    """Every V row equal to u makes O = u in every row (the softmax weights sum
    to one), so the fused output must be u.H for every query row and head:
    this fixes the rotation's element order and signs."""
    rng = np.random.default_rng(77)
    S, H, d = 300, 2, 128
    q = rng.standard_normal((1, S, H, d)).astype(np.float32)
    k = rng.standard_normal((1, S, H, d)).astype(np.float32)
    u = rng.standard_normal(128).astype(np.float32)
    v = np.broadcast_to(u, (1, S, H, 128)).copy()
    dq, dk, dv = (oracle.descale_amax(x) for x in (q, k, v))
    enc = [oracle.quantize_e4m3(x, dd) for x, dd in zip((q, k, v), (dq, dk, dv))]
    dev = [u8_to_device(x) for x in enc]
    o, _ = pkg.flash_attn_func(*dev, softmax_scale=0.1, causal=True, q_descale=dq, k_descale=dk,
                               v_descale=dv, hadamard_o=True)
    torch.cuda.synchronize()
    go = o_to_f64(o)
    uh = oracle.hadamard(oracle.decode_e4m3(enc[2][0, 0, 0]) * dv)
    err = np.abs(go - uh).max() / np.abs(uh).max()
    print("constant-V rotation max error %.3e" % err)
    # the e4m3 rounding of P cancels in sum(p u) / sum(p): what is left is the
    # bf16 rounding of O, at most 2^-8 of the largest element
    assert err <= 5e-3


def test_fwd_ex_without_flags_equals_fwd_bitwise(oracle):
    rng = np.random.default_rng(5)
    xs = [rng.standard_normal((1, 400, 2, 128)).astype(np.float32) for _ in range(3)]
    ds = [oracle.descale_amax(x) for x in xs]
    dev = [u8_to_device(oracle.quantize_e4m3(x, dd)) for x, dd in zip(xs, ds)]
    outs = []
    for ex in (False, True):
        o = torch.empty((1, 400, 2, 128), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((1, 2, 400), dtype=torch.float32, device=DEV)
        args = [t.data_ptr() for t in dev] + [o.data_ptr(), lse.data_ptr(), 1, 400, 2, 128, 128,
                                              0.09, 1, 1, ds[0], ds[1], ds[2]]
        st = pkg.attn_fwd_ex(*args, 0) if ex else pkg.attn_fwd(*args)
        assert st == 0
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).clone(), lse.view(torch.int32).clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
