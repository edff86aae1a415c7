"""The library's GPU amax and E4M3FN quantizer are bit-exact with the
oracle's codec (integer/byte results: exact equality)."""
import numpy as np
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg

from gpu_util import DEV

pytestmark = pytest.mark.gpu


def _special_values(oracle):
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode_e4m3(codes)
    vals = vals[np.isfinite(vals)]
    pos = np.unique(np.abs(vals))
    mids = (pos[1:] + pos[:-1]) / 2
    extra = np.array([448.0, 449.0, 463.9, 464.0, 464.1, 479.0, 480.0, 1e4, 3e38, np.inf,
                      2.0 ** -10, 2.0 ** -11, 1e-30, 1e-45, 0.0])
    base = np.concatenate([pos, mids, extra]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(0))
    allv = np.concatenate([base, up, dn])
    return np.concatenate([allv, -allv]).astype(np.float32)


def test_quantize_special_values_bit_exact(oracle):
    x = _special_values(oracle)
    for descale in (1.0, 0.25, 3.0, 0.0123):
        ref = oracle.quantize_e4m3(x, descale)
        tx = torch.from_numpy(x).to(DEV)
        out = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
        assert pkg.attn_quantize_e4m3(tx.data_ptr(), x.size, descale, out.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, [(float(x[i]), descale, hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_quantize_nan_maps_to_0x7f(oracle):
    x = np.array([np.nan, -np.nan], np.float32)
    tx = torch.from_numpy(x).to(DEV)
    out = torch.empty((2,), dtype=torch.uint8, device=DEV)
    assert pkg.attn_quantize_e4m3(tx.data_ptr(), 2, 1.0, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert list(out.cpu().numpy()) == [0x7F, 0x7F] == list(oracle.quantize_e4m3(x, 1.0))


@pytest.mark.parametrize("recipe_scale", [1.0, 37.5, 1e-3])
def test_quantize_fp8_random_tensor(oracle, recipe_scale):
    rng = np.random.default_rng(99)
    x = (rng.standard_normal(3_000_001) * recipe_scale).astype(np.float32)
    x[12345] = -7.5 * recipe_scale * 10
    codes, descale = pkg.quantize_fp8(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    assert np.float32(descale) == np.float32(oracle.descale_amax(x))
    assert np.array_equal(codes.cpu().numpy(), oracle.quantize_e4m3(x, oracle.descale_amax(x)))


def test_amax_zero_and_nan(oracle):
    x = np.zeros(1000, np.float32)
    codes, descale = pkg.quantize_fp8(torch.from_numpy(x).to(DEV))
    assert descale == 1.0 and int(codes.sum()) == 0
    x[17] = np.nan
    x[500] = -3.0
    out = torch.empty((1,), dtype=torch.float32, device=DEV)
    tx = torch.from_numpy(x).to(DEV)
    assert pkg.attn_amax_f32(tx.data_ptr(), x.size, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert float(out.item()) == 3.0


@pytest.mark.parametrize("rotate,d", [(0, 100), (0, 128), (1, 128), (1, 192)])
def test_quantize_fp8_entry_point(oracle, rotate, d):
    """attn_quantize_fp8 runs the whole quantization on the device: its
    descale is the oracle's amax/448 of the (rotated) tensor and its codes are
    the oracle's encoding with that descale, bit for bit."""
    rng = np.random.default_rng(123 + d + rotate)
    x = (rng.standard_normal((777, d)) * np.exp(rng.standard_normal(d))).astype(np.float32)
    tx = torch.from_numpy(x).to(DEV)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    ds = torch.empty((1,), dtype=torch.float32, device=DEV)
    assert pkg.attn_quantize_fp8(tx.data_ptr(), 777, d, rotate, codes.data_ptr(), ds.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    if rotate:
        # the library rotates in fp32; take its rotated tensor as the input of
        # the oracle's codec (the rotation itself is checked against the oracle
        # in the Hadamard tests)
        xr = pkg.hadamard(tx).cpu().numpy()
    else:
        xr = x
    ref_ds = oracle.descale_amax(xr)
    assert np.float32(ds.item()) == np.float32(ref_ds)
    assert np.array_equal(codes.cpu().numpy(), oracle.quantize_e4m3(xr, ref_ds))


def test_quantize_fp8_all_zero():
    x = torch.zeros((64, 128), dtype=torch.float32, device=DEV)
    codes, descale = pkg.quantize_fp8(x)
    assert descale == 1.0 and int(codes.sum()) == 0
    codes, descale = pkg.quantize_fp8(x, rotate=True)
    assert descale == 1.0 and int(codes.sum()) == 0


@pytest.mark.parametrize("x_off,o_off", [(0, 0), (1, 0), (0, 3), (2, 5)])
def test_quantize_and_amax_alignment_and_tails(oracle, x_off, o_off):
    """Aligned buffers take vector paths (whole runs of 1024 values a wave at
    a time, then groups of 16 values per thread) and the rest a scalar loop;
    every length from 1 to 70, lengths around whole runs, and both
    alignments give the oracle's codes and amax exactly; length 0 is
    refused."""
    rng = np.random.default_rng(7 + x_off + 10 * o_off)
    base = (rng.standard_normal(6000) * 40).astype(np.float32)
    tb = torch.from_numpy(base).to(DEV)
    ob = torch.empty((6000,), dtype=torch.uint8, device=DEV)
    amax = torch.empty((1,), dtype=torch.float32, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    assert pkg.attn_quantize_e4m3(tb.data_ptr(), 0, 1.0, ob.data_ptr(), st) != 0
    assert pkg.attn_amax_f32(tb.data_ptr(), 0, amax.data_ptr(), st) != 0
    for n in list(range(1, 71)) + [1008, 1023, 1024, 1025, 1040, 2047, 2048 + 16 + 3, 5003]:
        x = base[x_off:x_off + n]
        ob.fill_(0xAA)
        assert pkg.attn_quantize_e4m3(tb.data_ptr() + 4 * x_off, n, 0.37, ob.data_ptr() + o_off,
                                      st) == 0
        assert pkg.attn_amax_f32(tb.data_ptr() + 4 * x_off, n, amax.data_ptr(), st) == 0
        torch.cuda.synchronize()
        got = ob.cpu().numpy()
        assert np.array_equal(got[o_off:o_off + n], oracle.quantize_e4m3(x, 0.37)), n
        assert np.all(got[:o_off] == 0xAA) and np.all(got[o_off + n:] == 0xAA), n
        assert float(amax.item()) == float(np.abs(x).max()), n
