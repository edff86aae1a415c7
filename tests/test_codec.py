"""P9: the oracle's E4M3FN / bf16 codecs against the OCP format definition
and torch's casts (library routines), exhaustively over all codes."""
import numpy as np
import torch


def _torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_decode_all_codes_match_torch(oracle):
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3(codes)
    ref = _torch_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(mine[~nan], ref[~nan])


def test_decode_table_spot_values(oracle):
    # OCP E4M3: bias 7, 3 mantissa bits, max 448, min subnormal 2^-9
    spots = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, val in spots.items():
        assert oracle.decode_e4m3(np.array([c], np.uint8))[0] == val


def test_encode_roundtrip_all_finite_codes(oracle):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        val = oracle.decode_e4m3(np.array([c], np.uint8))[0]
        assert oracle.encode_e4m3_scalar(val) == c, hex(c)


def test_encode_midpoints_tie_to_even_and_saturate(oracle):
    pos = [c for c in range(0x7F)]
    vals = oracle.decode_e4m3(np.array(pos, np.uint8))
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (vals[a] + vals[b]) / 2
        if np.float32(mid) != mid:
            continue
        got = oracle.encode_e4m3_scalar(mid)
        assert got == (a if a % 2 == 0 else b), (hex(a), hex(b), mid)
        # just above / below the midpoint
        assert oracle.encode_e4m3_scalar(np.nextafter(np.float32(mid), np.float32(0))) == a
        assert oracle.encode_e4m3_scalar(np.nextafter(np.float32(mid), np.float32(1e9))) == b
    for big in (448.0, 449.0, 464.0, 470.0, 1e4, 3e38, float("inf")):
        assert oracle.encode_e4m3_scalar(big) == 0x7E
        assert oracle.encode_e4m3_scalar(-big) == 0xFE
    assert oracle.encode_e4m3_scalar(float("nan")) == 0x7F
    assert oracle.encode_e4m3_scalar(-0.0) == 0x80
    assert oracle.encode_e4m3_scalar(2.0 ** -10) == 0x00          # tie at half the smallest subnormal
    assert oracle.encode_e4m3_scalar(1.5 * 2.0 ** -10) == 0x01


def test_encode_matches_torch_cast_on_random_values(oracle):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 1, 10, 100)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    mine = oracle.quantize_e4m3(x, 1.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_quantizer_descale_and_division(oracle):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(10000) * 3).astype(np.float32)
    d = oracle.descale_amax(x)
    assert d == np.float32(np.abs(x).max()) / np.float32(448.0)
    codes = oracle.quantize_e4m3(x, d)
    ref = torch.from_numpy(np.clip(x / np.float32(d), -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(codes, ref.view(torch.uint8).numpy())
    assert np.abs(oracle.decode_e4m3(codes)).max() == 448.0
    assert oracle.descale_amax(np.zeros(5, np.float32)) == 1.0


def test_bf16_decode_matches_torch(oracle):
    bits = np.arange(0, 65536, 37, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
