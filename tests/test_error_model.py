"""CPU pins of the constants of the FP8 error model the GPU parity tests use
(tests/gpu_util.py): the largest relative error of one encoded probability,
for the lean code and for round-to-nearest exp2 values, computed here from
the oracle's E4M3FN codec over the e4m3 normal range.

The lean code (the "one multiply-add and one integer conversion" probability
of "Como o motor de atencao FP8 da Zyphra funciona" on the miraibroadcast.com
page, as the FP8 kernel reads it): the e4m3 bit pattern of 2^y is the
integer round-half-even(8 (y + 7) - 0.4567); the exponent field takes the
integer part of y and the mantissa 8 frac(y), i.e. 2^f is replaced by 1 + f,
with a shift that centres the ratio on 1.  The kernel reaches that integer
through a 16-bit normalised conversion (round to nearest, clamp to [0, 1]) of
(256 z + 127.5) / 65535 computed in binary32, z = 8 (y + 7) - 0.4567, and
keeps the high byte; the test checks that this gives the same codes.  Exact
P: exp2(y) rounded to nearest even in e4m3.
"""
import numpy as np

from gpu_util_cpu import EPS_P, FLUSH

Y = np.linspace(-6.0, 8.0, 1_400_001)   # the e4m3 normal range of 2^y: [2^-6, 2^8]


def test_lean_code_relative_error(oracle):
    codes = np.rint(8.0 * (Y + 7.0) - 0.4567)
    assert codes.min() >= 8 and codes.max() <= 120          # normal codes 2^-6 .. 2^8
    ratio = oracle.decode_e4m3(codes.astype(np.uint8)) / 2.0 ** Y
    worst = float(np.abs(ratio - 1.0).max())
    print("lean code: ratio %.5f .. %.5f, mean %.5f" % (ratio.min(), ratio.max(), ratio.mean()))
    assert worst <= EPS_P["lean"] and worst >= 0.99 * EPS_P["lean"]
    assert abs(ratio.mean() - 1.0) < 1e-3                     # unbiased on average
    # the high byte of the 16-bit normalised conversion gives the same codes
    z = 8.0 * (Y + 7.0) - 0.4567
    x = ((256.0 * z + 127.5) / 65535.0).astype(np.float32)
    u16 = np.rint(np.clip(x.astype(np.float64), 0.0, 1.0) * 65535.0)
    assert np.array_equal(np.floor(u16 / 256.0), codes)
    # y = 8 (a block maximum at the row maximum) is encoded exactly
    assert oracle.decode_e4m3(np.array([round(8 * 15 - 0.4567)], np.uint8))[0] == 256.0


def test_exact_rounding_relative_error(oracle):
    x = (2.0 ** Y).astype(np.float32)
    ratio = oracle.decode_e4m3(oracle.quantize_e4m3(x, 1.0)) / x.astype(np.float64)
    worst = float(np.abs(ratio - 1.0).max())
    # half a unit of 2^-3 at a significand of 1 + 2^-4: (2^-4) / (1 + 2^-4) = 1/17
    assert worst <= EPS_P["exact"] and worst >= 0.99 * EPS_P["exact"]


def test_flush_share():
    # a block's maximum probability is scaled into (2^7, 2^8]; values below the
    # normal range (2^-6) are under 2^-13 of it, and a block has 64 keys
    assert FLUSH == 64 * 2.0 ** -6 / 2.0 ** 7
