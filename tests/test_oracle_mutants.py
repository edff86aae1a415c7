"""Planted mistakes in the oracle are caught by its pins.

Each case copies the oracle (its C source and its Python module) into a
temporary directory and plants one plausible mistake in the copy:
- a dropped term or scale, a wrong sign or base;
- an off-by-one or ignored causal mask;
- a transposed or wrong index;
- a wrong constant of the E4M3 or bf16 codecs, or a wrong rounding rule;
- a descale left out;
- a wrong statistic;
- a wrong Hadamard matrix;
- a wrong page, slot or head mapping in the paged decode.
The copy is built and imported on its own, and the pins of
test_oracle_pins.py, test_codec.py, test_oracle_stats_pins.py and
test_oracle_decode_pins.py run against it. At least one pin must fail for
every mistake. The unmodified copy must pass all of them, so a failure
means the pins noticed the mistake, not that the battery is broken. The real
oracle is never touched.
"""
import importlib.util
import itertools
import os
import shutil

import pytest

import test_codec as C
import test_oracle_decode_pins as D
import test_oracle_pins as P
import test_oracle_stats_pins as ST

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")
BF16, FP8 = 0, 1

# every pin, with one parameter set each where the pin is parametrized
BATTERY = [
    ("P1 brute force, causal", lambda o: P.test_p1_bruteforce_mpmath(o, 2, 2, 8, 4, 2, True)),
    ("P1 brute force, full", lambda o: P.test_p1_bruteforce_mpmath(o, 1, 1, 5, 8, 8, False)),
    ("torch SDPA bf16", lambda o: P.test_matches_torch_sdpa_fp64(o, "bf16", 1, 2, 64, 192, 128, True)),
    ("torch SDPA fp8", lambda o: P.test_matches_torch_sdpa_fp64(o, "fp8", 2, 3, 37, 128, 128, True)),
    ("torch SDPA fp8, full", lambda o: P.test_matches_torch_sdpa_fp64(o, "fp8", 1, 1, 130, 16, 8, False)),
    ("P2 weights and mask", P.test_p2_weights_rows_sum_to_one_and_mask),
    ("P3 query 0", P.test_p3_query_zero_returns_v0),
    ("P4 uniform scores", lambda o: P.test_p4_uniform_scores_prefix_mean(o, "q_zero")),
    ("P5 two tokens", P.test_p5_two_tokens_closed_form),
    ("P6 one-hot limit", P.test_p6_one_hot_limit),
    ("P7 key shift", P.test_p7_key_shift_invariance),
    ("P8 linearity", P.test_p8_linearity_in_v),
    ("P8 permutation", P.test_p8_head_and_batch_permutation),
    ("P8 causal vs full", P.test_p8_causal_vs_noncausal),
    ("row subset", P.test_row_subset_matches_full),
    ("fp8 descales", P.test_fp8_descales_are_applied),
    ("lse merge", P.test_lse_merge_of_key_halves_is_causal_attention),
    ("hadamard by hand", P.test_hadamard_matrix_small_orders_by_hand),
    ("hadamard orthogonal", lambda o: P.test_hadamard_matrix_orthogonal_symmetric_pm_entries(o, 64)),
    ("hadamard rows d192", lambda o: P.test_hadamard_rows_are_isometric_and_self_inverse(o, 192)),
    ("hadamard outlier", P.test_hadamard_spreads_an_outlier_channel),
    ("e4m3 decode vs torch", C.test_decode_all_codes_match_torch),
    ("e4m3 decode table", C.test_decode_table_spot_values),
    ("e4m3 round trip", C.test_encode_roundtrip_all_finite_codes),
    ("e4m3 ties and saturation", C.test_encode_midpoints_tie_to_even_and_saturate),
    ("e4m3 encode vs torch", C.test_encode_matches_torch_cast_on_random_values),
    ("quantizer", C.test_quantizer_descale_and_division),
    ("bf16 decode", C.test_bf16_decode_matches_torch),
    ("stats: query 0", ST.test_query_zero_and_constant_v),
    ("stats: two keys", ST.test_two_keys_closed_form),
    ("stats: kappa", ST.test_kappa_is_the_first_order_error_gain),
    ("stats: wmax", ST.test_wmax_with_ties_and_uniform_scores),
    ("stats: sabs", ST.test_sabs_counts_magnitudes_not_the_cancelled_score),
    ("stats: fp8", ST.test_fp8_stats_use_descales),
    ("decode vs SDPA", lambda o: D.test_decode_matches_torch_sdpa_on_unpaged_keys(o, 8, 2, 128, 64)),
    ("decode = last prefill row, bf16", lambda o: D.test_decode_is_last_row_of_causal_prefill(o, BF16)),
    ("decode = last prefill row, fp8", lambda o: D.test_decode_is_last_row_of_causal_prefill(o, FP8)),
    ("decode brute force", D.test_decode_brute_force_40_digits_with_groups),
    ("decode one key, empty", D.test_decode_single_key_and_empty_sequence),
    ("decode head mapping", D.test_decode_query_head_to_kv_head_mapping),
    ("decode fp8 descales", D.test_decode_fp8_descales),
]

# (name, file, old text, new text, number of occurrences of old, all of
# which are replaced).  Every mistake keeps memory accesses in bounds.
MUTANTS = [
    ("mask drops the diagonal", "c", "const int64_t nvis = causal ? i + 1 : S;",
     "const int64_t nvis = causal ? i : S;", 1),
    ("mask lets one future key through", "c", "const int64_t nvis = causal ? i + 1 : S;",
     "const int64_t nvis = causal ? (i + 2 < S ? i + 2 : S) : S;", 1),
    ("causal flag ignored", "c", "const int64_t nvis = causal ? i + 1 : S;",
     "const int64_t nvis = i + 1;", 1),
    ("softmax scale dropped", "c", "s[j] = tau * dot;", "s[j] = dot;", 1),
    ("max subtracted with the wrong sign", "c", "const double p = exp(s[j] - m);",
     "const double p = exp(m - s[j]);", 1),
    ("no division by the row sum", "c", "orow[c] = acc[c] / l;", "orow[c] = acc[c];", 1),
    ("lse without the max", "c", "lse[srow] = m + log(l);", "lse[srow] = log(l);", 1),
    ("lse in base 2", "c", "lse[srow] = m + log(l);", "lse[srow] = m + log2(l);", 1),
    ("query row read with head and position transposed", "c",
     "qi[c] = elem(q, ((b * S + i) * H + h) * d_qk + c, dtype, dq);",
     "qi[c] = elem(q, ((b * H + h) * S + i) * d_qk + c, dtype, dq);", 1),
    ("value row of the query instead of the key", "c",
     "const int64_t vb = ((b * S + j) * H + h) * d_v;\n        for (int64_t c = 0; c < d_v; ++c) acc[c]",
     "const int64_t vb = ((b * S + i) * H + h) * d_v;\n        for (int64_t c = 0; c < d_v; ++c) acc[c]", 1),
    ("k descale left out", "c", "dot += qi[c] * elem(k, kb + c, dtype, dk);",
     "dot += qi[c] * elem(k, kb + c, dtype, 1.0);", 1),
    ("v descale left out", "c", "acc[c] += p * elem(v, vb + c, dtype, dv);",
     "acc[c] += p * elem(v, vb + c, dtype, 1.0);", 1),
    ("q descale used for k", "c", "dot += qi[c] * elem(k, kb + c, dtype, dk);",
     "dot += qi[c] * elem(k, kb + c, dtype, dq);", 1),
    ("e4m3 exponent bias 8", "c", "v = ldexp(1.0 + m / 8.0, e - 7);",
     "v = ldexp(1.0 + m / 8.0, e - 8);", 1),
    ("e4m3 subnormal step 2^-10", "c", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);", 1),
    ("e4m3 NaN at the 448 code", "c", "if (e == 0xF && m == 0x7) return NAN;",
     "if (e == 0xF && m >= 0x6) return NAN;", 1),
    ("e4m3 ties rounded away from zero", "c",
     "if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;",
     "if (frac >= 0.5) r += 1.0;", 1),
    ("e4m3 overflow to NaN", "c", "if (a >= 448.0) return sign | 0x7E;",
     "if (a >= 448.0) return sign | 0x7F;", 1),
    ("e4m3 subnormal range one binade too deep", "c", "if (unb < -6) unb = -6;",
     "if (unb < -7) unb = -7;", 1),
    ("descale from the e4m3fnuz maximum 240", "c", "return amax / 448.0f;",
     "return amax / 240.0f;", 1),
    ("quantizer multiplies by the descale", "c", "float t = x[i] / descale;",
     "float t = x[i] * descale;", 1),
    ("bf16 widened by a 15-bit shift", "c", "uint32_t u = (uint32_t)bits << 16;",
     "uint32_t u = (uint32_t)bits << 15;", 1),
    ("kappa with unsquared weights", "c", "num += w * w * dist;", "num += w * dist;", 1),
    ("wmax counts only the last key", "c", "at_max += s[j] == m;", "at_max = s[j] == m;", 1),
    ("sabs of signed terms", "c", "a += fabs(qi[c] * elem(k, kb + c, dtype, dk));",
     "a += qi[c] * elem(k, kb + c, dtype, dk);", 1),
    ("hadamard scaled by 1/n", "py", "return h / np.sqrt(n)", "return h / n", 1),
    ("hadamard with the sign in the wrong block", "py", "h = np.block([[h, h], [h, -h]])",
     "h = np.block([[h, h], [-h, h]])", 1),
    ("hadamard blocks of 32 at d = 192", "py", "return {128: 128, 192: 64}[d]",
     "return {128: 128, 192: 32}[d]", 1),
    ("decode slot off by one", "py", "kb = dec(k_cache[page, j % ps]) * k_descale",
     "kb = dec(k_cache[page, (j + 1) % ps]) * k_descale", 1),
    ("decode heads interleaved instead of grouped", "py", "h // group", "h % hkv", 2),
    ("decode lse without the max", "py", "lse[b, h] = m + np.log(e.sum())",
     "lse[b, h] = np.log(e.sum())", 1),
    ("decode softmax scale dropped", "py", "s = tau * (kb[:, h // group, :] @ qf[b, h])",
     "s = (kb[:, h // group, :] @ qf[b, h])", 1),
    ("decode v scaled by the k descale", "py", "vb = dec(v_cache[page, j % ps]) * v_descale",
     "vb = dec(v_cache[page, j % ps]) * k_descale", 1),
]

_ids = itertools.count()


def _oracle_copy(tmp_path, mutant=None):
    """Import a private copy of the oracle, with one mistake planted."""
    d = tmp_path / ("oracle_copy_%d" % next(_ids))
    d.mkdir()
    files = {"c": "attn_oracle.c", "py": "__init__.py"}
    for f in files.values():
        shutil.copy(os.path.join(ORACLE_DIR, f), d / f)
    if mutant is not None:
        _, which, old, new, count = mutant
        path = d / files[which]
        text = path.read_text()
        assert text.count(old) == count, "the oracle changed; update this mutant: %r" % old
        path.write_text(text.replace(old, new))
    spec = importlib.util.spec_from_file_location(d.name, d / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build(force=True)
    assert os.path.dirname(mod._LIB) == str(d)
    return mod


def test_unmodified_copy_passes_every_pin(tmp_path):
    mod = _oracle_copy(tmp_path)
    for name, pin in BATTERY:
        pin(mod)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # some mistakes produce NaN
@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, mutant):
    mod = _oracle_copy(tmp_path, mutant)
    for name, pin in BATTERY:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 -- any failure of a pin counts
            print("%s: caught by '%s' (%s)" % (mutant[0], name, type(e).__name__))
            return
    pytest.fail("no pin notices: %s" % mutant[0])
