"""GPU parity at sequence lengths around the 64-key tile and the 32-row wave
and 256-row workgroup boundaries, for both element types and head shapes,
causal and not (through the C ABI).

Each wave runs a straight-line form of its key loop while the next tile is
fully visible to all of its rows and a general form for the last, masked
tiles; the switch point depends on the wave's first row and the length, and
an odd number of straight-line iterations ends with a copy of the carried
scores.  These lengths put the switch on both parities, at the first tile,
and past a ragged tail.
"""
import pytest

from causal_prefill_attention_attn_amd import synth

from gpu_util import check, make_inputs, run_gpu

pytestmark = pytest.mark.gpu

LENGTHS = [63, 64, 65, 96, 191, 192, 193, 255, 256, 257, 320, 449, 511, 513]
SHAPES = [(synth.FP8, 128), (synth.FP8, 192), (synth.BF16, 128), (synth.BF16, 192)]


@pytest.mark.parametrize("dtype,d_qk", SHAPES)
@pytest.mark.parametrize("S", LENGTHS)
def test_causal_tile_edges(oracle, dtype, d_qk, S):
    w = synth.Workload("edge_%d_%d_%d" % (dtype, d_qk, S), 80 + S % 17, dtype, 1, 2, S, d_qk, 128,
                       "gaussian", "tile edges")
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse)


@pytest.mark.parametrize("dtype,d_qk", SHAPES)
@pytest.mark.parametrize("S", [64, 65, 257, 513])
def test_non_causal_tile_edges(oracle, dtype, d_qk, S):
    w = synth.Workload("edge_nc_%d_%d_%d" % (dtype, d_qk, S), 90 + S % 13, dtype, 1, 2, S, d_qk,
                       128, "gaussian", "tile edges, non-causal")
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds, causal=False)
    check(oracle, w, enc, ds, o, lse, causal=False)


@pytest.mark.parametrize("dtype,d_qk", [(synth.FP8, 128), (synth.BF16, 128)])
def test_llm_like_tile_edges(oracle, dtype, d_qk):
    """Near-one-hot rows (the running maximum jumps often and by a lot)."""
    w = synth.Workload("edge_llm_%d" % dtype, 97, dtype, 1, 2, 577, d_qk, 128, "llm",
                       "tile edges, LLM-like")
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse)
