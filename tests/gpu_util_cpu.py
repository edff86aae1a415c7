"""Constants of the error model of the GPU parity tests (see gpu_util.py),
importable without a GPU so that CPU tests can pin them."""
from causal_prefill_attention_attn_amd import synth

TOL = {synth.BF16: 1e-2, synth.FP8: 5e-2}
EPS_P = {"lean": 0.0796, "exact": 1.0 / 17.0}   # largest relative error of one encoded probability
GAMMA8 = 7 * 2.0 ** -13                         # FP8 score error per unit of tau * sum_c |q_c k_c|
FLUSH = 2.0 ** -7                               # share of a row below a block's e4m3 normal range
