"""GPU parity when the running row maximum keeps growing (through the C ABI).

Keys are built so that every query's scores rise steadily with the key
index: the maximum of each row moves at almost every tile.  The FP8 kernel
refreshes the maximum (and rescales O and the row sum) on every increase;
the BF16 kernel only when it has grown by more than 8 octaves, so here it
runs stretches of tiles with probabilities above 1 and then refreshes.  Both
must still match the oracle, including the log-sum-exp.
"""
import numpy as np
import pytest

from causal_prefill_attention_attn_amd import synth

from gpu_util import check, make_inputs, run_gpu

pytestmark = pytest.mark.gpu


def _rising(w, octaves_per_key):
    """Seeded inputs whose score of key j for any query grows by about
    `octaves_per_key` per key: channel 0 of every query is a constant and
    channel 0 of key j grows linearly with j; the other channels are small
    N(0,1) noise."""
    qf, kf, vf = synth.generate(w)
    qf *= 0.05
    kf *= 0.05
    qf[..., 0] = 4.0
    step = octaves_per_key / (4.0 * w.softmax_scale * np.log2(np.e))
    kf[..., 0] = (np.arange(w.S, dtype=np.float32) * step)[None, :, None]
    return qf, kf, vf


@pytest.mark.parametrize("dtype,d_qk,rate", [(synth.BF16, 128, 0.05), (synth.BF16, 128, 0.4),
                                             (synth.BF16, 192, 0.2), (synth.FP8, 128, 0.05),
                                             (synth.FP8, 128, 0.4), (synth.FP8, 192, 0.2)])
def test_rising_scores(oracle, dtype, d_qk, rate):
    w = synth.Workload("rising_%d_%d_%g" % (dtype, d_qk, rate), 98, dtype, 1, 2, 700, d_qk, 128,
                       "gaussian", "rising scores")
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w, _rising(w, rate))
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse)
