"""Dense batches (B > 1) against the oracle: every batch entry has its own
data, so a wrong batch offset in q/k/v, o or the LSE shows as a mismatch in
the entries after the first."""
import dataclasses

import numpy as np
import pytest

from causal_prefill_attention_attn_amd import synth
from gpu_util import check, make_inputs, run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d_qk", [(synth.BF16, 128), (synth.FP8, 128), (synth.FP8, 192),
                                        (synth.BF16, 192)])
def test_dense_batch_matches_oracle(oracle, dtype, d_qk):
    base = synth.WORKLOADS["C2" if dtype == synth.BF16 else ("C5" if d_qk == 192 else "C3")]
    w = dataclasses.replace(base, B=3, H=2, S=300, d_qk=d_qk)
    print("case %s B=3 H=2 S=300 d_qk=%d" % (base.name, d_qk), flush=True)
    rng = np.random.default_rng(600 + d_qk + dtype)
    qkv = tuple(rng.standard_normal((3, 300, 2, d)).astype(np.float32)
                for d in (d_qk, d_qk, 128))
    enc, ds, dev = make_inputs(oracle, w, qkv)
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse)
