"""Partial attention over key subsets merged through the returned LSE.

The sequence-parallel split of the kernel (each GPU holds a slice of the
queries and sees the earlier keys in pieces) needs only the identity

    o = sum_r exp(lse_r) o_r / sum_r exp(lse_r),   lse = log sum_r exp(lse_r)

for attention of the same queries over disjoint key sets r.  One GPU can show
it: the queries of the second half of a sequence attend to the first half
without a mask and to their own half with the causal mask, in two launches,
and the merge of the two results must equal the causal attention of those
rows over the whole sequence (the oracle).  The merge runs in fp64 on the
host, as a caller combining shards would.
"""
import numpy as np
import pytest

from causal_prefill_attention_attn_amd import synth
from gpu_util import bf16_to_device, judge, o_to_f64, run_gpu, u8_to_device
from merge_util import merge

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d_qk", [(synth.BF16, 128), (synth.FP8, 128), (synth.FP8, 192)])
def test_two_key_halves_merge_to_causal_attention(oracle, dtype, d_qk):
    N, H = 320, 2                          # half length (ragged against the tiles)
    w = synth.Workload("merge", 91, dtype, 1, H, 2 * N, d_qk, 128, "gaussian", "merge")
    qf, kf, vf = synth.generate(w)
    if dtype == synth.BF16:
        enc = [synth.to_bf16_bits(x) for x in (qf, kf, vf)]
        ds = [1.0, 1.0, 1.0]
        up = bf16_to_device
    else:
        ds = [oracle.descale_amax(x) for x in (qf, kf, vf)]
        enc = [oracle.quantize_e4m3(x, d) for x, d in zip((qf, kf, vf), ds)]
        up = u8_to_device
    q, k, v = enc
    q2 = np.ascontiguousarray(q[:, N:])
    shard = w.with_shape(S=N)
    # keys 0..N-1: every query of the second half sees all of them
    o_a, l_a = run_gpu([up(q2), up(np.ascontiguousarray(k[:, :N])),
                        up(np.ascontiguousarray(v[:, :N]))], shard, ds, causal=False)
    # keys N..2N-1: the causal mask of the half is the global one shifted by N
    o_b, l_b = run_gpu([up(q2), up(np.ascontiguousarray(k[:, N:])),
                        up(np.ascontiguousarray(v[:, N:]))], shard, ds, causal=True)
    parts = [(o_to_f64(o_a), l_a.cpu().numpy().astype(np.float64)),
             (o_to_f64(o_b), l_b.cpu().numpy().astype(np.float64))]
    go, gl = merge(parts)
    rows = np.arange(N, 2 * N)
    ro, rl, st = oracle.attention(q, k, v, dtype, w.softmax_scale, True, rows=rows,
                                  q_descale=ds[0], k_descale=ds[1], v_descale=ds[2], stats=True)
    # each half encodes its own maximum exactly, not necessarily the row's
    judge("merge d%d" % d_qk, dtype, go, gl, ro, rl, st, top_exact=False)
