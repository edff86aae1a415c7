"""Packed variable-length sequences (attn_fwd_varlen) against the oracle run
on each sequence alone, and against the dense entry point when all lengths
are equal.  Variable-length batches are listed among the kernels' future
work in "Ce que couvrent les noyaux" on the ai-daily-news.org page; the
oracle of a packed batch is independent attention per sequence."""
import numpy as np
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg
from causal_prefill_attention_attn_amd import synth
from gpu_util import DEV, TOL, bf16_to_device, judge, u8_to_device

pytestmark = pytest.mark.gpu


def _packed(oracle, dtype, total, H, d_qk, seed):
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal((total, H, d)).astype(np.float32) for d in (d_qk, d_qk, 128)]
    if dtype == synth.BF16:
        enc = [synth.to_bf16_bits(x) for x in xs]
        return enc, [1.0, 1.0, 1.0], [bf16_to_device(x) for x in enc]
    ds = [oracle.descale_amax(x) for x in xs]
    enc = [oracle.quantize_e4m3(x, d) for x, d in zip(xs, ds)]
    return enc, ds, [u8_to_device(x) for x in enc]


@pytest.mark.parametrize("dtype,d_qk,causal", [(synth.BF16, 128, True), (synth.FP8, 128, True),
                                               (synth.FP8, 192, True), (synth.BF16, 128, False)])
def test_varlen_matches_per_sequence_oracle(oracle, dtype, d_qk, causal):
    lens = [1, 63, 64, 0, 65, 257, 700, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total, H = int(cu[-1]), 2
    tau = 1.0 / np.sqrt(d_qk)
    enc, ds, dev = _packed(oracle, dtype, total, H, d_qk, 31 + d_qk + dtype)
    o, lse = pkg.flash_attn_varlen_func(*dev, torch.from_numpy(cu).to(DEV), max(lens),
                                        softmax_scale=tau, causal=causal, q_descale=ds[0],
                                        k_descale=ds[1], v_descale=ds[2])
    torch.cuda.synchronize()
    go = o.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    for s, n in enumerate(lens):
        if n == 0:
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        seq = [np.ascontiguousarray(x[a:b][None]) for x in enc]
        ro, rl, st = oracle.attention(*seq, dtype, tau, causal, q_descale=ds[0],
                                      k_descale=ds[1], v_descale=ds[2], stats=True)
        judge("seq %d len %d" % (s, n), dtype, go[a:b][None], gl[None, :, a:b], ro, rl, st)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP8])
def test_equal_lengths_equal_dense_bitwise(oracle, dtype):
    B, L, H = 3, 333, 2
    enc, ds, dev = _packed(oracle, dtype, B * L, H, 128, 77 + dtype)
    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device=DEV)
    ov, lv = pkg.flash_attn_varlen_func(*dev, cu, L, q_descale=ds[0], k_descale=ds[1],
                                        v_descale=ds[2])
    dense = [x.view(B, L, H, x.shape[-1]) for x in dev]
    od, ld = pkg.flash_attn_func(*dense, q_descale=ds[0], k_descale=ds[1], v_descale=ds[2])
    torch.cuda.synchronize()
    assert torch.equal(ov.view(B, L, H, 128).view(torch.int16), od.view(torch.int16))
    # lse: varlen [H, B*L], dense [B, H, L]
    assert torch.equal(lv.view(H, B, L).permute(1, 0, 2).contiguous().view(torch.int32),
                       ld.view(torch.int32))


def test_malformed_offsets_are_clamped(oracle):
    """cu_seqlens entries outside [0, total] or decreasing are clamped by the
    kernels (documented: results unspecified, accesses in bounds): the call
    returns and the well-formed sequences are still exact."""
    lens = [100, 50, 200]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total, H = int(cu[-1]), 2
    enc, ds, dev = _packed(oracle, synth.BF16, total, H, 128, 404)
    bad = cu.copy()
    bad[2] = 10 ** 6       # sequence 1 ends past total, sequence 2 starts past it
    o, lse = pkg.flash_attn_varlen_func(*dev, torch.from_numpy(bad).to(DEV), 200)
    torch.cuda.synchronize()
    go = o.float().cpu().numpy().astype(np.float64)
    # sequence 0 is untouched by the bad entry
    seq = [np.ascontiguousarray(x[0:100][None]) for x in enc]
    ro, rl, st = oracle.attention(*seq, synth.BF16, 1.0 / np.sqrt(128), True, stats=True)
    judge("seq 0 beside clamped offsets", synth.BF16, go[0:100][None], None, ro, rl, st)
