"""attn_decode_paged against the oracle's decode step (oracle.decode_paged).

The decode kernels keep probabilities in fp32 and round only the output to
bf16, so each output row is within 2^-9 (relative rel-L2) of the exact
result plus fp32 accumulation error: the bar here is a row rel-L2 of 3e-3 for
both element types, inside the prefill tolerances (1e-2 BF16, 5e-2 FP8).
Caches are scattered over randomly ordered pages whose unused slots hold inf
(bf16) or NaN (e4m3), so a read past a sequence's end shows as a non-finite
output.  Decode and paged KV caches are listed among the kernels' future work
in "Ce que couvrent les noyaux" on the ai-daily-news.org page."""
import math

import numpy as np
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg
from causal_prefill_attention_attn_amd import synth
from decode_util import scatter
from gpu_util import DEV, bf16_to_device, u8_to_device

pytestmark = pytest.mark.gpu

ROW_TOL = 3e-3


def _inputs(oracle, dtype, lens, hq, hkv, dqk, ps, seed):
    rng = np.random.default_rng(seed)
    B, lmax = len(lens), max(max(lens), 1)
    x = [rng.standard_normal(s).astype(np.float32)
         for s in ((B, hq, dqk), (B, lmax, hkv, dqk), (B, lmax, hkv, 128))]
    if dtype == synth.BF16:
        enc, ds = [synth.to_bf16_bits(t) for t in x], [1.0, 1.0, 1.0]
    else:
        ds = [oracle.descale_amax(t) for t in x]
        enc = [oracle.quantize_e4m3(t, d) for t, d in zip(x, ds)]
    kp, vp, table = scatter(rng, enc[1], enc[2], lens, ps)
    host = (enc[0], kp, vp, table)
    up = bf16_to_device if dtype == synth.BF16 else u8_to_device
    dev = (up(enc[0]), up(kp), up(vp), torch.from_numpy(table).to(DEV),
           torch.from_numpy(np.asarray(lens, np.int32)).to(DEV))
    return host, ds, dev


def _compare(oracle, dtype, host, ds, lens, o, lse, tau):
    ro, rl = oracle.decode_paged(*host, np.asarray(lens), dtype, tau, q_descale=ds[0],
                                 k_descale=ds[1], v_descale=ds[2])
    go = o.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(go).all(), "non-finite output"
    live = np.asarray(lens) > 0
    assert (go[~live] == 0).all() and np.isneginf(gl[~live]).all(), "empty sequence"
    num = np.linalg.norm(go[live] - ro[live], axis=-1)
    den = np.linalg.norm(ro[live], axis=-1)
    worst = float((num / den).max()) if live.any() else 0.0
    lerr = float(np.abs(gl[live] - rl[live]).max()) if live.any() else 0.0
    lbound = 1e-4 + 1e-5 * float(np.abs(rl[live]).max()) if live.any() else 0.0
    msg = "worst row rel-L2 %.3e (tol %.0e), max|dlse| %.3e (tol %.1e)" % (worst, ROW_TOL, lerr,
                                                                             lbound)
    print(msg, flush=True)
    assert worst <= ROW_TOL and lerr <= lbound, msg


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP8])
# every (d_qk, G = hq / hkv) kernel instance: G = 1, 2, 4, 8 at d_qk 128 and 192
# (and larger pages: 256 and 1024 keys, a split inside one page)
@pytest.mark.parametrize("dqk,hq,hkv,ps", [(128, 2, 2, 16), (128, 4, 2, 32), (128, 8, 2, 64),
                                           (128, 16, 2, 32), (192, 2, 2, 32), (192, 4, 2, 16),
                                           (192, 16, 4, 64), (192, 8, 1, 128), (128, 4, 2, 256),
                                           (192, 8, 2, 1024)])
def test_decode_matches_oracle(oracle, dtype, dqk, hq, hkv, ps):
    lens = [0, 1, 15, 16, 17, 300, 1025, 2000]
    host, ds, dev = _inputs(oracle, dtype, lens, hq, hkv, dqk, ps, 100 + dqk + hq + ps + dtype)
    tau = 1.0 / math.sqrt(dqk)
    print("decode dtype %d d_qk %d H_q %d H_kv %d page %d lens %s" % (dtype, dqk, hq, hkv, ps,
                                                                      lens), flush=True)
    o, lse = pkg.flash_attn_decode_paged(*dev, max(lens), softmax_scale=tau, q_descale=ds[0],
                                         k_descale=ds[1], v_descale=ds[2])
    torch.cuda.synchronize()
    _compare(oracle, dtype, host, ds, lens, o, lse, tau)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP8])
def test_decode_many_splits_and_bitwise_repeat(oracle, dtype):
    """One long sequence on few heads, so the keys are cut into many splits
    (the merge order is exercised), and two calls give identical bits."""
    lens = [20000, 3]
    host, ds, dev = _inputs(oracle, dtype, lens, 4, 1, 128, 256, 7 + dtype)
    n = pkg.attn_decode_workspace_bytes(2, 4, 1, max(lens), 128)
    assert n // (2 * 4 * 129 * 4) > 30, "expected many key splits"
    o1, l1 = pkg.flash_attn_decode_paged(*dev, max(lens), q_descale=ds[0], k_descale=ds[1],
                                         v_descale=ds[2])
    o2, l2 = pkg.flash_attn_decode_paged(*dev, max(lens), q_descale=ds[0], k_descale=ds[1],
                                         v_descale=ds[2])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    _compare(oracle, dtype, host, ds, lens, o1, l1, 1.0 / math.sqrt(128))


def test_decode_large_batch_sampled(oracle):
    """8 sequences of up to 32K keys, 32 query heads on 8 key/value heads,
    FP8: every output is compared (the oracle gathers each sequence once)."""
    rng = np.random.default_rng(2025)
    lens = [int(x) for x in rng.integers(1, 32769, 8)]
    lens[0] = 32768
    host, ds, dev = _inputs(oracle, synth.FP8, lens, 32, 8, 128, 64, 55)
    o, lse = pkg.flash_attn_decode_paged(*dev, 32768, q_descale=ds[0], k_descale=ds[1],
                                         v_descale=ds[2])
    torch.cuda.synchronize()
    _compare(oracle, synth.FP8, host, ds, lens, o, lse, 1.0 / math.sqrt(128))


def test_decode_stale_lengths_are_clamped(oracle):
    """seq_lens entries beyond max_seqlen are clamped to it and negative ones
    to 0 (documented), so any contents keep the accesses in bounds."""
    lens = [64, 64]
    host, ds, dev = _inputs(oracle, synth.BF16, lens, 2, 2, 128, 16, 3)
    bad = torch.tensor([1 << 30, -5], dtype=torch.int32, device=DEV)
    o, lse = pkg.flash_attn_decode_paged(dev[0], dev[1], dev[2], dev[3], bad, 64)
    torch.cuda.synchronize()
    _compare(oracle, synth.BF16, host, ds, [64, 0], o, lse, 1.0 / math.sqrt(128))


def test_decode_out_of_range_pages_are_clamped(oracle):
    """Block-table entries outside [0, pages) are clamped into the pool
    (documented: results unspecified, accesses in bounds): the call returns,
    the output is finite, and the rows whose pages are all valid are exact."""
    lens = [40, 40]
    host, ds, dev = _inputs(oracle, synth.BF16, lens, 2, 2, 128, 16, 12)
    bad = dev[3].clone()
    bad[1, 0] = -7                  # sequence 1: first page below the pool
    bad[1, 2] = 1 << 20             # and its last page far past it
    o, lse = pkg.flash_attn_decode_paged(dev[0], dev[1], dev[2], bad, dev[4], 40)
    torch.cuda.synchronize()
    go = o.float().cpu().numpy()
    assert np.isfinite(go).all() and np.isfinite(lse.cpu().numpy()).all()
    ro, rl = oracle.decode_paged(*host, np.asarray(lens), synth.BF16, 1.0 / math.sqrt(128))
    err = np.linalg.norm(go[0] - ro[0]) / np.linalg.norm(ro[0])
    assert err <= ROW_TOL, err


@pytest.mark.parametrize("ps", [64, 16])
def test_decode_bf16_long_splits(oracle, ps):
    """bf16 caches take fewer, longer key splits (at most 4096 keys and 64
    pages): 16 sequences of up to 4096 keys on 16 key/value heads give splits
    of 2048 keys, i.e. 32 pages of 64 keys, or with pages of 16 keys the
    64-page cap of 1024 keys."""
    lens = [4096] * 15 + [3000]
    host, ds, dev = _inputs(oracle, synth.BF16, lens, 32, 16, 128, ps, 77 + ps)
    print("decode bf16 long splits, page %d" % ps, flush=True)
    o, lse = pkg.flash_attn_decode_paged(*dev, max(lens))
    torch.cuda.synchronize()
    _compare(oracle, synth.BF16, host, ds, lens, o, lse, 1.0 / math.sqrt(128))


def test_decode_cache_beyond_4gib(oracle):
    """A pool of more than 5 GiB per cache whose sequences sit in its last
    pages: every byte they read lies past 4 GiB from the pool's start.  The
    pool's other pages are never written (uninitialised device memory) and
    must never be read."""
    lens = [300, 1025, 64]
    hq, hkv, dqk, ps = 8, 2, 128, 64
    host, ds, dev = _inputs(oracle, synth.BF16, lens, hq, hkv, dqk, ps, 4242)
    page_bytes = ps * hkv * dqk * 2
    pool = (5 << 30) // page_bytes + 16
    used = dev[1].shape[0]
    base = pool - used
    print("decode with a pool of %d pages (%.2f GiB per cache), pages %d.. used" % (
        pool, pool * page_bytes / 2.0 ** 30, base), flush=True)
    kbig = torch.empty((pool, ps, hkv, dqk), dtype=torch.bfloat16, device=DEV)
    vbig = torch.empty((pool, ps, hkv, 128), dtype=torch.bfloat16, device=DEV)
    kbig[base:] = dev[1]
    vbig[base:] = dev[2]
    table = dev[3] + base
    o, lse = pkg.flash_attn_decode_paged(dev[0], kbig, vbig, table, dev[4], max(lens))
    torch.cuda.synchronize()
    del kbig, vbig
    _compare(oracle, synth.BF16, host, ds, lens, o, lse, 1.0 / math.sqrt(128))
