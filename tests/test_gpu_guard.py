"""Output bounds: every kernel writes only inside its outputs.

o, lse and the decode workspace are placed in the middle of larger buffers
whose surrounding bytes hold a sentinel pattern; after the call (through the
C ABI) every sentinel byte must be unchanged and every output byte written.
Cases: ragged sequence lengths (1, 7, 129, 1000) for both element types and
head shapes, packed batches with empty sequences, and decode steps with many
key splits (the workspace has its own guards; the allocation-free decode
writes only o and lse)."""
import numpy as np
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg
from causal_prefill_attention_attn_amd import synth

from gpu_util import DEV

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of sentinel before and after each output
SENT = 0xA5


class Guarded:
    """nbytes of output inside a sentinel-filled allocation, 256-byte aligned."""

    def __init__(self, nbytes):
        self.n = nbytes
        self.buf = torch.full((GUARD + nbytes + GUARD,), SENT, dtype=torch.uint8, device=DEV)
        self.ptr = self.buf.data_ptr() + GUARD
        assert self.ptr % 256 == 0

    def check(self, name, fully_written=True):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        assert (b[:GUARD] == SENT).all(), "%s: bytes before the buffer changed" % name
        assert (b[GUARD + self.n:] == SENT).all(), "%s: bytes after the buffer changed" % name
        return b[GUARD:GUARD + self.n]


def _inputs(dtype, shape_qk, shape_v, seed):
    g = torch.Generator().manual_seed(seed)
    x = [torch.randn(s, generator=g) for s in (shape_qk, shape_qk, shape_v)]
    if dtype == synth.BF16:
        return [t.to(torch.bfloat16).to(DEV) for t in x], [1.0] * 3
    out, ds = [], []
    for t in x:
        c, d = pkg.quantize_fp8(t.to(DEV))
        out.append(c)
        ds.append(d)
    return out, ds


@pytest.mark.parametrize("dtype,d_qk", [(synth.BF16, 128), (synth.BF16, 192), (synth.FP8, 128),
                                        (synth.FP8, 192)])
@pytest.mark.parametrize("S", [1, 7, 129, 1000])
def test_prefill_writes_only_its_outputs(dtype, d_qk, S):
    B, H = 2, 3
    print("case dtype %d d_qk %d S %d" % (dtype, d_qk, S), flush=True)
    (q, k, v), ds = _inputs(dtype, (B, S, H, d_qk), (B, S, H, 128), 100 + S + d_qk)
    o = Guarded(B * S * H * 128 * 2)
    lse = Guarded(B * H * S * 4)
    st = pkg.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.ptr, lse.ptr, B, S, H, d_qk, 128,
                      1.0 / np.sqrt(d_qk), 1, dtype, *ds, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    ob = o.check("o").view(np.uint16)
    lb = lse.check("lse").view(np.float32)
    # every output element written: no sentinel pattern left, finite values
    assert not (ob == 0xA5A5).any() and np.isfinite(lb).all()


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP8])
def test_varlen_with_empty_sequences(dtype):
    lens = [0, 5, 0, 0, 300, 1, 0, 257, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total, H = int(cu[-1]), 2
    (q, k, v), ds = _inputs(dtype, (total, H, 128), (total, H, 128), 7 + dtype)
    tcu = torch.from_numpy(cu).to(DEV)
    o = Guarded(total * H * 128 * 2)
    lse = Guarded(H * total * 4)
    st = pkg.attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.ptr, lse.ptr,
                             tcu.data_ptr(), len(lens), total, max(lens), H, 128, 128,
                             1.0 / np.sqrt(128), 1, dtype, *ds,
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert not (o.check("o").view(np.uint16) == 0xA5A5).any()
    assert np.isfinite(lse.check("lse").view(np.float32)).all()


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP8])
def test_decode_many_splits_writes_only_its_outputs(dtype, noalloc):
    B, Hq, Hkv, ps, D = 3, 8, 2, 64, 128
    lens = [20000, 0, 7777]                  # tens of key splits per sequence
    lmax = max(lens)
    pages_per = (lmax + ps - 1) // ps
    npages = B * pages_per
    g = torch.Generator().manual_seed(55 + dtype)
    x = [torch.randn(s, generator=g) for s in ((B, Hq, D), (npages, ps, Hkv, D), (npages, ps, Hkv, D))]
    if dtype == synth.BF16:
        (q, kc, vc), ds = [t.to(torch.bfloat16).to(DEV) for t in x], [1.0] * 3
    else:
        enc = [pkg.quantize_fp8(t.to(DEV)) for t in x]
        (q, kc, vc), ds = [c for c, _ in enc], [d for _, d in enc]
    table = torch.randperm(npages, generator=g).to(torch.int32).view(B, pages_per).to(DEV)
    tl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = Guarded(B * Hq * D * 2)
    lse = Guarded(B * Hq * 4)
    st_ = torch.cuda.current_stream().cuda_stream
    args = (B, Hq, Hkv, D, D, npages, ps, pages_per, lmax, 1.0 / np.sqrt(D), dtype, *ds)
    if noalloc:
        rc = pkg.attn_decode_paged_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                           table.data_ptr(), tl.data_ptr(), o.ptr, lse.ptr,
                                           *args, st_)
    else:
        need = pkg.attn_decode_workspace_bytes(B, Hq, Hkv, lmax, D)
        assert need // (B * Hq * 129 * 4) >= 16          # many splits
        ws = Guarded(need)
        rc = pkg.attn_decode_paged(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), table.data_ptr(),
                                   tl.data_ptr(), o.ptr, lse.ptr, ws.ptr, need, *args, st_)
    assert rc == 0
    ob = o.check("o").view(np.uint16)
    lb = lse.check("lse").view(np.float32)
    if not noalloc:
        ws.check("workspace")
    assert not (ob == 0xA5A5).any()
    # the empty sequence: o = 0, lse = -inf; the others finite
    assert np.isneginf(lb.reshape(B, Hq)[1]).all() and np.isfinite(lb.reshape(B, Hq)[[0, 2]]).all()
