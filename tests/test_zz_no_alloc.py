"""The allocation-free decode step (attn_decode_paged_noalloc) against the
workspace entry point (attn_decode_paged) through the C ABI: same kernels, so
bitwise equal outputs, on two calls in a row (the second with a smaller
step), and against the oracle.  The allocation-free call keeps the split
partials in the library's static per-GPU scratch; it is for callers that
cannot allocate."""
import numpy as np
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg
from causal_prefill_attention_attn_amd import synth
from decode_util import scatter
from gpu_util import DEV, bf16_to_device, u8_to_device

pytestmark = pytest.mark.gpu


def _case(oracle, dtype, lens, hq, hkv, dqk, ps, seed):
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
    up = bf16_to_device if dtype == synth.BF16 else u8_to_device
    dev = dict(q=up(enc[0]), k=up(kp), v=up(vp), table=torch.from_numpy(table).to(DEV),
               lens=torch.from_numpy(np.asarray(lens, np.int32)).to(DEV))
    host = (enc[0], kp, vp, table)
    return dict(dev=dev, host=host, ds=ds, lens=lens, B=B, hq=hq, hkv=hkv, dqk=dqk, ps=ps,
                pages=kp.shape[0], lmax=lmax, dtype=dtype)


def _run(c, noalloc):
    d = c["dev"]
    o = torch.full((c["B"], c["hq"], 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((c["B"], c["hq"]), float("nan"), dtype=torch.float32, device=DEV)
    tau = 1.0 / np.sqrt(c["dqk"])
    st = torch.cuda.current_stream().cuda_stream
    common = (d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["table"].data_ptr(),
              d["lens"].data_ptr(), o.data_ptr(), lse.data_ptr())
    sizes = (c["B"], c["hq"], c["hkv"], c["dqk"], 128, c["pages"], c["ps"], d["table"].shape[1],
             c["lmax"], tau, c["dtype"], *c["ds"])
    if noalloc:
        rc = pkg.attn_decode_paged_noalloc(*common, *sizes, st)
    else:
        need = pkg.attn_decode_workspace_bytes(c["B"], c["hq"], c["hkv"], c["lmax"], 128)
        ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
        rc = pkg.attn_decode_paged(*common, ws.data_ptr(), need, *sizes, st)
    assert rc == 0, pkg.attn_status_string(rc)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP8])
def test_noalloc_equals_workspace_entry_point(oracle, dtype):
    big = _case(oracle, dtype, [3000, 17, 0, 9000, 4100, 1, 700, 8192], 32, 8, 128, 64, 11 + dtype)
    small = _case(oracle, dtype, [5, 300, 1025], 8, 2, 192, 32, 12 + dtype)
    for c in (big, small):          # two calls in a row, the second smaller
        print("case B %d hq %d hkv %d dqk %d lens %s" % (c["B"], c["hq"], c["hkv"], c["dqk"],
                                                        c["lens"]), flush=True)
        need = pkg.attn_decode_workspace_bytes(c["B"], c["hq"], c["hkv"], c["lmax"], 128)
        assert 0 < need <= pkg.ATTN_DECODE_SCRATCH_BYTES
        o_n, l_n = _run(c, True)
        o_w, l_w = _run(c, False)
        assert torch.equal(o_n.view(torch.int16), o_w.view(torch.int16))
        assert torch.equal(l_n.view(torch.int32), l_w.view(torch.int32))
        ro, rl = oracle.decode_paged(*c["host"], np.asarray(c["lens"]), dtype,
                                     1.0 / np.sqrt(c["dqk"]), q_descale=c["ds"][0],
                                     k_descale=c["ds"][1], v_descale=c["ds"][2])
        live = np.asarray(c["lens"]) > 0
        go = o_n.float().cpu().numpy().astype(np.float64)
        err = np.linalg.norm(go[live] - ro[live], axis=-1) / np.linalg.norm(ro[live], axis=-1)
        assert err.max() <= 3e-3, err.max()
    # the larger step again after the smaller one: the scratch keeps the last
    # call's partials, which the next step must not depend on
    o_n, l_n = _run(big, True)
    o_w, l_w = _run(big, False)
    assert torch.equal(o_n.view(torch.int16), o_w.view(torch.int16))
    assert torch.equal(l_n.view(torch.int32), l_w.view(torch.int32))


def test_noalloc_too_large_is_rejected_before_launch():
    x = torch.zeros((16,), dtype=torch.uint8, device=DEV)
    o = torch.zeros((16,), dtype=torch.uint8, device=DEV)
    p = x.data_ptr()
    rc = pkg.attn_decode_paged_noalloc(p, p, p, p, p, o.data_ptr(), None, 512, 64, 8, 128, 128,
                                       1 << 20, 64, 1 << 14, 1 << 20, 0.1, 0, 1.0, 1.0, 1.0, None)
    assert rc == -10
    torch.cuda.synchronize()
    assert int(o.sum()) == 0
