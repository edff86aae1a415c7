"""GPU parity of the FP8 e4m3 path against the fp64 oracle run on the same
e4m3 codes and descales (through the C ABI)."""
import hashlib

import numpy as np
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg
from causal_prefill_attention_attn_amd import synth

from gpu_util import check, make_inputs, o_to_f64, run_gpu

pytestmark = pytest.mark.gpu


def _w(name, B, H, S, d_qk=128, index=70, recipe="gaussian"):
    return synth.Workload(name, index, synth.FP8, B, H, S, d_qk, 128, recipe, name)


@pytest.mark.parametrize("d_qk", [128, 192])
@pytest.mark.parametrize("S", [1, 7, 127, 129, 300, 1000])
def test_ragged_lengths(oracle, S, d_qk):
    w = _w("fp8_%d_%d" % (d_qk, S), 2, 2, S, d_qk=d_qk, index=70 + S % 13)
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse)


@pytest.mark.parametrize("d_qk", [128, 192])
def test_non_causal(oracle, d_qk):
    w = _w("fp8_nc_%d" % d_qk, 1, 2, 333, d_qk=d_qk, index=71)
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds, causal=False)
    check(oracle, w, enc, ds, o, lse, causal=False)


def test_llm_like_small(oracle):
    w = _w("fp8_llm", 1, 4, 2048, index=72, recipe="llm")
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse)


def test_row0_bitwise(oracle):
    # query 0 sees key 0 only: P = 1 exactly (256 * 2^-8), l = 1, so
    # O[0] = bf16(fp32(decode(v) * v_descale))
    w = _w("fp8_row0", 2, 3, 260, index=73)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    v0 = dev[2][:, 0].view(torch.float8_e4m3fn).float() * torch.tensor(ds[2], dtype=torch.float32,
                                                                      device=dev[2].device)
    assert torch.equal(o[:, 0].view(torch.int16), v0.to(torch.bfloat16).view(torch.int16))


def test_zero_query_prefix_mean(oracle):
    w = _w("fp8_qzero", 1, 2, 900, index=74)
    qf, kf, vf = synth.generate(w)
    qf[:] = 0
    enc, ds, dev = make_inputs(oracle, w, (qf, kf, vf))
    o, lse = run_gpu(dev, w, ds)
    vh = oracle.decode_e4m3(enc[2]) * ds[2]
    prefix = np.cumsum(vh, axis=1) / np.arange(1, w.S + 1)[None, :, None, None]
    assert np.abs(o_to_f64(o) - prefix).max() <= 2e-2 * np.abs(vh).max()
    np.testing.assert_allclose(lse.cpu().numpy(), np.broadcast_to(np.log(np.arange(1, w.S + 1)), (1, 2, w.S)),
                               rtol=0, atol=1e-4)


def test_deterministic(oracle):
    w = _w("fp8_det", 1, 8, 4096, index=75)
    enc, ds, dev = make_inputs(oracle, w)
    hashes = set()
    for _ in range(20):
        o, lse = pkg.flash_attn_func(*dev, causal=True, q_descale=ds[0], k_descale=ds[1], v_descale=ds[2])
        torch.cuda.synchronize()
        hashes.add(hashlib.sha256(o.view(torch.int16).cpu().numpy().tobytes() +
                                  lse.cpu().numpy().tobytes()).hexdigest())
    assert len(hashes) == 1


@pytest.mark.parametrize("name", ["C3", "C4", "C4g", "C5"])
def test_full_size_sampled_rows(oracle, name):
    """Every head, 256 sampled rows each (first rows, tile and workgroup
    edges, the middle, the end, seeded uniform rows), at the bench's launch
    configuration: at 32K tokens the grid runs the XCD head-major order."""
    w = synth.WORKLOADS[name]
    print("case", name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    rows = synth.sample_rows(w.S, 256)
    check(oracle, w, enc, ds, o, lse, rows=rows)
    del dev, o, lse
    torch.cuda.empty_cache()


def test_two_batches_at_32k(oracle):
    """B = 2, H = 4 at 32K tokens: B*H = 8 problems of 128 query blocks take
    the XCD head-major grid order with a batch index above 0."""
    w = _w("fp8_b2_32k", 2, 4, 32768, index=76)
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse, rows=synth.sample_rows(w.S, 128))
    del dev, o, lse
    torch.cuda.empty_cache()


def _run_exact(dev, w, ds):
    o, lse = pkg.flash_attn_func(*dev, softmax_scale=w.softmax_scale, causal=True,
                                 q_descale=ds[0], k_descale=ds[1], v_descale=ds[2], exact_p=True)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d_qk", [128, 192])
@pytest.mark.parametrize("S", [7, 129, 1000])
def test_exact_p_ragged_lengths(oracle, S, d_qk):
    """Probabilities by exp2 and the rounding conversion (ATTN_FLAG_EXACT_P)."""
    w = _w("exactp%d_%d" % (S, d_qk), 1, 2, S, d_qk=d_qk, index=90 + S % 7 + d_qk)
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = _run_exact(dev, w, ds)
    check(oracle, w, enc, ds, o, lse, exact_p=True)


def test_exact_p_full_size_sampled_rows(oracle):
    w = synth.WORKLOADS["C4g"]
    print("case C4g exact P", flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = _run_exact(dev, w, ds)
    rows = synth.sample_rows(w.S, 256)
    check(oracle, w, enc, ds, o, lse, rows=rows, exact_p=True)
    del dev, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d_qk", [128, 192])
def test_non_causal_many_passes(oracle, d_qk):
    """Non-causal at S = 4096: every tile of every row is visible, so the
    interior loop runs whole passes (eight or four tiles each) many times
    with no mask; 256 sampled rows on every head against the oracle."""
    w = _w("fp8_nc4k_%d" % d_qk, 1, 4, 4096, d_qk=d_qk, index=76)
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds, causal=False)
    check(oracle, w, enc, ds, o, lse, rows=synth.sample_rows(w.S), causal=False)
