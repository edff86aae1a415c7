"""GPU parity of the BF16 path against the fp64 oracle (through the C ABI)."""
import hashlib

import numpy as np
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg
from causal_prefill_attention_attn_amd import synth

from gpu_util import DEV, bf16_to_device, check, make_inputs, o_to_f64, run_gpu

pytestmark = pytest.mark.gpu


def _w(name, B, H, S, d_qk=128, d_v=128, index=50, recipe="gaussian"):
    return synth.Workload(name, index, synth.BF16, B, H, S, d_qk, d_v, recipe, name)


def test_c1_full(oracle):
    w = synth.WORKLOADS["C1"]
    print("case C1", flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse)


@pytest.mark.parametrize("S", [1, 7, 31, 33, 64, 129, 1000])
def test_ragged_lengths(oracle, S):
    w = _w("ragged%d" % S, 2, 3, S, index=60 + S % 17)
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse)


@pytest.mark.parametrize("S", [1, 100, 257])
def test_non_causal(oracle, S):
    w = _w("noncausal%d" % S, 1, 2, S, index=80)
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds, causal=False)
    check(oracle, w, enc, ds, o, lse, causal=False)


@pytest.mark.parametrize("S", [130, 513])
def test_mla_shape_bf16(oracle, S):
    w = _w("mla%d" % S, 1, 2, S, d_qk=192, index=81)
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    check(oracle, w, enc, ds, o, lse)


def test_row0_is_v0_bitwise(oracle):
    w = _w("row0", 2, 4, 300, index=82)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    # query 0 sees only key 0: P = 1, l = 1, so O[0] is V[0] exactly
    assert torch.equal(o[:, 0].view(torch.int16), dev[2][:, 0].view(torch.int16))
    s00 = w.softmax_scale * np.einsum("bhc,bhc->bh", *(x[:, 0].astype(np.float64) for x in (
        o_to_f64(dev[0]), o_to_f64(dev[1]))))
    np.testing.assert_allclose(lse[:, :, 0].cpu().numpy(), s00, rtol=1e-5, atol=1e-5)


def test_zero_query_prefix_mean(oracle):
    w = _w("qzero", 1, 2, 700, index=83)
    qf, kf, vf = synth.generate(w)
    qf[:] = 0
    enc, ds, dev = make_inputs(oracle, w, (qf, kf, vf))
    o, lse = run_gpu(dev, w, ds)
    vh = o_to_f64(dev[2])
    prefix = np.cumsum(vh, axis=1) / np.arange(1, w.S + 1)[None, :, None, None]
    go = o_to_f64(o)
    assert np.abs(go - prefix).max() <= 2e-2
    np.testing.assert_allclose(lse.cpu().numpy(), np.broadcast_to(np.log(np.arange(1, w.S + 1)), (1, 2, w.S)),
                               rtol=0, atol=1e-4)


def test_lse_optional(oracle):
    w = _w("nolse", 1, 2, 200, index=84)
    enc, ds, dev = make_inputs(oracle, w)
    o1, _ = run_gpu(dev, w, ds, lse=False)
    o2, _ = run_gpu(dev, w, ds, lse=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_deterministic(oracle):
    w = _w("det", 1, 8, 2048, index=85)
    enc, ds, dev = make_inputs(oracle, w)
    hashes = set()
    for _ in range(20):
        o, lse = pkg.flash_attn_func(*dev, causal=True)
        torch.cuda.synchronize()
        hashes.add(hashlib.sha256(o.view(torch.int16).cpu().numpy().tobytes() +
                                  lse.cpu().numpy().tobytes()).hexdigest())
    assert len(hashes) == 1


def test_c2_full_size_sampled_rows(oracle):
    w = synth.WORKLOADS["C2"]
    print("case C2", flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    rows = synth.sample_rows(w.S, 256)
    check(oracle, w, enc, ds, o, lse, rows=rows)


def test_bad_arguments_raise():
    x = torch.zeros((1, 4, 1, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pkg.AttnError) as e:
        pkg.flash_attn_func(x, x, x)
    assert e.value.status == -4  # d = 64 is not a supported head dimension
    y = torch.zeros((1, 4, 1, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pkg.AttnError) as e:
        pkg.flash_attn_func(y, y, y, softmax_scale=float("nan"))
    assert e.value.status == -5


def test_c2x_full_size_sampled_rows(oracle):
    """The BF16 workload at 32K (B1 H32 S32768): 256 sampled rows of every head."""
    w = synth.WORKLOADS["C2x"]
    print("case C2x", flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    rows = synth.sample_rows(w.S, 256)
    check(oracle, w, enc, ds, o, lse, rows=rows)


def test_c5b_full_size_sampled_rows(oracle):
    """BF16 in the MLA shape at 32K (B1 H16 S32768, d_qk 192, d_v 128)."""
    w = synth.WORKLOADS["C5b"]
    print("case C5b", flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds)
    rows = synth.sample_rows(w.S, 256)
    check(oracle, w, enc, ds, o, lse, rows=rows)


@pytest.mark.parametrize("d_qk", [128, 192])
def test_non_causal_many_passes(oracle, d_qk):
    """Non-causal at S = 4096: the interior loop runs whole passes of four
    tiles many times with no mask; 256 sampled rows on every head."""
    w = synth.Workload("bf16_nc4k_%d" % d_qk, 81, synth.BF16, 1, 4, 4096, d_qk, 128, "gaussian",
                       "bf16 non-causal 4096")
    print("case", w.name, flush=True)
    enc, ds, dev = make_inputs(oracle, w)
    o, lse = run_gpu(dev, w, ds, causal=False)
    check(oracle, w, enc, ds, o, lse, rows=synth.sample_rows(w.S), causal=False)
