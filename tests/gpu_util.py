"""Helpers shared by the GPU parity tests: device upload of seeded inputs,
the error metrics, and the tolerances.

Pass criteria against the fp64 oracle (tol = 1e-2 for BF16, 5e-2 for FP8,
the FP8 oracle running on the same e4m3 codes and descales):
  pooled    ||O_gpu - O_ref|| / ||O_ref|| over all checked rows   <= tol
  row-RMS   sqrt(mean over rows of (row rel-L2 error)^2)           <= tol
  worst row max over rows of the row rel-L2 error  <= tol (BF16), 10*tol (FP8)
  LSE       |lse_gpu - lse_ref| <= tol + LSE_REL[dtype] * |lse_ref|
The FP8 worst-row bound is loose because a row whose few dominant V rows
cancel (small ||o|| against large ||v||) turns the ~2^-4 relative rounding
of e4m3 probabilities into a large relative row error; the relative LSE term
covers fp32 accumulation of large FP8 logits inside the matrix cores.
"""
import numpy as np
import torch

import causal_prefill_attention_attn_amd as pkg
from causal_prefill_attention_attn_amd import synth

TOL = {synth.BF16: 1e-2, synth.FP8: 5e-2}
WORST_ROW = {synth.BF16: 1.0, synth.FP8: 10.0}   # multiples of TOL
LSE_REL = {synth.BF16: 0.0, synth.FP8: 5e-4}
DEV = torch.device("cuda:0")


def bf16_to_device(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_to_device(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).to(DEV)


def make_inputs(oracle, w: synth.Workload, qkv=None):
    """Host encodings (q, k, v), descales and device tensors for workload w."""
    qf, kf, vf = synth.generate(w) if qkv is None else qkv
    if w.dtype == synth.BF16:
        enc = [synth.to_bf16_bits(x) for x in (qf, kf, vf)]
        ds = [1.0, 1.0, 1.0]
        dev = [bf16_to_device(x) for x in enc]
    else:
        ds = [oracle.descale_amax(x) for x in (qf, kf, vf)]
        enc = [oracle.quantize_e4m3(x, d) for x, d in zip((qf, kf, vf), ds)]
        dev = [u8_to_device(x) for x in enc]
    return enc, ds, dev


def run_gpu(dev, w: synth.Workload, ds, causal=True, tau=None, lse=True):
    tau = w.softmax_scale if tau is None else tau
    o, l = pkg.flash_attn_func(*dev, softmax_scale=tau, causal=causal, q_descale=ds[0],
                               k_descale=ds[1], v_descale=ds[2], return_lse=lse)
    torch.cuda.synchronize()
    return o, l


def o_to_f64(o: torch.Tensor) -> np.ndarray:
    return o.float().cpu().numpy().astype(np.float64)


def errors(go: np.ndarray, ro: np.ndarray):
    """(pooled rel-L2, row-RMS of rel-L2, worst row rel-L2) over rows [b, i, h, :]."""
    diff = go - ro
    pooled = float(np.linalg.norm(diff) / np.linalg.norm(ro))
    num = np.linalg.norm(diff, axis=-1)
    den = np.linalg.norm(ro, axis=-1)
    r = num / np.maximum(den, 1e-30)
    return pooled, float(np.sqrt(np.mean(r ** 2))), float(r.max())


def check(oracle, w, enc, ds, o, lse, rows=None, causal=True, tau=None, heads=None):
    """Compare GPU o/lse with the oracle on the given rows (all when None)."""
    tau = w.softmax_scale if tau is None else tau
    q, k, v = enc
    if heads is not None:
        q, k, v = (np.ascontiguousarray(x[:, :, heads]) for x in (q, k, v))
    ro, rl = oracle.attention(q, k, v, w.dtype, tau, causal, rows=rows, q_descale=ds[0],
                              k_descale=ds[1], v_descale=ds[2])
    go = o_to_f64(o)
    gl = lse.cpu().numpy().astype(np.float64) if lse is not None else None
    if heads is not None:
        go = go[:, :, heads]
        gl = gl[:, heads] if gl is not None else None
    if rows is not None:
        go = go[:, rows]
        gl = gl[:, :, rows] if gl is not None else None
    pooled, rms, worst = errors(go, ro)
    tol = TOL[w.dtype]
    if gl is not None:
        lexcess = float((np.abs(gl - rl) - LSE_REL[w.dtype] * np.abs(rl)).max())
        lerr = float(np.abs(gl - rl).max())
    else:
        lexcess = lerr = 0.0
    msg = "%s pooled %.3e row-RMS %.3e worst-row %.3e max|dlse| %.3e (tol %.0e)" % (
        w.name, pooled, rms, worst, lerr, tol)
    print(msg, flush=True)
    assert np.isfinite(go).all(), "non-finite output"
    assert pooled <= tol and rms <= tol and worst <= WORST_ROW[w.dtype] * tol, msg
    assert lexcess <= tol, msg
    return pooled, rms, worst, lerr
