"""Helpers shared by the GPU parity tests: device upload of seeded inputs,
the error metrics, and the pass criteria.

Pass criteria against the fp64 oracle (tol = 1e-2 for BF16, 5e-2 for FP8,
the FP8 oracle running on the same e4m3 codes and descales), over the checked
rows i (per-row relative L2 error err_i of the output row):
  pooled   ||O_gpu - O_ref|| / ||O_ref|| over all checked rows     <= tol
  row-RMS  sqrt(mean_i err_i^2)                                    <= tol
  BF16     err_i <= tol and |dlse_i| <= tol for every row
  FP8      every row within its own first-order error bound:
             err_i    <= max(tol, kappa_i * (EPS_P + GAMMA8 * sabs_i))
             |dlse_i| <= -ln(1 - EPS_P * (1 - wmax_i)) + FLUSH
                         + GAMMA8 * sabs_i + 2^-22 |lse_i|
           with the oracle's per-row kappa_i, wmax_i and sabs_i.

The FP8 error model.  The row's probabilities reach P.V, and the row sum,
each with a relative error from two sources:
  - the e4m3 encoding of P, at most EPS_P in magnitude: 0.0796 for the lean
    code (its largest deviation from 2^y over the e4m3 normal range, from
    below) and 1/17 for round-to-nearest exp2 values; zero for the keys at
    the row maximum, whose probability is exactly 2^8 (a block's values more
    than 2^13 below its maximum fall into the subnormal range and may be
    lost; their share of any row is below FLUSH = 2^-7);
  - the score, evaluated by the FP8 matrix instruction, which sums each group
    of 8 consecutive products with every product truncated toward zero to 13
    bits below the largest product of its group (measured, see
    test_gpu_score_accuracy.py): at most 7 * 2^-13 of the group's largest
    term per group, so |ds_ij| <= GAMMA8 * tau * sum_c |q_ic k_jc| with
    GAMMA8 = 7 * 2^-13.
A common shift of a row's scores cancels in the softmax; the remaining
relative errors e_j of the weights move the row by sum_j w_ij e_j (v_j - o_i),
whose RMS over independent errors of size e is e * kappa_i * |o_i| (kappa_i is
the oracle's sensitivity of the row to relative errors of its probabilities),
and move the log-sum-exp by sum_j w_ij e_j.  The bounds above take e as the
largest error a single probability can carry.  BF16 rounds P to bf16 (2^-9
relative) and sums scores in fp32, far inside tol.
"""
import numpy as np
import torch

import causal_prefill_attention_attn_amd as pkg
from causal_prefill_attention_attn_amd import synth

from gpu_util_cpu import EPS_P, FLUSH, GAMMA8, TOL  # noqa: F401  (constants of the error model)

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


def judge(name, dtype, go, gl, ro, rl, st, exact_p=False, top_exact=True):
    """Apply the pass criteria of this module's docstring.

    go, ro: [B, rows, H, d_v] GPU and oracle outputs (fp64); gl, rl: [B, H,
    rows] LSEs (gl may be None); st: the oracle's per-row statistics.
    ``exact_p``: the probabilities were rounded exp2 values, not the lean
    code.  ``top_exact`` False: the result is not one softmax whose largest
    probability was encoded exactly (a merge of partial results), so no mass
    is taken as exact in the LSE bound."""
    fp8 = dtype == synth.FP8
    assert np.isfinite(go).all(), "non-finite output"
    pooled = float(np.linalg.norm(go - ro) / np.linalg.norm(ro))
    err = np.linalg.norm(go - ro, axis=-1) / np.maximum(np.linalg.norm(ro, axis=-1), 1e-30)
    err = np.transpose(err, (0, 2, 1))            # [B, H, rows], the layout of the statistics
    rms = float(np.sqrt(np.mean(err ** 2)))
    tol = TOL[dtype]
    kap, sabs = st["kappa"], st["sabs"]
    wmax = st["wmax"] if top_exact else np.zeros_like(kap)
    if fp8:
        eps = EPS_P["exact" if exact_p else "lean"]
        row_bound = np.maximum(tol, kap * (eps + GAMMA8 * sabs))
        lse_bound = (-np.log1p(-eps * (1.0 - wmax)) + FLUSH + GAMMA8 * sabs
                     + 2.0 ** -22 * np.abs(rl))
    else:
        row_bound = np.full(err.shape, tol)
        lse_bound = np.full(err.shape, tol)
    above = err > tol
    lerr = float(np.abs(gl - rl).max()) if gl is not None else 0.0
    lratio = float((np.abs(gl - rl) / lse_bound).max()) if gl is not None else 0.0
    msg = ("%s rows %d pooled %.3e row-RMS %.3e worst-row %.3e (max err/bound %.3f; %d rows above "
           "tol, kappa %.2f..%.2f) max|dlse| %.3e (max |dlse|/bound %.3f) (tol %.0e)" % (
               name, err.size, pooled, rms, float(err.max()), float((err / row_bound).max()),
               int(above.sum()), float(kap[above].min()) if above.any() else 0.0,
               float(kap[above].max()) if above.any() else 0.0, lerr, lratio, tol))
    print(msg, flush=True)
    assert pooled <= tol and rms <= tol, msg
    assert (err <= row_bound).all(), msg
    assert lratio <= 1.0, msg
    return pooled, rms, float(err.max()), lerr


def check(oracle, w, enc, ds, o, lse, rows=None, causal=True, tau=None, heads=None,
          exact_p=False):
    """Compare GPU o/lse with the oracle on the given rows (all when None) and
    heads (all when None) under the criteria of this module's docstring."""
    tau = w.softmax_scale if tau is None else tau
    q, k, v = enc
    if heads is not None:
        q, k, v = (np.ascontiguousarray(x[:, :, heads]) for x in (q, k, v))
    ro, rl, st = oracle.attention(q, k, v, w.dtype, tau, causal, rows=rows, q_descale=ds[0],
                                  k_descale=ds[1], v_descale=ds[2], stats=True)
    go = o_to_f64(o)
    gl = lse.cpu().numpy().astype(np.float64) if lse is not None else None
    if heads is not None:
        go = go[:, :, heads]
        gl = gl[:, heads] if gl is not None else None
    if rows is not None:
        go = go[:, rows]
        gl = gl[:, :, rows] if gl is not None else None
    return judge(w.name, w.dtype, go, gl, ro, rl, st, exact_p=exact_p)
