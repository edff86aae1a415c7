"""Benchmark: causal prefill attention forward TFLOP/s on one MI355X.

One step = one attn_fwd call over the whole workload (every query block of
every head), inputs resident in HBM.  Prints ONE JSON line: the headline
workload (C4 by default) at the top level, and under "also" the same record
for further workloads (by default C2x, BF16 at 32K, and C5, the FP8 MLA
shape), each with its own timed steps, roofline, sustained window (power,
clock, clock-adjusted fraction) and a bitwise determinism check over many
launches.

  python bench.py [--steps K] [--warmup W] [--workload C4] [--gpus 1]
                  [--also C2x,C5|none] [--det-launches N] [--sub-energy S]
                  [--cpu-seconds 12] [--no-cpu] [--varlen N] [--hadamard]
                  [--energy SECONDS] [--decode D1,D2,D3,D4]

Workloads (seeded synthetic inputs, recipes in causal_prefill_attention_attn_amd/synth.py):
  C4  (default) FP8 e4m3, B1 H32 S32768 d128, LLM-like activations
  C4g FP8 e4m3, B1 H32 S32768 d128, N(0,1)
  C5  FP8 e4m3 MLA, B1 H16 S32768 d_qk192 d_v128, N(0,1)
  C3  FP8 e4m3, B1 H32 S16384 d128, N(0,1)
  C2  BF16, B1 H32 S4096 d128, N(0,1)
  C2x BF16, B1 H32 S32768 d128, N(0,1)
  C5b BF16 MLA, B1 H16 S32768 d_qk192 d_v128, N(0,1)
  C4h4 FP8 e4m3, B1 H4 S32768 d128, LLM-like (one GPU's share of C4's heads)
FLOPs per step: B*H*S^2*(d_qk+d_v) (both products over the causal half).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C4")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--hadamard", action="store_true",
                    help="also time the Hadamard rotation of Q, K, V (fp32) and of O (bf16) "
                         "at the workload's shape, the optional step before FP8 quantization")
    ap.add_argument("--varlen", type=int, default=0,
                    help="also time attn_fwd_varlen on the workload's tokens split into this "
                         "many packed sequences of seeded random lengths")
    ap.add_argument("--energy", type=float, default=6.0,
                    help="run the kernel back to back for this many seconds (0: skip) and report "
                         "joules from the GPU's energy accumulator, average watts, TFLOP/J and "
                         "the shader clock sampled meanwhile (median, p10)")
    ap.add_argument("--decode", default="",
                    help="also time attn_decode_paged on these decode workloads (comma "
                         "separated names from synth.DECODE_WORKLOADS, or 'all')")
    ap.add_argument("--also", default="C2x,C5",
                    help="also measure these workloads in the same run, each as a sub-record "
                         "of the JSON line with its own timed steps, roofline, sustained "
                         "window and determinism check ('none' to skip); the metric covers "
                         "FP8 and BF16 at 32K, and C5 is the pages' MLA shape")
    ap.add_argument("--sub-energy", type=float, default=3.0,
                    help="sustained window (seconds) of each sub-record")
    ap.add_argument("--det-launches", type=int, default=7200,
                    help="launches of the headline workload whose outputs are each compared "
                         "bitwise, on the device, with the first launch's (sub-records: a "
                         "tenth of it)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one float32 elementwise copy of this many MiB before the "
                         "warmup (reads and writes exactly that many bytes): the reference "
                         "for scaling HBM byte counters")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_inputs(w, torch, pkg, synth):
    """Seeded inputs on the device: bf16, or e4m3 codes quantized by the library."""
    qf, kf, vf = synth.generate(w)
    dev = torch.device("cuda:0")
    if w.dtype == synth.BF16:
        t = [torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (qf, kf, vf)]
        return t, [1.0, 1.0, 1.0], (qf, kf, vf)
    t, ds = [], []
    for x in (qf, kf, vf):
        codes, d = pkg.quantize_fp8(torch.from_numpy(x).to(dev))
        t.append(codes)
        ds.append(d)
    torch.cuda.synchronize()
    return t, ds, (qf, kf, vf)


def profiled(w, dtname):
    """Figures rocprofv3 measured for this workload's kernel, from profiles/:
    HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known
    size), the sustained shader clock (GRBM_GUI_ACTIVE / duration) and the
    MFMA-busy and VALU-busy fractions.  All None when no summary exists or
    the kernel source changed since it was taken."""
    import hashlib
    import re
    none = {"traffic": None, "sclk_mhz": None, "mfma_busy": None, "valu_busy": None}
    path = os.path.join(ROOT, "profiles", "attn_fwd_%s_d%d_%s.md" % (dtname, w.d_qk, w.name))
    if not os.path.exists(path):
        return none
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_launch", "kernel_source",
                                                      "kernel_source_sha256"):
            k, val = line.split(":", 1)
            fields[k] = val.strip()
        m = re.search(r"sustained clock .*: (\d+) MHz", line)
        if m:
            fields["sclk_mhz"] = m.group(1)
        m = re.match(r"- (MFMA|VALU) busy = .*: ([0-9.]+)%", line)
        if m:
            fields[m.group(1).lower() + "_busy"] = float(m.group(2)) / 100.0
    try:
        src = open(os.path.join(ROOT, fields["kernel_source"]), "rb").read()
    except (KeyError, OSError):
        return none
    if hashlib.sha256(src).hexdigest() != fields.get("kernel_source_sha256"):
        return none
    return {"traffic": int(fields["traffic_bytes_per_launch"]),
            "sclk_mhz": int(fields["sclk_mhz"]) if "sclk_mhz" in fields else None,
            "mfma_busy": fields.get("mfma_busy"), "valu_busy": fields.get("valu_busy")}


def input_stats(w, host, nrows=64):
    """Logit spread and effective number of attended keys, 1 / sum_j p_ij^2,
    over seeded sample rows of head 0 (fp32 host inputs; diagnostics of the
    workload, not a parity check)."""
    qf, kf, _ = host
    rng = np.random.default_rng(777)
    rows = np.sort(rng.choice(w.S, size=min(nrows, w.S), replace=False))
    k0 = kf[0, :, 0, :].astype(np.float64)
    std, neff = [], []
    for i in rows:
        s = (k0[: i + 1] @ qf[0, i, 0, :].astype(np.float64)) * w.softmax_scale
        p = np.exp(s - s.max())
        p /= p.sum()
        std.append(float(s.std()) if i > 0 else 0.0)
        neff.append(float(1.0 / np.sum(p * p)))
    return {"sample_rows": int(rows.size), "logit_std_median": round(float(np.median(std)), 3),
            "n_eff_median": round(float(np.median(neff)), 2)}


def cpu_baseline(w, host, seconds, synth, gpu_head0=None):
    """Time the fp64 oracle on a bounded sample of the same workload: a growing
    set of query rows of head 0, until about `seconds` of CPU work.  With
    `gpu_head0` ({name: (o [B,S,d_v], lse [B,S])} of head 0 from GPU launches)
    the same oracle rows also give the accuracy of each GPU output: pooled
    relative L2 of O, the worst row's relative L2 and the largest |dlse|."""
    import oracle
    oracle.build()
    qf, kf, vf = host
    h = 0
    if w.dtype == synth.BF16:
        enc = [synth.to_bf16_bits(np.ascontiguousarray(x[:, :, h:h + 1])) for x in (qf, kf, vf)]
        ds = [1.0, 1.0, 1.0]
    else:
        ds = [oracle.descale_amax(x) for x in (qf, kf, vf)]
        enc = [oracle.quantize_e4m3(np.ascontiguousarray(x[:, :, h:h + 1]), d)
               for x, d in zip((qf, kf, vf), ds)]
    rng = np.random.default_rng(4242)
    n, spent, flops, nrows = 8, 0.0, 0.0, 0
    got = []  # (rows, o [B,rows,d_v], lse [B,rows]) of every chunk
    full_flops = w.B * w.H * w.S * (w.S + 1) / 2.0 * (w.d_qk + w.d_v) * 2.0
    while spent < seconds:
        # each chunk draws distinct rows; chunks are capped at S rows and repeat
        # until the time budget is spent
        rows = np.sort(rng.choice(w.S, size=min(n, w.S), replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        ro, rl = oracle.attention(enc[0], enc[1], enc[2], w.dtype, w.softmax_scale, True,
                                  rows=rows, q_descale=ds[0], k_descale=ds[1], v_descale=ds[2])
        spent += time.perf_counter() - t0
        got.append((rows, ro[:, :, 0, :], rl[:, 0, :]))
        flops += float(np.sum(rows + 1)) * (w.d_qk + w.d_v) * 2.0 * w.B
        nrows += rows.size
        n *= 2
    res = {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "kind": "oracle", "full_run_estimate_s": round(spent * full_flops / flops, 1),
           "sample": "%d uniformly drawn query rows (chunks of at most S distinct rows) of head 0 (batch %d) of %s, causal, "
                     "fp64 oracle, %.1f s" % (nrows, w.B, w.name, spent)}
    if gpu_head0:
        rows = np.concatenate([g[0] for g in got])
        ro = np.concatenate([g[1] for g in got], axis=1)   # [B, n, d_v]
        rl = np.concatenate([g[2] for g in got], axis=1)   # [B, n]
        rows, first = np.unique(rows, return_index=True)  # chunks may repeat rows
        ro, rl = ro[:, first], rl[:, first]
        acc = {"distinct_rows": int(rows.size) * w.B, "head": 0}
        for name, (go, gl) in gpu_head0.items():
            d = go[:, rows, :].astype(np.float64) - ro
            num = np.linalg.norm(d, axis=-1)
            den = np.linalg.norm(ro, axis=-1)
            live = den > 0
            acc[name] = {
                "o_rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ro)),
                "o_worst_row_rel_l2": float((num[live] / den[live]).max()),
                "o_row_rel_l2_rms": float(np.sqrt(np.mean((num[live] / den[live]) ** 2))),
                "lse_max_abs_diff": float(np.abs(gl[:, rows].astype(np.float64) - rl).max())}
        res["gpu_vs_oracle"] = acc
    return res


def time_varlen(w, t, ds, pkg, torch, stream, nseq, reps):
    """TFLOP/s of attn_fwd_varlen on the same tokens (batch 0's rows) cut into
    `nseq` sequences with lognormal(0, 1) lengths (seeded) summing to S; the
    causal FLOPs are sum_s L_s^2 (d_qk + d_v)."""
    rng = np.random.default_rng(2024)
    wts = np.exp(rng.standard_normal(nseq))
    lens = np.maximum(1, np.floor(wts / wts.sum() * w.S)).astype(np.int64)
    lens[-1] += w.S - lens.sum()
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(t[0].device)
    pk = [x[0] for x in t]                       # [S, H, D] views of batch 0
    o = torch.empty((w.S, w.H, w.d_v), dtype=torch.bfloat16, device=t[0].device)
    lse = torch.empty((w.H, w.S), dtype=torch.float32, device=t[0].device)

    def run():
        pkg.flash_attn_varlen_func(*pk, cu, int(lens.max()), softmax_scale=w.softmax_scale,
                                   causal=True, q_descale=ds[0], k_descale=ds[1],
                                   v_descale=ds[2], out=o, lse=lse)
    run()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        run()
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    flops = float(np.sum(lens.astype(np.float64) ** 2)) * w.H * (w.d_qk + w.d_v)
    return {"n_seqs": nseq, "min_len": int(lens.min()), "max_len": int(lens.max()),
            "ms": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}


def energy_run(step, flops, torch, seconds):
    """Energy efficiency of the sustained kernel: launches back to back for
    about `seconds`, bracketed by reads of the device's energy accumulator
    (amdsmi, counter x resolution in microjoules) after a synchronize.  The
    device is the one whose PCI bus matches torch's device 0.  The pages quote
    TFLOP/J for their kernels on captured model layers (miraibroadcast page,
    "ZYFA acelera atencao em ate 1,76x com menos erro"); here the workload is
    the synthetic one being benchmarked."""
    try:
        import amdsmi
    except Exception as e:  # pragma: no cover - depends on the image
        return {"error": "amdsmi not importable: %s" % e}
    try:
        amdsmi.amdsmi_init()
    except Exception as e:
        return {"error": "amdsmi_init failed: %s" % e}
    try:
        bus = torch.cuda.get_device_properties(0).pci_bus_id
        handles = amdsmi.amdsmi_get_processor_handles()
        match = [h for h in handles
                 if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus]
        if len(match) != 1:
            return {"error": "no unique amdsmi device on PCI bus %#x (%d handles)"
                    % (bus, len(handles))}
        h = match[0]

        def joules():
            """(joules, counter timestamp): the accumulator is updated in
            steps, so power is its difference over the difference of the
            timestamps it carries, not over host time"""
            c = amdsmi.amdsmi_get_energy_count(h)
            return c["energy_accumulator"] * c["counter_resolution"] * 1e-6, c["timestamp"]

        # time one launch to size the loop, then run unmeasured for a while:
        # board power and clock take about a second to settle
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step()
        torch.cuda.synchronize()
        per = max(time.perf_counter() - t0, 1e-4)
        warm = max(1.0, seconds / 3.0)
        for i in range(max(1, int(warm / per))):
            step()
            if i % 64 == 63:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        n = max(10, int(seconds / per))
        watts_s, mhz = [], []

        def sample():  # while launches are queued, so the GPU is busy
            try:
                p = amdsmi.amdsmi_get_power_info(h).get("current_socket_power")
                if isinstance(p, (int, float)):
                    watts_s.append(p)
                c = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX).get("clk")
                if isinstance(c, (int, float)):
                    mhz.append(c)
            except Exception:
                pass

        (e0, c0), t0 = joules(), time.perf_counter()
        for i in range(n):
            step()
            if i % 16 == 8:
                sample()
            if i % 64 == 63:
                torch.cuda.synchronize()  # keep the launch queue short
        torch.cuda.synchronize()
        (e1, c1), t1 = joules(), time.perf_counter()
        j, sec = e1 - e0, t1 - t0
        # timestamp unit: the power of ten that makes the counter's window
        # closest to the host's
        dc = float(c1 - c0)
        unit = min((1e-9, 1e-6, 1e-3, 1.0), key=lambda u: abs(np.log(max(dc * u, 1e-12) / sec)))
        win = dc * unit
        watts = j / win if win > 0 else None
        tflops = flops * n / sec / 1e12
        pmed = float(np.median(watts_s)) if watts_s else None
        return {"warmup_seconds": round(warm, 2), "launches": n, "seconds": round(sec, 3),
                "joules": round(j, 2), "counter_window_s": round(win, 3),
                "avg_watts": round(watts, 1) if watts else None,
                "TFLOP/s": round(tflops, 1),
                "TFLOP/J": round(tflops / watts, 3) if watts else None,
                "TFLOP/J_from_sampled_power": round(tflops / pmed, 3) if pmed else None,
                "socket_watts_sampled_median": pmed,
                "gfx_mhz_sampled_median": float(np.median(mhz)) if mhz else None,
                "gfx_mhz_sampled_p10": float(np.percentile(mhz, 10)) if mhz else None,
                "samples": len(watts_s)}
    except Exception as e:
        return {"error": "energy read failed: %s" % e}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def determinism(step, o, lse, torch, n):
    """Run `n` more launches and compare every one's o and lse bitwise with
    the output before them, on the device (a mismatch counter, read once at
    the end), so the check does not pace the launches."""
    if n <= 0:
        return None
    step()
    torch.cuda.synchronize()
    ref_o, ref_l = o.clone(), lse.clone()
    bad = torch.zeros((), dtype=torch.int64, device=o.device)
    for i in range(n):
        step()
        bad += ((o.view(torch.int16) != ref_o.view(torch.int16)).any()
                | (lse.view(torch.int32) != ref_l.view(torch.int32)).any())
        if i % 64 == 63:
            torch.cuda.synchronize()  # keep the launch queue short
    torch.cuda.synchronize()
    nbad = int(bad.item())
    return {"launches": n, "identical": nbad == 0, "mismatching_launches": nbad}


def time_decode(names, pkg, synth, torch, stream, steps, warmup):
    """HBM throughput of one decode step (attn_decode_paged: the split kernel
    and the merge kernel) per decode workload.  Algorithmic bytes: every
    cached key and value row of every sequence once, q, o, the LSE, the
    lengths and the block-table entries used; the partial results in the
    workspace are the kernels' own traffic and are not counted.  Times are
    HIP events on the launching stream around each call, inputs resident."""
    dev = torch.device("cuda:0")
    res = {}
    for name in names:
        w = synth.DECODE_WORKLOADS[name]
        q, kc, vc, table, lens_d = synth.decode_device_inputs(w, torch, dev)
        lens = w.seq_lens().astype(np.int64)
        maxlen = int(lens.max())
        esz = 2 if w.dtype == synth.BF16 else 1
        need = pkg.attn_decode_workspace_bytes(w.B, w.H_q, w.H_kv, maxlen, w.d_v)
        ws = torch.empty((need,), dtype=torch.uint8, device=dev)
        o = torch.empty((w.B, w.H_q, w.d_v), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H_q), dtype=torch.float32, device=dev)

        def call():
            pkg.flash_attn_decode_paged(q, kc, vc, table, lens_d, maxlen, out=o, lse=lse,
                                        workspace=ws)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        # the same step captured in a HIP graph (10 calls per replay): what a
        # serving loop that replays graphs would see, launch overhead removed
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                for _ in range(10):
                    call()
        torch.cuda.current_stream().wait_stream(cs)
        g.replay()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        for _ in range(max(1, steps // 10)):
            g.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        graph_ms = ga.elapsed_time(gb) / (10 * max(1, steps // 10))
        del g
        pages_used = int(((lens + w.page_size - 1) // w.page_size).sum())
        nbytes = (int(lens.sum()) * w.H_kv * (w.d_qk + w.d_v) * esz
                  + w.B * w.H_q * (w.d_qk * esz + w.d_v * 2 + 4) + w.B * 4 + pages_used * 4)
        mean = float(np.mean(ms))
        gbs = nbytes / (mean * 1e-3) / 1e9
        res[name] = {"description": w.description, "bytes": nbytes, "ms_mean": round(mean, 4),
                     "ms_p10_median_p90": [round(float(x), 4)
                                           for x in np.percentile(ms, [10, 50, 90])],
                     "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                     "graph_ms_per_step": round(graph_ms, 4),
                     "graph_GB/s": round(nbytes / (graph_ms * 1e-3) / 1e9, 1),
                     "workspace_bytes": need}
        log("bench: decode %s %.4f ms %.0f GB/s" % (name, mean, gbs))
        del q, kc, vc, ws
    return res


def time_hadamard(w, host, pkg, torch, stream, attn_ms, dev_in, ds, reps=10):
    """Cost of the optional Hadamard rotation, per tensor, as mean times of
    HIP events on the launching stream: the plain per-tensor quantization
    (amax pass + encode pass) of Q, K, V against the fused rotate+quantize
    passes, the standalone rotation of O (bf16) that undoes a rotated V, and
    the attention itself with that O rotation fused into its epilogue (FP8).
    Rates count one read of the input per pass and one write of the codes.
    A pass over a small tensor can take less time than the host needs to
    issue it, so every rep is queued behind a ~20 ms spin kernel before the
    start event runs: the events then bracket GPU time only."""
    dev = torch.device("cuda:0")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            torch.cuda._sleep(40_000_000)
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    st = stream.cuda_stream
    res, extra = {}, 0.0
    for name, x in zip("qkv", host):
        t = torch.from_numpy(x).to(dev)
        d = t.shape[-1]
        rows, n = t.numel() // d, t.numel()
        amax = torch.empty((1,), dtype=torch.float32, device=dev)
        codes = torch.empty(t.shape, dtype=torch.uint8, device=dev)
        plain = timed(lambda: (pkg.attn_amax_f32(t.data_ptr(), n, amax.data_ptr(), st),
                               pkg.attn_quantize_e4m3(t.data_ptr(), n, 1.0, codes.data_ptr(), st)))
        rot = timed(lambda: (pkg.attn_hadamard_amax_f32(t.data_ptr(), rows, d, amax.data_ptr(), st),
                             pkg.attn_hadamard_quantize_e4m3(t.data_ptr(), rows, d, 1.0,
                                                             codes.data_ptr(), st)))
        gbs = (2 * 4 + 1) * n / (rot * 1e-3) / 1e9
        res[name] = {"quantize_ms": round(plain, 4), "rotate_quantize_ms": round(rot, 4),
                     "rotate_quantize_GB/s": round(gbs, 1)}
        extra += rot - plain
        del t, codes
    o = torch.empty((w.B, w.S, w.H, w.d_v), dtype=torch.bfloat16, device=dev).normal_()
    y = torch.empty_like(o)
    orot = timed(lambda: pkg.hadamard(o, out=y))
    res["o_rotate_ms"] = round(orot, 4)
    res["o_rotate_GB/s"] = round(2 * o.numel() * 2 / (orot * 1e-3) / 1e9, 1)
    res["added_ms"] = round(extra + orot, 4)
    res["added_frac_of_attention"] = round((extra + orot) / attn_ms, 4)
    from causal_prefill_attention_attn_amd import synth
    if w.dtype == synth.FP8:
        def attn(rot):
            return lambda: pkg.flash_attn_func(*dev_in, softmax_scale=w.softmax_scale,
                                               causal=True, q_descale=ds[0], k_descale=ds[1],
                                               v_descale=ds[2], out=y, hadamard_o=rot)
        plain_ms, fused_ms = timed(attn(False)), timed(attn(True))
        res["attention_ms"] = round(plain_ms, 4)
        res["attention_with_fused_o_rotation_ms"] = round(fused_ms, 4)
        res["added_ms_with_fused_o_rotation"] = round(extra + fused_ms - plain_ms, 4)
        res["added_frac_with_fused_o_rotation"] = round((extra + fused_ms - plain_ms) / plain_ms, 4)
    return res



def measure(w, args, torch, pkg, synth, energy_seconds, det_launches, calib_mb=0,
            accuracy_heads=False):
    """One workload: inputs on the device, warmup, exactly args.steps timed
    launches (HIP events on the launching stream around each, wall clock
    around all), a sustained window for power and clock, and the
    determinism loop.  With `accuracy_heads`, head 0 of the outputs for the
    oracle leg (for e4m3 also from one exact-P launch after the timed ones).
    Returns (record, step, host inputs, device inputs, descales, mean kernel
    ms, head 0 outputs or None)."""
    dtname = "bf16" if w.dtype == synth.BF16 else "fp8"
    log("bench: workload %s (%s)" % (w.name, w.description))
    t, ds, host = device_inputs(w, torch, pkg, synth)
    dev = t[0].device
    o = torch.empty((w.B, w.S, w.H, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    if calib_mb:
        n = calib_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("bench: calibration copy of %d MiB done" % calib_mb)
        del src, dst

    def step():
        pkg.flash_attn_func(t[0], t[1], t[2], softmax_scale=w.softmax_scale, causal=True,
                            q_descale=ds[0], k_descale=ds[1], v_descale=ds[2], out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("bench: warmup done")
    ref_o, ref_lse = o.clone(), lse.clone()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in ev]
    identical = bool(torch.equal(o.view(torch.int16), ref_o.view(torch.int16)) and
                     torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)))
    del ref_o, ref_lse
    # head 0 of the outputs, for the accuracy figures of the oracle leg; for
    # e4m3 also one (untimed) launch with exact-rounded probabilities.  Only
    # when the oracle leg runs, so that a profiled run holds timed-kind
    # launches only.
    head0 = None
    if accuracy_heads:
        head0 = {("lean_p" if dtname == "fp8" else "default"):
                 (o[:, :, 0].float().cpu().numpy(), lse[:, 0].cpu().numpy())}
    if accuracy_heads and dtname == "fp8":
        oe, le = torch.empty_like(o), torch.empty_like(lse)
        pkg.flash_attn_func(t[0], t[1], t[2], softmax_scale=w.softmax_scale, causal=True,
                            q_descale=ds[0], k_descale=ds[1], v_descale=ds[2], exact_p=True,
                            out=oe, lse=le)
        torch.cuda.synchronize()
        head0["exact_p"] = (oe[:, :, 0].float().cpu().numpy(), le[:, 0].cpu().numpy())
        del oe, le
    prof = profiled(w, dtname)
    ms_step = wall * 1e3 / args.steps
    flops = w.causal_flops
    value = flops / (ms_step * 1e-3) / 1e12
    avg_kern = float(np.mean(kern_ms))
    achieved = flops / (avg_kern * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtname]
    log("bench: %s %d steps, wall %.3f ms/step, kernel mean %.3f ms (median %.3f, min %.3f)"
        % (w.name, args.steps, ms_step, avg_kern, float(np.median(kern_ms)), float(np.min(kern_ms))))
    esz = 2 if w.dtype == synth.BF16 else 1
    rows = w.B * w.S * w.H
    compulsory = rows * (2 * w.d_qk + w.d_v) * esz + rows * w.d_v * 2 + w.B * w.H * w.S * 4
    rec = {
        "workload": w.name, "description": w.description, "dtype": dtname,
        "config": {"B": w.B, "H": w.H, "S": w.S, "d_qk": w.d_qk, "d_v": w.d_v, "causal": True,
                   "softmax_scale": w.softmax_scale, "flops_per_step": flops,
                   # flash_attn_func's default path: the shortest query blocks
                   # are shared among the XCDs through a counter
                   "entry_point": "attn_fwd_balanced"},
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "TFLOP/s": round(value, 2), "frac_of_peak": round(value / peak, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": prof["traffic"],
                     "kernel": "attn_fwd_%s_kernel<%d>" % (dtname, w.d_qk),
                     "kernel_ms_mean": round(avg_kern, 4),
                     "kernel_ms_p10_median_p90": [round(float(x), 4) for x in
                                                  np.percentile(kern_ms, [10, 50, 90])],
                     "sclk_mhz_profiled": prof["sclk_mhz"],
                     "mfma_busy_profiled": prof["mfma_busy"],
                     "valu_busy_profiled": prof["valu_busy"],
                     "compulsory_bytes": compulsory},
        "bitwise_identical_launches": identical,
    }
    if energy_seconds > 0:
        log("bench: %s sustained run of %.0f s for energy and clock" % (w.name, energy_seconds))
        en = energy_run(step, flops, torch, energy_seconds)
        rec["energy"] = en
        mhz = en.get("gfx_mhz_sampled_median")
        if mhz and en.get("TFLOP/s"):
            # throughput and clock of the same sustained window
            rec["roofline"]["frac_clock_adjusted"] = round(
                en["TFLOP/s"] / (peak * mhz / 2400.0), 4)
            rec["roofline"]["frac_clock_adjusted_source"] = (
                "TFLOP/s of the sustained window over the peak scaled by the gfx clock amdsmi "
                "sampled in that window (median %.0f MHz)" % mhz)
    det = determinism(step, o, lse, torch, det_launches)
    if det is not None:
        rec["determinism"] = det
        log("bench: %s %d launches compared bitwise: %s" % (
            w.name, det["launches"], "identical" if det["identical"] else "MISMATCH"))
    return rec, step, host, t, ds, avg_kern, head0


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the kernel runs on one device and "
              "multi-GPU runs are not part of this library; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import causal_prefill_attention_attn_amd as pkg
    from causal_prefill_attention_attn_amd import synth

    w = synth.WORKLOADS[args.workload]
    rec, step, host, t, ds, avg_kern, head0 = measure(w, args, torch, pkg, synth, args.energy,
                                                      args.det_launches, args.calib_copy_mb,
                                                      accuracy_heads=not args.no_cpu)
    stream = torch.cuda.current_stream(t[0].device)
    out = {
        "metric": "causal prefill attention TFLOP/s (FP8 & BF16) and % of MFMA peak at 32K",
        "value": rec["TFLOP/s"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": "synthetic",
        "config": dict(workload=w.name, description=w.description, **rec["config"],
                       frac_of_peak=rec["frac_of_peak"]),
        "roofline": rec["roofline"],
        "bitwise_identical_launches": rec["bitwise_identical_launches"],
        "inputs": input_stats(w, host),
    }
    for k in ("energy", "determinism"):
        if k in rec:
            out[k] = rec[k]
    if args.varlen:
        out["varlen"] = time_varlen(w, t, ds, pkg, torch, stream, args.varlen, args.steps)
    if args.hadamard:
        out["hadamard"] = time_hadamard(w, host, pkg, torch, stream, avg_kern, t, ds)
    if args.decode:
        names = (sorted(synth.DECODE_WORKLOADS) if args.decode == "all"
                 else args.decode.split(","))
        out["decode"] = time_decode(names, pkg, synth, torch, stream, args.steps, args.warmup)
    if not args.no_cpu:
        log("bench: timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds, synth, head0)
    del t, step
    torch.cuda.empty_cache()
    also = [] if args.also in ("", "none") else [x for x in args.also.split(",") if x != w.name]
    if also:
        out["also"] = {}
        for name in also:
            sub, step, _, t, _, _, _ = measure(synth.WORKLOADS[name], args, torch, pkg, synth,
                                               args.sub_energy, args.det_launches // 10)
            out["also"][name] = sub
            del t, step
            torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
