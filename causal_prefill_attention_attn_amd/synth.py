"""Seeded synthetic workloads (inputs only; no attention arithmetic here).

The pages measure on Gaussian inputs at 32K tokens and on activations
captured from Mistral-7B, Qwen3-8B and DeepSeek-V2-Lite at 16K ("ZYFA acelera
atencao em ate 1,76x com menos erro", miraibroadcast.com page; "Les resultats
revendiques", ai-daily-news.org page).  Captured activations need trained
weights, so the LLM-like recipe below (per-channel lognormal scales with a few
outlier channels) stands in for them, and the MLA recipe takes
DeepSeek-V2-Lite's head shape (QK dim 192 = 128 + 64 rope part, V dim 128).

Every array is drawn with numpy's PCG64 from the seed
``1000 * config_index + {q: 0, k: 1, v: 2}``.  Values are returned as float32;
BF16 workloads are rounded to bf16 by torch's cast (round-to-nearest-even)
and FP8 workloads are quantized by whoever consumes them (the CPU reference
codec in tests, the library's quantizer in the benchmark).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16 = 0
FP8 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    dtype: int          # BF16 or FP8
    B: int
    H: int
    S: int
    d_qk: int
    d_v: int
    recipe: str         # "gaussian" or "llm"
    description: str

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def causal_flops(self) -> float:
        # 2 * B * H * S^2 * (d_qk + d_v) / 2: both products over the causal half
        return float(self.B) * self.H * self.S * self.S * (self.d_qk + self.d_v)

    def with_shape(self, B=None, H=None, S=None) -> "Workload":
        return dataclasses.replace(self, B=B or self.B, H=H or self.H, S=S or self.S)


WORKLOADS = {
    "C1": Workload("C1", 0, BF16, 1, 1, 256, 128, 128, "gaussian",
                   "BF16 causal fwd, B=1 H=1 S=256 d=128, N(0,1)"),
    "C2": Workload("C2", 1, BF16, 1, 32, 4096, 128, 128, "gaussian",
                   "BF16 causal fwd, B=1 H=32 S=4096 d=128, N(0,1)"),
    "C3": Workload("C3", 2, FP8, 1, 32, 16384, 128, 128, "gaussian",
                   "FP8 e4m3 causal fwd, B=1 H=32 S=16384 d=128, N(0,1), per-tensor descale"),
    "C4": Workload("C4", 3, FP8, 1, 32, 32768, 128, 128, "llm",
                   "FP8 e4m3 causal fwd, B=1 H=32 S=32768 d=128, LLM-like activations"),
    "C5": Workload("C5", 4, FP8, 1, 16, 32768, 192, 128, "gaussian",
                   "FP8 e4m3 causal MLA fwd, B=1 H=16 S=32768 d_qk=192 d_v=128, N(0,1)"),
    # supplementary: the Gaussian 32K FP8 case the pages quote, and BF16 at 32K
    "C4g": Workload("C4g", 5, FP8, 1, 32, 32768, 128, 128, "gaussian",
                    "FP8 e4m3 causal fwd, B=1 H=32 S=32768 d=128, N(0,1)"),
    "C2x": Workload("C2x", 6, BF16, 1, 32, 32768, 128, 128, "gaussian",
                    "BF16 causal fwd, B=1 H=32 S=32768 d=128, N(0,1)"),
    # one GPU's share when C4's 32 heads are split over eight GPUs
    "C4h4": Workload("C4h4", 7, FP8, 1, 4, 32768, 128, 128, "llm",
                     "FP8 e4m3 causal fwd, B=1 H=4 S=32768 d=128, LLM-like (1/8 of C4's heads)"),
    # the MLA shape in BF16
    "C5b": Workload("C5b", 8, BF16, 1, 16, 32768, 192, 128, "gaussian",
                    "BF16 causal MLA fwd, B=1 H=16 S=32768 d_qk=192 d_v=128, N(0,1)"),
}


def _draw(rng: np.random.Generator, recipe: str, B: int, S: int, H: int, D: int) -> np.ndarray:
    if recipe == "gaussian":
        return rng.standard_normal((B, S, H, D), dtype=np.float32)
    if recipe == "llm":
        # per (head, channel) std ~ lognormal(0, 1), four outlier channels x20
        sigma = np.exp(rng.standard_normal((H, D))).astype(np.float32)
        for h in range(H):
            ch = rng.choice(D, size=4, replace=False)
            sigma[h, ch] *= 20.0
        x = rng.standard_normal((B, S, H, D), dtype=np.float32)
        x *= sigma[None, None, :, :]
        return x
    raise ValueError(recipe)


def generate(w: Workload, seed_base: int | None = None):
    """Return float32 (q, k, v) of shapes [B,S,H,d_qk], [B,S,H,d_qk], [B,S,H,d_v]."""
    base = 1000 * w.index if seed_base is None else seed_base
    out = []
    for which, D in ((0, w.d_qk), (1, w.d_qk), (2, w.d_v)):
        rng = np.random.default_rng(np.random.PCG64(base + which))
        out.append(_draw(rng, w.recipe, w.B, w.S, w.H, D))
    return tuple(out)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even, torch's cast) as uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def sample_rows(S: int, n: int = 256, seed: int = 12345) -> np.ndarray:
    """Query rows checked at long S: the first rows, tile and workgroup edges,
    the middle and the end, plus seeded uniform rows; sorted, unique."""
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 255, 256, S // 2 - 1, S // 2, S - 2, S - 1]
    rows = {r for r in fixed if 0 <= r < S}
    rng = np.random.default_rng(np.random.PCG64(seed))
    while len(rows) < min(n, S):
        rows.add(int(rng.integers(0, S)))
    return np.array(sorted(rows), dtype=np.int64)


# ------------------------------------------------------------------ decode
@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: B sequences each add one query token and attend to
    their cached keys, held in pages of page_size slots.  The 32 query heads on
    8 key/value heads of D1-D3 are the head layout of Mistral-7B and Qwen3-8B,
    two of the models the pages capture activations from; D4 and D5 have one
    key/value head per query head."""
    name: str
    index: int
    dtype: int
    B: int
    H_q: int
    H_kv: int
    d_qk: int
    d_v: int
    page_size: int
    lengths: str        # "uniform:L" or "lognormal:median:lo:hi"
    description: str

    def seq_lens(self) -> np.ndarray:
        kind, *a = self.lengths.split(":")
        if kind == "uniform":
            return np.full(self.B, int(a[0]), np.int32)
        med, lo, hi = (int(x) for x in a)
        rng = np.random.default_rng(np.random.PCG64(1000 * self.index + 7))
        x = np.exp(rng.standard_normal(self.B)) * med
        return np.clip(np.round(x), lo, hi).astype(np.int32)

    def block_table(self, lens: np.ndarray):
        """Pages of the sequences in a seeded random order over a pool with
        no free pages: (table [B, max pages], number of pages)."""
        need = (lens.astype(np.int64) + self.page_size - 1) // self.page_size
        total = int(need.sum())
        order = np.random.default_rng(np.random.PCG64(1000 * self.index + 8)).permutation(total)
        table = np.zeros((self.B, max(int(need.max()), 1)), np.int32)
        at = 0
        for b, n in enumerate(need):
            table[b, :n] = order[at:at + n]
            at += n
        return table, total


DECODE_WORKLOADS = {
    "D1": DecodeWorkload("D1", 20, BF16, 32, 32, 8, 128, 128, 64, "uniform:8192",
                         "BF16 decode, B=32 L=8192, H_q=32 on H_kv=8, d=128, pages of 64"),
    "D2": DecodeWorkload("D2", 21, FP8, 32, 32, 8, 128, 128, 64, "uniform:8192",
                         "FP8 e4m3 decode, B=32 L=8192, H_q=32 on H_kv=8, d=128, pages of 64"),
    "D3": DecodeWorkload("D3", 22, FP8, 64, 32, 8, 128, 128, 64, "lognormal:4096:64:32768",
                         "FP8 e4m3 decode, B=64 lognormal lengths (median 4096, 64..32768), "
                         "H_q=32 on H_kv=8, d=128, pages of 64"),
    "D4": DecodeWorkload("D4", 23, BF16, 16, 32, 32, 128, 128, 64, "uniform:16384",
                         "BF16 decode, B=16 L=16384, H_q=H_kv=32, d=128, pages of 64"),
    "D5": DecodeWorkload("D5", 24, FP8, 16, 32, 32, 128, 128, 64, "uniform:16384",
                         "FP8 e4m3 decode, B=16 L=16384, H_q=H_kv=32, d=128, pages of 64"),
}


def decode_device_inputs(w: DecodeWorkload, torch, device):
    """Device tensors (q, k_cache, v_cache, block_table, seq_lens) of a decode
    workload: N(0,1) values from a torch generator seeded with the workload
    index (bf16, or cast to e4m3 with descale 1), lengths and pages as above."""
    lens = w.seq_lens()
    table, pages = w.block_table(lens)
    g = torch.Generator(device=device)
    g.manual_seed(1000 * w.index)
    dt = torch.bfloat16 if w.dtype == BF16 else torch.float8_e4m3fn

    def draw(shape):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dt)
        return x if w.dtype == BF16 else x.view(torch.uint8)
    q = draw((w.B, w.H_q, w.d_qk))
    kc = draw((pages, w.page_size, w.H_kv, w.d_qk))
    vc = draw((pages, w.page_size, w.H_kv, w.d_v))
    return (q, kc, vc, torch.from_numpy(table).to(device),
            torch.from_numpy(lens).to(device))
