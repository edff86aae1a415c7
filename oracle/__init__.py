"""CPU fp64 oracle for causal prefill attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path
(``causal_prefill_attention_attn_amd``) never imports it and shares no code
with it.

The attention arithmetic lives in ``attn_oracle.c`` (plain C, binary64,
OpenMP over query rows); this module builds that file with gcc and marshals
numpy arrays through ctypes.  See the header of ``attn_oracle.c`` for the
definition it computes and the passages of the pages it follows.  Two
functions are written here in numpy instead: the Hadamard rotation that may
precede FP8 quantization (``hadamard``), a plain fp64 matrix product per
block, and the decode step against a paged KV cache (``decode_paged``), a
gather of the sequence's keys followed by the textbook softmax in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "libattn_oracle.so")

BF16 = 0
FP8 = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile attn_oracle.c with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_bf16_decode.restype = ctypes.c_double
        lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_descale_amax.restype = ctypes.c_float
        lib.oracle_descale_amax.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        lib.oracle_quantize_e4m3.restype = None
        lib.oracle_quantize_e4m3.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                             ctypes.c_void_p]
        lib.oracle_attn.restype = ctypes.c_int
        lib.oracle_attn.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_float, ctypes.c_float, ctypes.c_float,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_attn_stats.restype = ctypes.c_int
        lib.oracle_attn_stats.argtypes = lib.oracle_attn.argtypes + [ctypes.c_void_p] * 3
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


_bf16_table = None


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, through a table of all 65536 patterns
    filled by the C decoder."""
    global _bf16_table
    if _bf16_table is None:
        lib = _load()
        _bf16_table = np.array([lib.oracle_bf16_decode(b) for b in range(65536)], np.float64)
    return _bf16_table[np.asarray(bits, dtype=np.uint16)]


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    lib = _load()
    table = np.array([lib.oracle_e4m3_decode(c) for c in range(256)], np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3_scalar(x: float) -> int:
    return int(_load().oracle_e4m3_encode(float(np.float32(x))))


def descale_amax(x: np.ndarray) -> float:
    a = np.ascontiguousarray(x, dtype=np.float32)
    return float(_load().oracle_descale_amax(_ptr(a), a.size))


def quantize_e4m3(x: np.ndarray, descale: float) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().oracle_quantize_e4m3(_ptr(a), a.size, ctypes.c_float(descale), _ptr(out))
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, dtype: int, tau: float,
              causal: bool = True, rows=None, q_descale: float = 1.0, k_descale: float = 1.0,
              v_descale: float = 1.0, stats: bool = False):
    """fp64 attention on raw element encodings.

    q, k: [B,S,H,d_qk]; v: [B,S,H,d_v]; uint16 bf16 bit patterns (dtype BF16)
    or uint8 E4M3 codes (dtype FP8).  ``rows``: query rows to evaluate (all
    when None).  Returns (o [B,len(rows),H,d_v], lse [B,H,len(rows)]) float64,
    and with ``stats`` a third item: a dict of per-row arrays [B,H,len(rows)]
    ``kappa`` (sensitivity of the row to relative errors of its
    probabilities), ``wmax`` (softmax mass at the row maximum) and ``sabs``
    (softmax-weighted mean over keys of tau times the sum of |q_c k_c|), as
    defined in attn_oracle.c.
    """
    lib = _load()
    want = np.uint16 if dtype == BF16 else np.uint8
    q = np.ascontiguousarray(q, dtype=want)
    k = np.ascontiguousarray(k, dtype=want)
    v = np.ascontiguousarray(v, dtype=want)
    B, S, H, dqk = q.shape
    dv = v.shape[3]
    assert k.shape == (B, S, H, dqk) and v.shape[:3] == (B, S, H)
    rows = np.arange(S, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    o = np.empty((B, rows.size, H, dv), np.float64)
    lse = np.empty((B, H, rows.size), np.float64)
    st = {n: np.empty((B, H, rows.size), np.float64) for n in ("kappa", "wmax", "sabs")} \
        if stats else None
    extra = [_ptr(st[n]) for n in ("kappa", "wmax", "sabs")] if stats else [None] * 3
    rc = lib.oracle_attn_stats(_ptr(q), _ptr(k), _ptr(v), dtype, q_descale, k_descale,
                               v_descale, B, S, H, dqk, dv, float(tau), int(bool(causal)),
                               _ptr(rows), rows.size, _ptr(o), _ptr(lse), *extra)
    if rc != 0:
        raise ValueError("oracle_attn rejected its arguments")
    return (o, lse, st) if stats else (o, lse)


def decode_paged(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_table: np.ndarray, seq_lens: np.ndarray, dtype: int, tau: float,
                 q_descale: float = 1.0, k_descale: float = 1.0, v_descale: float = 1.0):
    """fp64 decode step against a paged KV cache: one new query token per
    sequence attends to every cached key of its sequence.

    Decode and paged KV caches are listed among the kernels' future work in
    "Ce que couvrent les noyaux" on the ai-daily-news.org page; the step is
    the last row of causal attention, so the definition is the textbook one,
    o = softmax(tau * q.K^T) V and lse = log sum exp(tau * q.K^T), over the
    sequence's keys 0 .. L-1 (the new token's own key and value are already
    in the cache).  Readings: key j of sequence b sits in page
    block_table[b, j // page_size], slot j % page_size; query head h reads
    key/value head h // (H_q / H_kv); an empty sequence gives o = 0 and
    lse = -inf.

    q: [B, H_q, d_qk]; k_cache: [pages, page_size, H_kv, d_qk];
    v_cache: [pages, page_size, H_kv, d_v]; raw encodings (uint16 bf16 bit
    patterns for BF16, uint8 E4M3 codes for FP8) times their descales.
    Returns (o [B, H_q, d_v], lse [B, H_q]) float64.
    """
    dec = decode_bf16 if dtype == BF16 else decode_e4m3
    B, hq, dqk = q.shape
    pages, ps, hkv, _ = k_cache.shape
    dv = v_cache.shape[3]
    assert hq % hkv == 0 and v_cache.shape[:3] == (pages, ps, hkv)
    group = hq // hkv
    qf = dec(q) * q_descale
    o = np.zeros((B, hq, dv), np.float64)
    lse = np.full((B, hq), -np.inf, np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        j = np.arange(n)
        page = np.asarray(block_table[b], np.int64)[j // ps]
        kb = dec(k_cache[page, j % ps]) * k_descale        # [n, H_kv, d_qk]
        vb = dec(v_cache[page, j % ps]) * v_descale        # [n, H_kv, d_v]
        for h in range(hq):
            s = tau * (kb[:, h // group, :] @ qf[b, h])
            m = s.max()
            e = np.exp(s - m)
            o[b, h] = (e @ vb[:, h // group, :]) / e.sum()
            lse[b, h] = m + np.log(e.sum())
    return o, lse


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def hadamard_matrix(n: int) -> np.ndarray:
    """Normalized Sylvester-Hadamard matrix of order n (a power of two), fp64:
    H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]], scaled by 1/sqrt(n).  The
    rotation of Q, K and V before FP8 quantization ("Precisao, estabilidade
    e efeito na pratica" on the miraibroadcast.com page) uses this matrix;
    the pages name the transform but not its order or normalization, so the
    plainest orthogonal reading is taken."""
    assert n >= 1 and n & (n - 1) == 0
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(n)


def hadamard_block(d: int) -> int:
    """Block order of the row rotation: 128 for rows of 128, 64 for 192."""
    return {128: 128, 192: 64}[d]


def hadamard(x: np.ndarray) -> np.ndarray:
    """x . H over the last dimension d in {128, 192}, in fp64, with H
    block-diagonal of normalized Sylvester-Hadamard blocks (one of 128, or
    three of 64): a plain matrix product per block."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    n = hadamard_block(d)
    h = hadamard_matrix(n)
    blocks = x.reshape(x.shape[:-1] + (d // n, n))
    return (blocks @ h).reshape(x.shape)
