"""MI355X (gfx950) causal prefill attention forward: Python binding.

This module only marshals arguments to the C ABI declared in
``include/attn.h`` (``libcpattn.so``, built in-tree by ``_build.py``).  Every
step of the computation runs in the library's HIP kernels; PyTorch supplies
device memory and the current stream.  There is no fallback: if the library
is missing or was built without a usable GPU, calls raise.

The operation is causal forward (prefill) attention in FP8 e4m3 and BF16 at
head dimension 128 and in the MLA 192/128 shape behind a flash_attn_func
style call, as the ZYFA pages describe it ("TL;DR" on the acheiumaia.com.br
page; "Ce que couvrent les noyaux" on the ai-daily-news.org page).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "ATTN_DTYPE_BF16", "ATTN_DTYPE_FP8", "AttnError", "lib_path", "load_library",
    "attn_fwd", "attn_fwd_ex", "attn_fwd_balanced", "attn_fwd_varlen", "attn_amax_f32", "attn_quantize_e4m3",
    "attn_quantize_fp8", "attn_status_string",
    "attn_version", "attn_hadamard_f32", "attn_hadamard_bf16", "attn_hadamard_amax_f32",
    "attn_hadamard_quantize_e4m3", "attn_decode_paged", "attn_decode_paged_noalloc",
    "attn_decode_workspace_bytes", "ATTN_DECODE_SCRATCH_BYTES",
    "flash_attn_func", "flash_attn_varlen_func", "flash_attn_decode_paged", "quantize_fp8",
    "hadamard",
]

ATTN_DTYPE_BF16 = 0
ATTN_DTYPE_FP8 = 1
ATTN_DECODE_SCRATCH_BYTES = 32 << 20   # include/attn.h: the static scratch of the allocation-free decode

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcpattn.so")
_lib = None


class AttnError(ValueError):
    """A non-zero status from the C ABI."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: status %d (%s)" % (where, status, attn_status_string(status)))


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libcpattn.so (raises OSError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise OSError("libcpattn.so is not built; run __graft_entry__.build() or "
                      "python -m causal_prefill_attention_attn_amd._build")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.attn_version.restype = i32
    lib.attn_version.argtypes = []
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i32]
    lib.attn_fwd.restype = i32
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, f32, i32, i32,
                             f32, f32, f32, vp]
    lib.attn_fwd_ex.restype = i32
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, f32, i32, i32,
                                f32, f32, f32, ctypes.c_uint32, vp]
    lib.attn_fwd_balanced.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, f32, i32,
                                      i32, f32, f32, f32, ctypes.c_uint32, vp, vp]
    lib.attn_fwd_varlen.restype = i32
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32,
                                    i32, i32, f32, f32, f32, vp]
    lib.attn_amax_f32.restype = i32
    lib.attn_amax_f32.argtypes = [vp, i64, vp, vp]
    lib.attn_quantize_e4m3.restype = i32
    lib.attn_quantize_e4m3.argtypes = [vp, i64, f32, vp, vp]
    lib.attn_quantize_fp8.restype = i32
    lib.attn_quantize_fp8.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    lib.attn_hadamard_f32.restype = i32
    lib.attn_hadamard_f32.argtypes = [vp, i64, i32, vp, vp]
    lib.attn_hadamard_bf16.restype = i32
    lib.attn_hadamard_bf16.argtypes = [vp, i64, i32, vp, vp]
    lib.attn_hadamard_amax_f32.restype = i32
    lib.attn_hadamard_amax_f32.argtypes = [vp, i64, i32, vp, vp]
    lib.attn_hadamard_quantize_e4m3.restype = i32
    lib.attn_hadamard_quantize_e4m3.argtypes = [vp, i64, i32, f32, vp, vp]
    lib.attn_decode_paged.restype = i32
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                      i32, i64, i64, i64, i64, f32, i32, f32, f32, f32, vp]
    lib.attn_decode_paged_noalloc.restype = i32
    lib.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                              i64, i64, i64, i64, f32, i32, f32, f32, f32, vp]
    lib.attn_decode_workspace_bytes.restype = i64
    lib.attn_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    _lib = lib
    return lib


def attn_version() -> int:
    return int(load_library().attn_version())


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


# ----------------------------------------------------------- raw C-ABI calls
def attn_fwd(q, k, v, o, lse, B, S, H, d_qk, d_v, softmax_scale, causal, dtype,
             q_descale=1.0, k_descale=1.0, v_descale=1.0, stream=None) -> int:
    """Direct call of the C function on integer addresses; returns the status."""
    return int(load_library().attn_fwd(q, k, v, o, lse, B, S, H, d_qk, d_v, softmax_scale,
                                       causal, dtype, q_descale, k_descale, v_descale, stream))


def attn_fwd_ex(q, k, v, o, lse, B, S, H, d_qk, d_v, softmax_scale, causal, dtype,
                q_descale=1.0, k_descale=1.0, v_descale=1.0, flags=0, stream=None) -> int:
    return int(load_library().attn_fwd_ex(q, k, v, o, lse, B, S, H, d_qk, d_v, softmax_scale,
                                          causal, dtype, q_descale, k_descale, v_descale, flags,
                                          stream))


def attn_fwd_balanced(q, k, v, o, lse, B, S, H, d_qk, d_v, softmax_scale, causal, dtype,
                      q_descale=1.0, k_descale=1.0, v_descale=1.0, flags=0, counter=None,
                      stream=None) -> int:
    return int(load_library().attn_fwd_balanced(q, k, v, o, lse, B, S, H, d_qk, d_v,
                                                softmax_scale, causal, dtype, q_descale,
                                                k_descale, v_descale, flags, counter, stream))


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, n_seqs, total, max_seqlen, H, d_qk, d_v,
                    softmax_scale, causal, dtype, q_descale=1.0, k_descale=1.0, v_descale=1.0,
                    stream=None) -> int:
    return int(load_library().attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, n_seqs, total,
                                              max_seqlen, H, d_qk, d_v, softmax_scale, causal,
                                              dtype, q_descale, k_descale, v_descale, stream))


def attn_amax_f32(x, n, amax_out, stream=None) -> int:
    return int(load_library().attn_amax_f32(x, n, amax_out, stream))


def attn_quantize_e4m3(x, n, descale, out, stream=None) -> int:
    return int(load_library().attn_quantize_e4m3(x, n, descale, out, stream))


def attn_quantize_fp8(x, rows, d, rotate, codes, descale, stream=None) -> int:
    return int(load_library().attn_quantize_fp8(x, rows, d, rotate, codes, descale, stream))


def attn_hadamard_f32(x, rows, d, y, stream=None) -> int:
    return int(load_library().attn_hadamard_f32(x, rows, d, y, stream))


def attn_hadamard_bf16(x, rows, d, y, stream=None) -> int:
    return int(load_library().attn_hadamard_bf16(x, rows, d, y, stream))


def attn_hadamard_amax_f32(x, rows, d, amax_out, stream=None) -> int:
    return int(load_library().attn_hadamard_amax_f32(x, rows, d, amax_out, stream))


def attn_hadamard_quantize_e4m3(x, rows, d, descale, out, stream=None) -> int:
    return int(load_library().attn_hadamard_quantize_e4m3(x, rows, d, descale, out, stream))


# ------------------------------------------------------------ torch helpers
def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, workspace,
                      workspace_bytes, B, H_q, H_kv, d_qk, d_v, num_pages, page_size,
                      max_pages_per_seq, max_seqlen, softmax_scale, dtype, q_descale=1.0,
                      k_descale=1.0, v_descale=1.0, stream=None) -> int:
    return int(load_library().attn_decode_paged(
        q, k_cache, v_cache, block_table, seq_lens, o, lse, workspace, workspace_bytes, B, H_q,
        H_kv, d_qk, d_v, num_pages, page_size, max_pages_per_seq, max_seqlen, softmax_scale,
        dtype, q_descale, k_descale, v_descale, stream))


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, H_q, H_kv,
                              d_qk, d_v, num_pages, page_size, max_pages_per_seq, max_seqlen,
                              softmax_scale, dtype, q_descale=1.0, k_descale=1.0, v_descale=1.0,
                              stream=None) -> int:
    return int(load_library().attn_decode_paged_noalloc(
        q, k_cache, v_cache, block_table, seq_lens, o, lse, B, H_q, H_kv, d_qk, d_v, num_pages,
        page_size, max_pages_per_seq, max_seqlen, softmax_scale, dtype, q_descale, k_descale,
        v_descale, stream))


def attn_decode_workspace_bytes(B, H_q, H_kv, max_seqlen, d_v) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, H_q, H_kv, max_seqlen, d_v))


def _torch():
    import torch
    return torch


def _stream_handle(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise AttnError(status, where)


def _check_buffer(name, t, shape, dtype, device):
    """A caller-supplied output buffer must be exactly what the C function
    writes: the library cannot see buffer sizes, so a wrong one would be
    written out of bounds."""
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _element_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return ATTN_DTYPE_FP8
    raise TypeError("q, k, v must be bfloat16, float8_e4m3fn or uint8 (e4m3 codes), got %s"
                    % t.dtype)


def flash_attn_func(q, k, v, softmax_scale=None, causal=True, q_descale=1.0, k_descale=1.0,
                    v_descale=1.0, out=None, lse=None, return_lse=True, hadamard_o=False,
                    exact_p=False, balanced=True):
    """Forward attention on [B, S, H, D] tensors.

    q, k: [B, S, H, d_qk]; v: [B, S, H, d_v]; all bfloat16, or all FP8 e4m3
    (``torch.float8_e4m3fn`` or uint8 codes) with per-tensor descales.
    ``hadamard_o`` (FP8): rows of O are multiplied by the normalised Hadamard
    matrix, undoing a V rotated before quantization (``quantize_fp8(v,
    rotate=True)``).  ``exact_p`` (FP8): probabilities by exp2 and a rounding
    conversion instead of the lean form.  ``balanced`` (default): the call
    goes through attn_fwd_balanced with a one-word counter from torch's
    allocator, so that the shortest query blocks are shared among the XCDs
    as they free up (same results bit for bit); False calls attn_fwd_ex.
    Returns ``(o, lse)``: o bfloat16 [B, S, H, d_v], lse float32 [B, H, S]
    (natural log); lse is None when ``return_lse`` is False.
    """
    torch = _torch()
    dt = _element_dtype(q)
    if _element_dtype(k) != dt or _element_dtype(v) != dt:
        raise TypeError("q, k and v must share one element type")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous 4-D [B, S, H, D] CUDA tensor" % name)
    B, S, H, d_qk = q.shape
    d_v = v.shape[3]
    if tuple(k.shape) != (B, S, H, d_qk) or tuple(v.shape[:3]) != (B, S, H):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                             tuple(v.shape)))
    for name, t in (("k", k), ("v", v)):
        if t.device != q.device:
            raise ValueError("%s must be on %s, got %s" % (name, q.device, t.device))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_qk)
    if out is None:
        out = torch.empty((B, S, H, d_v), dtype=torch.bfloat16, device=q.device)
    _check_buffer("out", out, (B, S, H, d_v), torch.bfloat16, q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if not return_lse:
        lse = None
    if lse is not None:
        _check_buffer("lse", lse, (B, H, S), torch.float32, q.device)
    # a fresh word per call: torch's allocator orders its reuse on the stream
    counter = torch.empty((1,), dtype=torch.int32, device=q.device) if balanced else None
    st = attn_fwd_balanced(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr() if lse is not None else None, B, S, H, d_qk, d_v,
                           float(softmax_scale), int(bool(causal)), dt, float(q_descale),
                           float(k_descale), float(v_descale),
                           (1 if hadamard_o else 0) | (2 if exact_p else 0),
                           counter.data_ptr() if counter is not None else None,
                           _stream_handle(q.device))
    _check(st, "attn_fwd_balanced")
    return out, lse


def flash_attn_varlen_func(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None, causal=True,
                           q_descale=1.0, k_descale=1.0, v_descale=1.0, out=None, lse=None,
                           return_lse=True):
    """Forward attention on packed sequences: q, k [total, H, d_qk], v
    [total, H, d_v] (bfloat16, or FP8 e4m3 with per-tensor descales), with
    sequence s in rows cu_seqlens[s] .. cu_seqlens[s+1]-1 (int32 CUDA tensor
    of n_seqs + 1 prefix sums; max_seqlen the longest).  Returns ``(o, lse)``:
    o bfloat16 [total, H, d_v], lse float32 [H, total] or None."""
    torch = _torch()
    dt = _element_dtype(q)
    if _element_dtype(k) != dt or _element_dtype(v) != dt:
        raise TypeError("q, k and v must share one element type")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 3 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous 3-D [total, H, D] CUDA tensor" % name)
    if (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda
            or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 CUDA tensor")
    total, H, d_qk = q.shape
    d_v = v.shape[2]
    if tuple(k.shape) != (total, H, d_qk) or tuple(v.shape[:2]) != (total, H):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                             tuple(v.shape)))
    for name, t in (("k", k), ("v", v), ("cu_seqlens", cu_seqlens)):
        if t.device != q.device:
            raise ValueError("%s must be on %s, got %s" % (name, q.device, t.device))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_qk)
    if out is None:
        out = torch.empty((total, H, d_v), dtype=torch.bfloat16, device=q.device)
    _check_buffer("out", out, (total, H, d_v), torch.bfloat16, q.device)
    if return_lse and lse is None:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if not return_lse:
        lse = None
    if lse is not None:
        _check_buffer("lse", lse, (H, total), torch.float32, q.device)
    st = attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr() if lse is not None else None, cu_seqlens.data_ptr(),
                         cu_seqlens.numel() - 1, total, int(max_seqlen), H, d_qk, d_v,
                         float(softmax_scale), int(bool(causal)), dt, float(q_descale),
                         float(k_descale), float(v_descale), _stream_handle(q.device))
    _check(st, "attn_fwd_varlen")
    return out, lse


def flash_attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, max_seqlen,
                            softmax_scale=None, q_descale=1.0, k_descale=1.0, v_descale=1.0,
                            out=None, lse=None, workspace=None, return_lse=True):
    """One decode step against a paged KV cache.

    q [B, H_q, d_qk]; k_cache [pages, page_size, H_kv, d_qk]; v_cache
    [pages, page_size, H_kv, d_v] (bfloat16, or FP8 e4m3 with per-tensor
    descales); block_table [B, max_pages_per_seq] and seq_lens [B] int32 CUDA
    tensors; max_seqlen bounds every seq_lens entry.  Query head h reads
    key/value head h // (H_q // H_kv).  ``workspace``: a CUDA tensor of at
    least attn_decode_workspace_bytes(...) bytes, allocated here when None.
    Returns ``(o, lse)``: o bfloat16 [B, H_q, d_v], lse float32 [B, H_q] or
    None."""
    torch = _torch()
    dt = _element_dtype(q)
    if _element_dtype(k_cache) != dt or _element_dtype(v_cache) != dt:
        raise TypeError("q and the caches must share one element type")
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B, H_q, d_qk] and the caches [pages, page_size, H_kv, d]")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous CUDA tensor" % name)
    for name, t, nd in (("block_table", block_table, 2), ("seq_lens", seq_lens, 1)):
        if t.dtype != torch.int32 or t.dim() != nd:
            raise ValueError("%s must be a %d-D int32 tensor" % (name, nd))
    B, H_q, d_qk = q.shape
    pages, page_size, H_kv, _ = k_cache.shape
    d_v = v_cache.shape[3]
    if (tuple(k_cache.shape) != (pages, page_size, H_kv, d_qk)
            or tuple(v_cache.shape[:3]) != (pages, page_size, H_kv)
            or block_table.shape[0] != B or seq_lens.shape[0] != B):
        raise ValueError("shape mismatch: q %s k_cache %s v_cache %s block_table %s seq_lens %s"
                         % (tuple(q.shape), tuple(k_cache.shape), tuple(v_cache.shape),
                            tuple(block_table.shape), tuple(seq_lens.shape)))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
                    ("seq_lens", seq_lens)):
        if t.device != q.device:
            raise ValueError("%s must be on %s, got %s" % (name, q.device, t.device))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_qk)
    need = attn_decode_workspace_bytes(B, H_q, H_kv, int(max_seqlen), d_v)
    _check(need if need < 0 else 0, "attn_decode_workspace_bytes")
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or workspace.dtype != torch.uint8 or workspace.dim() != 1 \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor on %s" % q.device)
    if workspace.numel() < need:
        raise ValueError("workspace holds %d bytes, the call needs %d" % (workspace.numel(), need))
    if out is None:
        out = torch.empty((B, H_q, d_v), dtype=torch.bfloat16, device=q.device)
    _check_buffer("out", out, (B, H_q, d_v), torch.bfloat16, q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    if not return_lse:
        lse = None
    if lse is not None:
        _check_buffer("lse", lse, (B, H_q), torch.float32, q.device)
    st = attn_decode_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                           block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                           lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), B, H_q, H_kv, d_qk,
                           d_v, pages, page_size, block_table.shape[1], int(max_seqlen),
                           float(softmax_scale), dt, float(q_descale), float(k_descale),
                           float(v_descale), _stream_handle(q.device))
    _check(st, "attn_decode_paged")
    return out, lse


def quantize_fp8(x, rotate=False):
    """Per-tensor E4M3FN quantization on the GPU (attn_quantize_fp8): returns
    (codes uint8, descale), descale = amax / 448 in fp32 (1.0 for an
    all-zero tensor), both computed by the library on the device; the descale
    is then copied to the host for the attention call.  With ``rotate`` the
    rows of the last dimension (128 or 192) are rotated by the Hadamard matrix
    H first (as ``hadamard``), inside the quantization passes: the codes are
    those of x . H."""
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be a contiguous float32 CUDA tensor")
    d = x.shape[-1]
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    descale = torch.empty((1,), dtype=torch.float32, device=x.device)
    _check(attn_quantize_fp8(x.data_ptr(), x.numel() // max(d, 1), d, int(bool(rotate)),
                             codes.data_ptr(), descale.data_ptr(), _stream_handle(x.device)),
           "attn_quantize_fp8")
    return codes, float(descale.item())


def hadamard(x, out=None):
    """Rotate the last dimension (128 or 192) of a contiguous float32 or
    bfloat16 CUDA tensor by the normalized block Walsh-Hadamard matrix H:
    returns x . H (``out`` may be ``x`` for an in-place rotation).  H is its
    own inverse, so ``hadamard(hadamard(x))`` restores x up to rounding; the
    attention output of Q.H, K.H, V.H rotated once more is the attention of
    Q, K, V."""
    torch = _torch()
    if not x.is_cuda or not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be a contiguous CUDA tensor")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16, got %s" % x.dtype)
    d = x.shape[-1]
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must match x in shape, dtype and layout")
    fn = attn_hadamard_f32 if x.dtype == torch.float32 else attn_hadamard_bf16
    _check(fn(x.data_ptr(), x.numel() // d, d, out.data_ptr(), _stream_handle(x.device)),
           "attn_hadamard")
    return out
