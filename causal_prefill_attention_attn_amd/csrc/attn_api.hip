// C-ABI front end: argument validation (host only, before any HIP call),
// instance selection and launch.  The declarations and their contract are in
// include/attn.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "attn_kernels.h"

namespace {

bool finite_positive(float x) { return isfinite(x) && x > 0.0f; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// half-open byte ranges [p, p + n) overlap
bool overlap(const void* p, int64_t np, const void* q, int64_t nq) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + (uintptr_t)nq && b < a + (uintptr_t)np;
}

}  // namespace

extern "C" {

int attn_version(void) { return 200; }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, S and H must be >= 1 and the problem must fit 32-bit grid indexing";
    case ATTN_ERR_DTYPE: return "dtype must be ATTN_DTYPE_BF16 (0) or ATTN_DTYPE_FP8 (1)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported (d_qk, d_v) (want (128,128) or (192,128)) or causal not 0/1";
    case ATTN_ERR_SCALE: return "softmax_scale and the FP8 descales must be finite and > 0";
    case ATTN_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned; lse, cu_seqlens and the counter 4-byte aligned";
    case ATTN_ERR_ALIAS: return "o, lse or the counter overlaps an input or another output";
    case ATTN_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    case ATTN_ERR_WORKSPACE: return "workspace smaller than attn_decode_workspace_bytes";
    case ATTN_ERR_SCRATCH: return "the step needs more than the library's static decode scratch (ATTN_DECODE_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Shared validation and launch of attn_fwd (cu null: B dense problems of S
// rows, total = B*S) and attn_fwd_varlen (B packed sequences bounded by cu,
// S the longest, total rows).
int fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu,
        int64_t total, int64_t B, int64_t S, int64_t H, int d_qk, int d_v, float softmax_scale,
        int causal, int dtype, float q_descale, float k_descale, float v_descale, unsigned flags,
        int32_t* counter, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B < 1 || S < 1 || H < 1 || total < 1) return ATTN_ERR_SHAPE;
  // 32-bit indices inside the kernels: rows, heads, problem*head and the grid
  if (S > INT32_MAX || H > INT32_MAX || B >= INT32_MAX || B * H > INT32_MAX) return ATTN_ERR_SHAPE;
  if (total > INT64_MAX / (H * 256)) return ATTN_ERR_SHAPE;
  const int64_t nqb = (S + 127) / 128;
  if (nqb * B * H > INT32_MAX) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP8) return ATTN_ERR_DTYPE;
  if (!((d_qk == 128 || d_qk == 192) && d_v == 128) || (causal != 0 && causal != 1))
    return ATTN_ERR_UNSUPPORTED;
  if ((flags & ~(ATTN_FLAG_HADAMARD_O | ATTN_FLAG_EXACT_P)) != 0 ||
      (flags != 0 && dtype != ATTN_DTYPE_FP8))
    return ATTN_ERR_UNSUPPORTED;
  if (!finite_positive(softmax_scale)) return ATTN_ERR_SCALE;
  if (dtype == ATTN_DTYPE_FP8 &&
      !(finite_positive(q_descale) && finite_positive(k_descale) && finite_positive(v_descale)))
    return ATTN_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)) || (cu && !aligned(cu, 4)) || (counter && !aligned(counter, 4)))
    return ATTN_ERR_ALIGN;
  const int64_t esz = dtype == ATTN_DTYPE_BF16 ? 2 : 1;
  // the kernels address one problem of q/k/v with 32-bit byte offsets (plus
  // a tile of slack past the last row)
  if ((S + 256) * H * d_qk * esz >= ((int64_t)1 << 32)) return ATTN_ERR_SHAPE;
  const int64_t rows = total * H;
  const int64_t nq = rows * d_qk * esz, nv = rows * d_v * esz, no = rows * d_v * 2;
  const int64_t nl = total * H * 4;
  if (overlap(o, no, q, nq) || overlap(o, no, k, nq) || overlap(o, no, v, nv)) return ATTN_ERR_ALIAS;
  if (lse && (overlap(lse, nl, q, nq) || overlap(lse, nl, k, nq) || overlap(lse, nl, v, nv) ||
              overlap(lse, nl, o, no)))
    return ATTN_ERR_ALIAS;
  if (cu && (overlap(cu, (B + 1) * 4, o, no) || (lse && overlap(cu, (B + 1) * 4, lse, nl))))
    return ATTN_ERR_ALIAS;
  if (counter && (overlap(counter, 4, q, nq) || overlap(counter, 4, k, nq) ||
                  overlap(counter, 4, v, nv) || overlap(counter, 4, o, no) ||
                  (lse && overlap(counter, 4, lse, nl))))
    return ATTN_ERR_ALIAS;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int rc;
  if (dtype == ATTN_DTYPE_BF16)
    rc = cpattn::launch_attn_bf16(q, k, v, o, lse, cu, total, (int)B, (int)S, (int)H, d_qk,
                                  softmax_scale, causal, counter, st);
  else
    rc = cpattn::launch_attn_fp8(q, k, v, o, lse, cu, total, (int)B, (int)S, (int)H, d_qk,
                                 softmax_scale, causal, q_descale, k_descale, v_descale,
                                 (flags & ATTN_FLAG_HADAMARD_O) != 0,
                                 (flags & ATTN_FLAG_EXACT_P) != 0, counter, st);
  return rc == 0 ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
             int64_t S, int64_t H, int d_qk, int d_v, float softmax_scale, int causal, int dtype,
             float q_descale, float k_descale, float v_descale, void* stream) {
  if (B >= 1 && S >= 1 && B > INT64_MAX / S) return ATTN_ERR_SHAPE;
  return fwd(q, k, v, o, lse, nullptr, B >= 1 && S >= 1 ? B * S : 0, B, S, H, d_qk, d_v,
             softmax_scale, causal, dtype, q_descale, k_descale, v_descale, 0u, nullptr, stream);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                int64_t S, int64_t H, int d_qk, int d_v, float softmax_scale, int causal,
                int dtype, float q_descale, float k_descale, float v_descale, unsigned flags,
                void* stream) {
  if (B >= 1 && S >= 1 && B > INT64_MAX / S) return ATTN_ERR_SHAPE;
  return fwd(q, k, v, o, lse, nullptr, B >= 1 && S >= 1 ? B * S : 0, B, S, H, d_qk, d_v,
             softmax_scale, causal, dtype, q_descale, k_descale, v_descale, flags, nullptr,
             stream);
}

int attn_fwd_balanced(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t S, int64_t H, int d_qk, int d_v, float softmax_scale,
                      int causal, int dtype, float q_descale, float k_descale, float v_descale,
                      unsigned flags, int32_t* counter, void* stream) {
  if (B >= 1 && S >= 1 && B > INT64_MAX / S) return ATTN_ERR_SHAPE;
  return fwd(q, k, v, o, lse, nullptr, B >= 1 && S >= 1 ? B * S : 0, B, S, H, d_qk, d_v,
             softmax_scale, causal, dtype, q_descale, k_descale, v_descale, flags, counter,
             stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int64_t n_seqs, int64_t total, int64_t max_seqlen,
                    int64_t H, int d_qk, int d_v, float softmax_scale, int causal, int dtype,
                    float q_descale, float k_descale, float v_descale, void* stream) {
  if (!cu_seqlens) return ATTN_ERR_NULL;
  return fwd(q, k, v, o, lse, cu_seqlens, total, n_seqs, max_seqlen, H, d_qk, d_v,
             softmax_scale, causal, dtype, q_descale, k_descale, v_descale, 0u, nullptr, stream);
}

int attn_amax_f32(const float* x, int64_t n, float* amax_out, void* stream) {
  if (!x || !amax_out) return ATTN_ERR_NULL;
  if (n < 1) return ATTN_ERR_SHAPE;
  if (!aligned(x, 4) || !aligned(amax_out, 4)) return ATTN_ERR_ALIGN;
  if (overlap(amax_out, 4, x, n * 4)) return ATTN_ERR_ALIAS;
  return cpattn::launch_amax_f32(x, n, amax_out, reinterpret_cast<hipStream_t>(stream)) == 0
             ? ATTN_OK
             : ATTN_ERR_LAUNCH;
}

int attn_quantize_e4m3(const float* x, int64_t n, float descale, uint8_t* out, void* stream) {
  if (!x || !out) return ATTN_ERR_NULL;
  if (n < 1) return ATTN_ERR_SHAPE;
  if (!finite_positive(descale)) return ATTN_ERR_SCALE;
  if (!aligned(x, 4)) return ATTN_ERR_ALIGN;
  if (overlap(out, n, x, n * 4)) return ATTN_ERR_ALIAS;
  return cpattn::launch_quantize_e4m3(x, n, descale, out, reinterpret_cast<hipStream_t>(stream)) == 0
             ? ATTN_OK
             : ATTN_ERR_LAUNCH;
}

int attn_quantize_fp8(const float* x, int64_t rows, int d, int rotate, uint8_t* codes,
                      float* descale, void* stream) {
  if (!x || !codes || !descale) return ATTN_ERR_NULL;
  if (rows < 1 || d < 1 || rows > INT64_MAX / ((int64_t)d * 4)) return ATTN_ERR_SHAPE;
  if (rotate != 0 && rotate != 1) return ATTN_ERR_UNSUPPORTED;
  if (rotate && d != 128 && d != 192) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 4) || !aligned(descale, 4)) return ATTN_ERR_ALIGN;
  const int64_t n = rows * d;
  if (overlap(codes, n, x, n * 4) || overlap(descale, 4, x, n * 4) || overlap(descale, 4, codes, n))
    return ATTN_ERR_ALIAS;
  return cpattn::launch_quantize_fp8(x, rows, d, rotate != 0, codes, descale,
                                     reinterpret_cast<hipStream_t>(stream)) == 0
             ? ATTN_OK
             : ATTN_ERR_LAUNCH;
}

}  // extern "C"

namespace {

int hadamard(const void* x, int64_t rows, int d, void* y, int esz, void* stream) {
  if (!x || !y) return ATTN_ERR_NULL;
  if (rows < 1) return ATTN_ERR_SHAPE;
  if (d != 128 && d != 192) return ATTN_ERR_UNSUPPORTED;
  if (rows > INT64_MAX / ((int64_t)d * esz)) return ATTN_ERR_SHAPE;
  if (!aligned(x, esz) || !aligned(y, esz)) return ATTN_ERR_ALIGN;
  const int64_t n = rows * d * esz;
  if (x != y && overlap(x, n, y, n)) return ATTN_ERR_ALIAS;
  return cpattn::launch_hadamard(x, rows, d, esz == 2, y, reinterpret_cast<hipStream_t>(stream)) == 0
             ? ATTN_OK
             : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_hadamard_f32(const float* x, int64_t rows, int d, float* y, void* stream) {
  return hadamard(x, rows, d, y, 4, stream);
}

int attn_hadamard_bf16(const void* x, int64_t rows, int d, void* y, void* stream) {
  return hadamard(x, rows, d, y, 2, stream);
}

int attn_hadamard_amax_f32(const float* x, int64_t rows, int d, float* amax_out, void* stream) {
  if (!x || !amax_out) return ATTN_ERR_NULL;
  if (rows < 1) return ATTN_ERR_SHAPE;
  if (d != 128 && d != 192) return ATTN_ERR_UNSUPPORTED;
  if (rows > INT64_MAX / ((int64_t)d * 4)) return ATTN_ERR_SHAPE;
  if (!aligned(x, 4) || !aligned(amax_out, 4)) return ATTN_ERR_ALIGN;
  if (overlap(amax_out, 4, x, rows * d * 4)) return ATTN_ERR_ALIAS;
  return cpattn::launch_hadamard_amax(x, rows, d, amax_out,
                                      reinterpret_cast<hipStream_t>(stream)) == 0
             ? ATTN_OK
             : ATTN_ERR_LAUNCH;
}

int attn_hadamard_quantize_e4m3(const float* x, int64_t rows, int d, float descale, uint8_t* out,
                                void* stream) {
  if (!x || !out) return ATTN_ERR_NULL;
  if (rows < 1) return ATTN_ERR_SHAPE;
  if (d != 128 && d != 192) return ATTN_ERR_UNSUPPORTED;
  if (rows > INT64_MAX / ((int64_t)d * 4)) return ATTN_ERR_SHAPE;
  if (!finite_positive(descale)) return ATTN_ERR_SCALE;
  if (!aligned(x, 4)) return ATTN_ERR_ALIGN;
  if (overlap(out, rows * d, x, rows * d * 4)) return ATTN_ERR_ALIAS;
  return cpattn::launch_hadamard_quantize(x, rows, d, descale, out,
                                          reinterpret_cast<hipStream_t>(stream)) == 0
             ? ATTN_OK
             : ATTN_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Sizes of attn_decode_paged that do not involve buffers.
int decode_sizes(int64_t B, int64_t H_q, int64_t H_kv, int64_t max_seqlen, int d_v) {
  if (B < 1 || B > 65535 || H_kv < 1 || H_kv > 65535 || H_q < 1 || max_seqlen < 1 ||
      max_seqlen >= ((int64_t)1 << 30))
    return ATTN_ERR_SHAPE;
  if (H_q % H_kv != 0 || B * H_q > INT32_MAX) return ATTN_ERR_SHAPE;
  const int64_t g = H_q / H_kv;
  if (!(g == 1 || g == 2 || g == 4 || g == 8) || d_v != 128) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int64_t attn_decode_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t max_seqlen,
                                    int d_v) {
  const int rc = decode_sizes(B, H_q, H_kv, max_seqlen, d_v);
  if (rc != ATTN_OK) return rc;
  return cpattn::decode_workspace_bytes(B, H_q, H_kv, max_seqlen);
}

}  // extern "C"

namespace {

// Validation and launch shared by attn_decode_paged (caller's workspace) and
// attn_decode_paged_noalloc (workspace null: the library's static scratch).
int decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
           const int32_t* seq_lens, void* o, float* lse, void* workspace, int64_t workspace_bytes,
           int64_t B, int64_t H_q, int64_t H_kv, int d_qk, int d_v, int64_t num_pages,
           int64_t page_size, int64_t max_pages_per_seq, int64_t max_seqlen,
           float softmax_scale, int dtype, float q_descale, float k_descale, float v_descale,
           void* stream) {
  const bool own = workspace == nullptr;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o) return ATTN_ERR_NULL;
  int rc = decode_sizes(B, H_q, H_kv, max_seqlen, d_v);
  if (rc != ATTN_OK) return rc;
  if (page_size < 16 || page_size > ((int64_t)1 << 20) || (page_size & (page_size - 1)) != 0 ||
      num_pages < 1 || num_pages > INT32_MAX || max_pages_per_seq < 1 ||
      max_pages_per_seq > INT32_MAX || max_seqlen > max_pages_per_seq * page_size ||
      B * max_pages_per_seq > ((int64_t)1 << 40))
    return ATTN_ERR_SHAPE;
  if (num_pages > INT64_MAX / (page_size * H_kv * 192 * 2)) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP8) return ATTN_ERR_DTYPE;
  if (d_qk != 128 && d_qk != 192) return ATTN_ERR_UNSUPPORTED;
  if (!finite_positive(softmax_scale)) return ATTN_ERR_SCALE;
  if (dtype == ATTN_DTYPE_FP8 &&
      !(finite_positive(q_descale) && finite_positive(k_descale) && finite_positive(v_descale)))
    return ATTN_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)) ||
      !aligned(workspace, 16))
    return ATTN_ERR_ALIGN;
  const int64_t need = cpattn::decode_workspace_bytes(B, H_q, H_kv, max_seqlen);
  if (own && need > cpattn::kDecodeScratchBytes) return ATTN_ERR_SCRATCH;
  if (!own && workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  const int64_t esz = dtype == ATTN_DTYPE_BF16 ? 2 : 1;
  const int64_t nq = B * H_q * d_qk * esz;
  const int64_t nk = num_pages * page_size * H_kv * d_qk * esz;
  const int64_t nv = num_pages * page_size * H_kv * d_v * esz;
  const int64_t nt = B * max_pages_per_seq * 4, nl = B * 4;
  const int64_t no = B * H_q * d_v * 2, nlse = B * H_q * 4;
  struct Buf { const void* p; int64_t n; };
  const Buf inputs[] = {{q, nq}, {k_cache, nk}, {v_cache, nv}, {block_table, nt}, {seq_lens, nl}};
  const Buf outputs[] = {{o, no}, {lse, nlse}, {workspace, need}};
  for (const Buf& out : outputs) {
    if (!out.p) continue;
    for (const Buf& in : inputs)
      if (overlap(out.p, out.n, in.p, in.n)) return ATTN_ERR_ALIAS;
  }
  if ((lse && overlap(o, no, lse, nlse)) || (!own && overlap(o, no, workspace, need)) ||
      (lse && !own && overlap(lse, nlse, workspace, need)))
    return ATTN_ERR_ALIAS;

  if (own) {
    workspace = cpattn::decode_scratch();
    if (workspace == nullptr) return ATTN_ERR_LAUNCH;
  }
  cpattn::DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.workspace = workspace;
  a.B = B;
  a.Hq = H_q;
  a.Hkv = H_kv;
  a.d_qk = d_qk;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.max_pages_per_seq = max_pages_per_seq;
  a.max_seqlen = max_seqlen;
  a.softmax_scale = softmax_scale;
  a.dtype_fp8 = dtype == ATTN_DTYPE_FP8;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  cpattn::decode_launch_policy(a, &a.split, &a.nsplit);
  rc = cpattn::launch_decode(a, reinterpret_cast<hipStream_t>(stream));
  return rc == 0 ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                      void* workspace, int64_t workspace_bytes, int64_t B, int64_t H_q,
                      int64_t H_kv, int d_qk, int d_v, int64_t num_pages, int64_t page_size,
                      int64_t max_pages_per_seq, int64_t max_seqlen, float softmax_scale,
                      int dtype, float q_descale, float k_descale, float v_descale,
                      void* stream) {
  if (!workspace) return ATTN_ERR_NULL;
  return decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, workspace, workspace_bytes,
                B, H_q, H_kv, d_qk, d_v, num_pages, page_size, max_pages_per_seq, max_seqlen,
                softmax_scale, dtype, q_descale, k_descale, v_descale, stream);
}

int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* o,
                              float* lse, int64_t B, int64_t H_q, int64_t H_kv, int d_qk, int d_v,
                              int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                              int64_t max_seqlen, float softmax_scale, int dtype, float q_descale,
                              float k_descale, float v_descale, void* stream) {
  return decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, nullptr, 0, B, H_q, H_kv,
                d_qk, d_v, num_pages, page_size, max_pages_per_seq, max_seqlen, softmax_scale,
                dtype, q_descale, k_descale, v_descale, stream);
}

}  // extern "C"
