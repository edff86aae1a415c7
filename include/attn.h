/*
 * attn.h -- C ABI of the MI355X (gfx950) causal prefill attention library.
 *
 * One forward operation:
 *
 *   O = softmax(tau * Q K^T + causal mask) V,     lse_i = log sum_j exp(s_ij)
 *
 * in BF16 or FP8 (OCP E4M3FN) inputs, for head dimension 128 and for the
 * DeepSeek-V2 latent-attention shape (QK dimension 192, V dimension 128).
 *
 * Source of the operation: the ZYFA announcement pages describe causal
 * forward (prefill) attention kernels in FP8 e4m3 and BF16 at head dimension
 * 128 and in the MLA 192/128 shape, exposed through a flash_attn_func style
 * call ("TL;DR" and "O que e o ZYFA?" on the acheiumaia.com.br page; "Ce que
 * couvrent les noyaux" on the ai-daily-news.org page), whose core is the two
 * matrix products Q.K^T and P.V with a softmax between them ("Por que a
 * atencao FP8 tem desempenho inferior no MI355X?" on the acheiumaia.com.br
 * page).  The pages print no formula; the one above is the textbook
 * definition of softmax attention with a causal mask.
 *
 * Conventions shared by every entry point:
 *   - Pointers marked "device" must be device memory (hipMalloc or a torch
 *     CUDA tensor); the caller owns every buffer.  The library allocates no
 *     device memory and keeps no mutable global state; calls are re-entrant.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it and the call returns without synchronizing; a return of
 *     ATTN_OK means "validated and enqueued".
 *   - Every argument check happens on the host before any HIP call.  A
 *     negative return means nothing was enqueued and no memory was touched.
 */
#ifndef CPATTN_ATTN_H
#define CPATTN_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ATTN_OK 0
#define ATTN_ERR_NULL (-1)        /* a required pointer is NULL */
#define ATTN_ERR_SHAPE (-2)       /* B, S or H < 1, or a size exceeds the 32-bit limits */
#define ATTN_ERR_DTYPE (-3)       /* dtype is not ATTN_DTYPE_BF16 / ATTN_DTYPE_FP8 */
#define ATTN_ERR_UNSUPPORTED (-4) /* (d_qk, d_v) not in {(128,128), (192,128)}, or causal not 0/1 */
#define ATTN_ERR_SCALE (-5)       /* softmax_scale or a descale not finite and > 0 */
#define ATTN_ERR_ALIGN (-6)       /* q/k/v/o not 16-byte aligned, or lse not 4-byte aligned */
#define ATTN_ERR_ALIAS (-7)       /* an output buffer overlaps an input or the other output */
#define ATTN_ERR_LAUNCH (-8)      /* the HIP runtime rejected the kernel launch */
#define ATTN_ERR_WORKSPACE (-9)   /* workspace smaller than attn_decode_workspace_bytes */
#define ATTN_ERR_SCRATCH (-10)    /* attn_decode_paged_noalloc: step needs more than
                                     ATTN_DECODE_SCRATCH_BYTES of scratch */

/* Size of the library's static per-GPU scratch used by attn_decode_paged_noalloc. */
#define ATTN_DECODE_SCRATCH_BYTES (32ll << 20)

/* flags of attn_fwd_ex */
#define ATTN_FLAG_HADAMARD_O 1u /* O rows times the normalised Hadamard matrix (FP8 only) */
#define ATTN_FLAG_EXACT_P 2u    /* FP8 probabilities by exp2 + rounding conversion */

/* element types of q, k, v */
#define ATTN_DTYPE_BF16 0 /* bfloat16 */
#define ATTN_DTYPE_FP8 1  /* OCP FP8 E4M3FN (bias 7, max 448, no inf) */

/* Library version, major*10000 + minor*100 + patch. */
int attn_version(void);

/* Static description of a status code (never NULL). */
const char* attn_status_string(int status);

/*
 * attn_fwd -- causal (or full) softmax attention, forward only.
 *
 * Operation (one independent problem per batch b and head h):
 *   qhat = q            (BF16)     or  decode_e4m3(q) * q_descale   (FP8)
 *   khat, vhat likewise with k_descale, v_descale
 *   s_ij  = softmax_scale * <qhat[b,i,h,:], khat[b,j,h,:]>
 *   key j is visible from query i iff (causal ? j <= i : 1)
 *   o[b,i,h,:]  = sum_visible softmax_j(s_ij) * vhat[b,j,h,:]   (rounded to bf16)
 *   lse[b,h,i]  = ln sum_visible exp(s_ij)                      (fp32)
 * The FP8 path rounds the probabilities to E4M3 before the P.V product,
 * after scaling each 64-key block of a row by a power of two, and removes
 * the factor inside the scaled matrix instruction (the block-scaling
 * technique in "Como o motor de atencao FP8 da Zyphra funciona" on the
 * miraibroadcast.com page); the row sum uses the rounded probabilities.
 *
 * Arguments:
 *   q    device, [B, S, H, d_qk] contiguous, bf16 or e4m3 codes
 *   k    device, [B, S, H, d_qk] contiguous, same type as q
 *   v    device, [B, S, H, d_v]  contiguous, same type as q
 *   o    device, [B, S, H, d_v]  contiguous, bf16 (written)
 *   lse  device, [B, H, S] contiguous, fp32 natural-log LSE (written);
 *        may be NULL to skip it
 *   B, S, H        >= 1 (S need not be a multiple of any tile size)
 *   d_qk, d_v      (128, 128) or (192, 128)
 *   softmax_scale  tau, finite and > 0 (callers usually pass 1/sqrt(d_qk))
 *   causal         1 = causal mask (j <= i), 0 = no mask
 *   dtype          ATTN_DTYPE_BF16 or ATTN_DTYPE_FP8
 *   q/k/v_descale  FP8 only: per-tensor dequantization factors, finite and
 *                  > 0 (ignored for BF16)
 *   stream         hipStream_t or NULL
 * q, k, v, o must be 16-byte aligned and lse 4-byte aligned; o and lse must
 * not overlap q, k, v or each other.  One batch of q/k (S*H*d_qk elements)
 * must stay below 4 GiB (the kernels use 32-bit offsets within a batch);
 * larger problems return ATTN_ERR_SHAPE.  Inputs holding NaN (or inf) give
 * unspecified outputs.  Repeated calls on the same inputs give bitwise
 * identical o and lse (no atomics, fixed reduction order).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
             int64_t S, int64_t H, int d_qk, int d_v, float softmax_scale, int causal, int dtype,
             float q_descale, float k_descale, float v_descale, void* stream);

/*
 * attn_fwd_ex -- attn_fwd with option flags.
 *   flags  0, or ATTN_FLAG_HADAMARD_O: each row of O (d_v = 128 values) is
 *          multiplied by the normalised Sylvester-Hadamard matrix of order
 *          128 before it is rounded to bf16.  This undoes a V whose rows were
 *          rotated by that matrix before FP8 quantization (attn_hadamard_*),
 *          the rotation that "Precisao, estabilidade e efeito na pratica" on
 *          the miraibroadcast.com page credits with about half of the FP8
 *          error, without a separate pass over O.  FP8 only.
 *          ATTN_FLAG_EXACT_P: each probability is computed as exp2 and
 *          rounded to e4m3 by the hardware conversion, instead of the default
 *          "lean" form (one multiply-add and an integer conversion giving the
 *          e4m3 bit pattern of 2^y directly, "Como o motor de atencao FP8 da
 *          Zyphra funciona" on the miraibroadcast.com page).  FP8 only.
 * Every other argument, check and return code is that of attn_fwd; unknown
 * flag bits, or any flag with BF16, return ATTN_ERR_UNSUPPORTED.
 * With flags = 0 the results equal those of attn_fwd bit for bit.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                int64_t S, int64_t H, int d_qk, int d_v, float softmax_scale, int causal,
                int dtype, float q_descale, float k_descale, float v_descale, unsigned flags,
                void* stream);

/*
 * attn_fwd_balanced -- attn_fwd_ex whose last part of the work is shared
 * among the chip's eight XCDs as they free up.  The operation is the one
 * the pages state for the kernels (causal prefill attention over query and
 * key blocks, "Como o motor de atencao FP8 da Zyphra funciona" on the
 * miraibroadcast.com page); only the assignment of query blocks to
 * workgroups differs.
 *   counter  device, one int32 the call uses to hand out the shortest query
 *            blocks (4-byte aligned, not overlapping q, k, v, o or lse); the
 *            call clears it with a kernel on `stream` before the attention
 *            kernel, so its contents on entry do not matter and no host-side
 *            clear is needed (the pair can be captured in a HIP graph).
 *            Calls that may run at the same time (on different streams)
 *            must not share a counter.  NULL: same as attn_fwd_ex.
 * Every other argument, check and return code is that of attn_fwd_ex.
 * The counter is used when every (b, h) has at least 32 query blocks of
 * 256 rows (S > 7936); the q_cut = nqb/4 shortest blocks of every head are
 * then claimed, longest first, through one atomic add per claiming
 * workgroup, by workgroups placed after the fixed part of the grid, so the
 * XCDs that finish their fixed part first take more of them.  Otherwise the
 * counter is left alone.
 * Results equal those of attn_fwd_ex with the same flags bit for bit: each
 * block is computed the same way whichever workgroup runs it.
 */
int attn_fwd_balanced(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t S, int64_t H, int d_qk, int d_v, float softmax_scale,
                      int causal, int dtype, float q_descale, float k_descale, float v_descale,
                      unsigned flags, int32_t* counter, void* stream);

/*
 * attn_fwd_varlen -- attn_fwd over a batch of sequences of different
 * lengths packed along the token dimension, each attending only within
 * itself (variable-length batches, which "Ce que couvrent les noyaux" on the
 * ai-daily-news.org page lists among the kernels' future work).  Sequence s holds
 * token rows cu_seqlens[s] .. cu_seqlens[s+1]-1 of every tensor.
 *   q, k        device, [total, H, d_qk] contiguous; v [total, H, d_v]
 *   o           device, [total, H, d_v] bf16 (written)
 *   lse         device, [H, total] fp32 (written), or NULL
 *   cu_seqlens  device, n_seqs + 1 int32 prefix sums: 0 = cu[0] <= cu[1] <=
 *               ... <= cu[n_seqs] = total, each difference <= max_seqlen.
 *               Read by the kernels, not validated on the host: other
 *               contents are clamped to [0, total] and max_seqlen, which
 *               keeps every access in bounds but gives unspecified results.
 *               Empty sequences are allowed.
 *   n_seqs      >= 1;  total >= 1;  max_seqlen >= 1 (the longest sequence)
 *   the other arguments, alignment (cu_seqlens: 4 bytes), aliasing (o and lse
 *   must not overlap q, k, v, cu_seqlens or each other), the per-sequence
 *   4 GiB limit (with max_seqlen in place of S), determinism and the return
 *   codes are those of attn_fwd.
 * With n_seqs equal sequences of length L the results equal those of
 * attn_fwd with B = n_seqs, S = L bit for bit (LSE in [H, total] order).
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int64_t n_seqs, int64_t total, int64_t max_seqlen,
                    int64_t H, int d_qk, int d_v, float softmax_scale, int causal, int dtype,
                    float q_descale, float k_descale, float v_descale, void* stream);

/*
 * attn_amax_f32 -- largest magnitude of a float32 tensor, for choosing the
 * per-tensor FP8 descale (amax / 448).  The pages attribute most of the FP8
 * error to this quantization of Q, K and V ("Precisao, estabilidade e
 * efeito na pratica" on the miraibroadcast.com page).
 *   x         device, n float32 values (NaN entries are ignored)
 *   n         >= 1
 *   amax_out  device, one float32 (written; overwritten, not accumulated)
 * The result is exact and independent of the launch (max is order-free).
 */
int attn_amax_f32(const float* x, int64_t n, float* amax_out, void* stream);

/*
 * attn_quantize_e4m3 -- out[i] = E4M3FN(fp32(x[i] / descale)): one IEEE
 * fp32 division, then round-to-nearest-even into E4M3FN, saturating
 * magnitudes above 448 to +-448 (never NaN from finite input; NaN maps to
 * 0x7F).
 *   x        device, n float32 values
 *   n        >= 1
 *   descale  finite and > 0
 *   out      device, n bytes (written); must not overlap x
 */
int attn_quantize_e4m3(const float* x, int64_t n, float descale, uint8_t* out, void* stream);

/*
 * attn_quantize_fp8 -- the whole per-tensor FP8 quantization of one tensor,
 * on the device, with nothing read back to the host:
 *   amax     = max |x[i]|                 (of the rotated rows x . H when rotate)
 *   descale  = amax / 448 in fp32, or 1 when amax = 0
 *   codes[i] = E4M3FN(fp32(x[i] / descale)) (of (x . H)[i] when rotate)
 * so the largest magnitude lands on 448, the largest finite E4M3FN value.
 * The pages attribute most of the FP8 error to this rounding of Q, K and V
 * and credit the rotation with about half of it ("Precisao, estabilidade e
 * efeito na pratica" on the miraibroadcast.com page); amax / 448 is the
 * plain reading of a per-tensor scale for the e4m3 format.  The rounding and
 * saturation are those of attn_quantize_e4m3, the rotation that of
 * attn_hadamard_f32, and the results equal attn_amax_f32 (or
 * attn_hadamard_amax_f32) followed by attn_quantize_e4m3 (or
 * attn_hadamard_quantize_e4m3) with that descale, bit for bit.
 *   x        device, rows*d float32 values, row-major (NaN entries are
 *            ignored by the amax and encode to 0x7F)
 *   rows     >= 1;  d >= 1, and 128 or 192 when rotate = 1
 *   rotate   0 or 1 (else ATTN_ERR_UNSUPPORTED)
 *   codes    device, rows*d bytes (written); must not overlap x
 *   descale  device, one float32 (written): the descale of the codes, to be
 *            passed (by value, after a copy to the host) as the q/k/v
 *            descale of attn_fwd; must not overlap x or codes
 * x and descale must be 4-byte aligned.
 */
int attn_quantize_fp8(const float* x, int64_t rows, int d, int rotate, uint8_t* codes,
                      float* descale, void* stream);

/*
 * attn_hadamard_f32 / attn_hadamard_bf16 -- y[r,:] = x[r,:] . H for `rows`
 * rows of d elements, with H the normalized Sylvester-Hadamard matrix of
 * order 128 (d = 128) or block-diagonal with three order-64 blocks
 * (d = 192).  H is symmetric and orthogonal: applying it twice restores x
 * (up to rounding), and rotating Q and K by the same H leaves Q.K^T, hence
 * the attention weights, unchanged.  Rotating Q, K and V before FP8
 * quantization spreads outlier channels over the row and shrinks the
 * quantization error, the largest part of the FP8 error ("Precisao,
 * estabilidade e efeito na pratica" on the miraibroadcast.com page); the
 * attention output of a rotated V is rotated back by applying H to O.
 *   x     device, rows*d values (float32, or bfloat16 for _bf16), row-major
 *   rows  >= 1
 *   d     128 or 192 (else ATTN_ERR_UNSUPPORTED)
 *   y     device, rows*d values (written); may be x itself (in place) but
 *         must not overlap it otherwise (ATTN_ERR_ALIAS)
 * Arithmetic is fp32; the bf16 variant rounds its result to nearest even.
 * x and y must be 4-byte (f32) / 2-byte (bf16) aligned.
 */
int attn_hadamard_f32(const float* x, int64_t rows, int d, float* y, void* stream);
int attn_hadamard_bf16(const void* x, int64_t rows, int d, void* y, void* stream);

/*
 * attn_hadamard_amax_f32 / attn_hadamard_quantize_e4m3 -- the per-tensor
 * quantization of attn_amax_f32 / attn_quantize_e4m3 applied to the rotated
 * rows x[r,:] . H (H as for attn_hadamard_f32) without writing the rotated
 * tensor: one pass finds the largest rotated magnitude, a second rotates
 * again and encodes, so the rotation adds no memory traffic to the
 * quantization.  Both passes evaluate the rotation identically.
 *   x         device, rows*d float32 values, row-major
 *   rows, d   as for attn_hadamard_f32
 *   amax_out  device, one float32 (written): max |(x . H)[i]|, NaN ignored
 *   descale   finite and > 0
 *   out       device, rows*d bytes (written): E4M3FN((x . H)[i] / descale),
 *             rounding and saturation as attn_quantize_e4m3; must not
 *             overlap x
 */
int attn_hadamard_amax_f32(const float* x, int64_t rows, int d, float* amax_out, void* stream);
int attn_hadamard_quantize_e4m3(const float* x, int64_t rows, int d, float descale, uint8_t* out,
                                void* stream);

/*
 * attn_decode_paged -- one decode step against a paged KV cache: the new
 * query token of each sequence attends to every cached key of its sequence,
 *
 *   o[b,h] = softmax(tau * q[b,h] . K_b^T) V_b,   lse[b,h] = log sum_j exp(...)
 *
 * over keys j = 0 .. L_b - 1 (the new token's own key and value already
 * written to the cache).  Decode and paged KV caches are listed among the
 * kernels' future work ("Ce que couvrent les noyaux" on the
 * ai-daily-news.org page); this is the last row of causal attention.
 *   q            device, [B, H_q, d_qk] contiguous (bf16, or e4m3 codes)
 *   k_cache      device, [num_pages, page_size, H_kv, d_qk]
 *   v_cache      device, [num_pages, page_size, H_kv, d_v]
 *   block_table  device, [B, max_pages_per_seq] int32: key j of sequence b is
 *                slot j % page_size of page block_table[b, j / page_size]
 *   seq_lens     device, [B] int32, 0 <= L_b <= max_seqlen
 *   o            device, [B, H_q, d_v] bf16 (written)
 *   lse          device, [B, H_q] fp32 (written), or NULL
 *   workspace    device, at least attn_decode_workspace_bytes(B, H_q, H_kv,
 *                max_seqlen, d_v) bytes, 16-byte aligned; scratch for the
 *                partial results of the key splits, overwritten
 *   B            1 .. 65535;  H_kv 1 .. 65535;  H_q = G * H_kv, G in {1,2,4,8}
 *                (query head h reads key/value head h / G); B * H_q < 2^31
 *   d_qk, d_v    (128, 128) or (192, 128)
 *   page_size    a power of two, 16 .. 2^20;  num_pages >= 1
 *   max_pages_per_seq >= 1;  max_seqlen 1 .. max_pages_per_seq * page_size
 *                and < 2^30 (the longest sequence; sizes the key splits)
 *   softmax_scale, dtype, q/k/v_descale as in attn_fwd.
 * block_table and seq_lens are read by the kernels, not on the host: page
 * numbers are clamped to [0, num_pages) and lengths to [0, max_seqlen], which
 * keeps every access in bounds but gives unspecified results for other
 * contents.  Slots past the end of a sequence are never read.  An empty
 * sequence gives o = 0 and lse = -inf.  Alignment: q, k_cache, v_cache, o
 * 16 bytes, block_table, seq_lens, lse 4 bytes.  o, lse and workspace must not
 * overlap an input or each other.  Arithmetic is fp32 (scores as sums of
 * bf16 products, which holds e4m3 values exactly); the keys are split into
 * ranges whose partial results merge in a fixed order, so repeated calls
 * give bitwise identical results.
 */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                      void* workspace, int64_t workspace_bytes, int64_t B, int64_t H_q,
                      int64_t H_kv, int d_qk, int d_v, int64_t num_pages, int64_t page_size,
                      int64_t max_pages_per_seq, int64_t max_seqlen, float softmax_scale,
                      int dtype, float q_descale, float k_descale, float v_descale,
                      void* stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation, harnesses without an allocator): the same step, the
 * same kernels and bitwise the same results as attn_decode_paged with a
 * workspace, but the partial results of the key splits go to a scratch
 * array the library holds in device memory, ATTN_DECODE_SCRATCH_BYTES
 * (32 MiB) on each GPU it runs on, kept until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   Arguments, checks and status codes are those of attn_decode_paged
 *   without workspace / workspace_bytes; a step whose
 *   attn_decode_workspace_bytes(B, H_q, H_kv, max_seqlen, d_v) exceeds
 *   ATTN_DECODE_SCRATCH_BYTES returns ATTN_ERR_SCRATCH before any HIP call.
 *   The scratch of the current device is used: `stream` must belong to it.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in
 * time on one GPU (on different streams, or from different host threads)
 * race and give undefined results; calls ordered on one stream do not.
 * The scratch needs no clearing between calls.  ATTN_ERR_LAUNCH is also
 * returned when the runtime cannot resolve the scratch's device address
 * (done once per device, on the first call there).
 */
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* o,
                              float* lse, int64_t B, int64_t H_q, int64_t H_kv, int d_qk, int d_v,
                              int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                              int64_t max_seqlen, float softmax_scale, int dtype, float q_descale,
                              float k_descale, float v_descale, void* stream);

/*
 * attn_decode_workspace_bytes -- workspace attn_decode_paged needs for these
 * sizes (it depends on them only, not on the cache contents), or a negative
 * status code when they are out of range (see attn_decode_paged).
 */
int64_t attn_decode_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t max_seqlen,
                                    int d_v);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_ATTN_H */
