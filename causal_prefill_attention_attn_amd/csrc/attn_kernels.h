// Internal launchers shared by the C-ABI front end (attn_api.hip) and the
// kernel translation units.  Arguments are already validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

// B problems of up to S rows each: dense [B,S,H,D] tensors when cu is null,
// else B packed sequences of a [total,H,D] tensor bounded by cu[0..B]
// (device), S being the longest.  Returns 0 or -1 (launch error).

// tail_ctr: null, or a device word the launch may use to share the shortest
// query blocks among the XCDs (block_claim); it is cleared by a kernel on the
// same stream before the attention kernel.  Results do not depend on it.

// BF16 q/k/v, d_qk in {128, 192}, d_v = 128.
int launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* cu, int64_t total, int B, int S, int H, int d_qk,
                     float softmax_scale, int causal, int32_t* tail_ctr, hipStream_t stream);

// FP8 E4M3FN q/k/v with per-tensor descales, d_qk in {128, 192}, d_v = 128;
// rot_o: O rows times the normalised Hadamard matrix of order 128; exact_p:
// probabilities by exp2 and a rounding conversion instead of the lean form.
int launch_attn_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu, int64_t total, int B, int S, int H, int d_qk,
                    float softmax_scale, int causal, float q_descale, float k_descale,
                    float v_descale, bool rot_o, bool exact_p, int32_t* tail_ctr,
                    hipStream_t stream);

// Grid of an attention launch with nqb query blocks per (b, h): the static
// order, or, with a counter on a dense problem of at least 32 blocks per
// head, the static part without the nqb/4 shortest blocks of every head
// plus twice as many claiming workgroups as there are claimed blocks.  (At
// 4K tokens, 16 blocks, sharing gained nothing measurable.)
struct BlockGrid {
  int grid, n_static, q_cut;
};
inline BlockGrid block_grid(int nqb, int BH, bool dense, bool counter) {
  if (counter && dense && nqb >= 32) {
    const int q_cut = nqb / 4;
    const int n_static = BH * (nqb - q_cut);
    return {n_static + 2 * BH * q_cut, n_static, q_cut};
  }
  return {nqb * BH, nqb * BH, 0};
}
// *p = 0, as a kernel on the stream (graph-capture safe)
int launch_clear_i32(int32_t* p, hipStream_t stream);

int launch_amax_f32(const float* x, int64_t n, float* amax_out, hipStream_t stream);
int launch_quantize_e4m3(const float* x, int64_t n, float descale, uint8_t* out,
                         hipStream_t stream);

// y[r] = x[r] . H for rows of d in {128, 192} elements (fp32, or bf16 when
// bf16 is set); y may equal x.
int launch_hadamard(const void* x, int64_t rows, int d, bool bf16, void* y, hipStream_t stream);
// amax of the rotated fp32 rows; e4m3 codes of the rotated rows / descale
int launch_hadamard_amax(const float* x, int64_t rows, int d, float* amax_out,
                         hipStream_t stream);
int launch_hadamard_quantize(const float* x, int64_t rows, int d, float descale, uint8_t* out,
                             hipStream_t stream);
// the same with the descale read from device memory
int launch_hadamard_quantize_dev(const float* x, int64_t rows, int d, const float* descale,
                                 uint8_t* out, hipStream_t stream);
// Whole per-tensor quantization on the device: amax (of the rotated rows when
// rotate, d in {128, 192}), descale = amax / 448 (1 when zero) written to
// *descale, then the codes of x / descale.
int launch_quantize_fp8(const float* x, int64_t rows, int d, bool rotate, uint8_t* codes,
                        float* descale, hipStream_t stream);

// Decode step against a paged KV cache (decode.hip).  split/nsplit come from
// decode_split_policy; the workspace holds B*Hq*nsplit partial outputs of 128
// floats followed by B*Hq*nsplit partial log-sum-exps.
struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  void* workspace;
  int64_t B, Hq, Hkv;
  int d_qk;
  int64_t num_pages, page_size, max_pages_per_seq, max_seqlen;
  float softmax_scale;
  bool dtype_fp8;
  float q_descale, k_descale, v_descale;
  int split, nsplit;
};
void decode_split_policy(int64_t B, int64_t Hkv, int64_t max_seqlen, int* split, int* nsplit);
// The split a call uses: decode_split_policy for e4m3, longer splits for bf16
// (never more of them).
void decode_launch_policy(const DecodeArgs& a, int* split, int* nsplit);
int64_t decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_seqlen);
int launch_decode(const DecodeArgs& a, hipStream_t stream);

// Library-held decode scratch (the allocation-free entry point): its size,
// and the current device's copy (resolved once per device), or null when the
// runtime cannot name it.
constexpr int64_t kDecodeScratchBytes = int64_t(32) << 20;
void* decode_scratch();

}  // namespace cpattn
