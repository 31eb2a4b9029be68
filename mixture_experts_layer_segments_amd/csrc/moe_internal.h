// Internal declarations shared by the HIP translation units of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

// Build with -DMOE_DEBUG_LAUNCH to print the pending HIP error after each
// launch point (diagnostics only; off in normal builds).
#ifdef MOE_DEBUG_LAUNCH
#include <stdio.h>
#define MOE_DBG(tag)                                                              \
  do {                                                                            \
    hipError_t e_ = hipPeekAtLastError();                                         \
    if (e_ != hipSuccess) fprintf(stderr, "[moe] %s: %s\n", tag, hipGetErrorString(e_)); \
  } while (0)
#else
#define MOE_DBG(tag) \
  do {               \
  } while (0)
#endif

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxWays = 4;
constexpr int kMaxBins = kMaxE * kMaxWays;
constexpr int kMaxSegments = kMaxE * kMaxWays;
constexpr size_t kAlign = 256;
constexpr int kSmallA = 1024;  // assignments up to which one workgroup routes and permutes

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

// Replicas per hot expert (1 when nothing is split) and the histogram bins
// per expert: a replica is its own bin only in the parity split.
inline int split_ways(const moe_config& c) { return c.n_hot_split > 0 ? c.split_ways : 1; }
inline int bin_ways(const moe_config& c) {
  return c.split_mode == MOE_SPLIT_PARITY ? split_ways(c) : 1;
}

// The one-wave planner applies: nothing split, at most 256 experts and the
// dropless layout (one segment and one bin per expert).
inline bool wave_plan(const moe_config& c) {
  return c.E <= 256 && !(c.n_hot_split > 0 && c.split_ways > 1) &&
         c.capacity_factor_permille <= 0;
}

// Slots per expert of the fixed-capacity layout, ceil(f * T*k / E) with
// f = capacity_factor_permille / 1000; 0 for the dropless layout.
inline int64_t capacity(const moe_config& c) {
  if (c.capacity_factor_permille <= 0) return 0;
  const int64_t num = (int64_t)c.T * c.k * c.capacity_factor_permille, den = 1000ll * c.E;
  return (num + den - 1) / den;
}
// Rows of x_perm / h / y_perm / row_to_token.
inline int64_t num_rows(const moe_config& c) {
  return c.capacity_factor_permille > 0 ? c.E * capacity(c) : (int64_t)c.T * c.k;
}

// Assignment chunk of one histogram / rank block: a multiple of 64, grown so
// that there are at most 256 chunks.  A rank block is one wave ranking its
// chunk 64 assignments at a time, serially, so small batches take 64-long
// chunks and more blocks (with 256-long ones, a 4000-token top-2 batch ran
// 32 waves of 4 rounds each).
inline int chunk_len(int64_t A) {
  int64_t c = (A + 255) / 256;
  c = (c + 63) / 64 * 64;
  if (c < 64) c = 64;
  return (int)c;
}
inline int num_chunks(int64_t A) { return (int)((A + chunk_len(A) - 1) / chunk_len(A)); }
// Row stride (ints) of the per-chunk count and base tables: the chunks
// rounded up to a multiple of 4, so that a lane moves 4 chunks in one
// 16-byte access.
inline int chunk_stride(int64_t A) { return (num_chunks(A) + 3) & ~3; }

// The grouped GEMMs take the weight-streaming decode tiles when a launch's
// rows are at most kDecodeRows per segment on average (the host never sees
// the segment lengths, so it decides from the mean).
constexpr int64_t kDecodeRows = 16;
inline bool uses_decode_tiles(int64_t rows, int64_t segments) {
  return rows <= kDecodeRows * segments;
}

// Offsets of the workspace regions (bytes).  P: permutation scratch;
// G: grouped-FFN scratch (h); L: layer intermediates.
struct Layout {
  size_t cnt_bin, blk_off, seg_of_bin, p_end;                 // region P
  size_t h, shared_h,                                         // region G
      h_q, h_s, shared_hq, shared_hs,                         //   (FP8 activations: h quantized)
      a_deq, g_end;                                           //   (FP8 activations, decode tiles:
                                                              //    the activations in bf16)
  size_t y_perm, shared_y, seg_offsets, seg_expert,           // region L
      assign_to_row, row_to_token, row_w,
      x_q, x_s, l_end;                                        //   (FP8 activations: x quantized)
};
Layout make_layout(const moe_config& c);
int32_t num_segments(const moe_config& c);

// ---- launchers (all asynchronous on `s`) ----
void launch_route(const moe_config& c, const float* logits, int32_t* ids, float* w,
                  hipStream_t s);
void launch_permute(const moe_config& c, const void* x, const int32_t* ids, void* x_perm,
                    int32_t* seg_offsets, int32_t* seg_expert, int32_t* a2r, int32_t* r2t,
                    int32_t* counts, float* bal, const float* w, float* row_w, char* ws,
                    const Layout& L, hipStream_t s);

// Routing and permutation in one single-workgroup launch, for T*k <= kSmallA
// (no x_perm; writes ids, w, counts, seg_offsets, seg_expert, assign_to_row,
// row_to_token, row_w and balancedness).
void launch_route_permute_small(const moe_config& c, const float* logits, int32_t* ids,
                                float* w, int32_t* counts, int32_t* seg_offsets,
                                int32_t* seg_expert, int32_t* a2r, int32_t* r2t, float* row_w,
                                float* bal, hipStream_t s);

// One grouped-FFN problem: segments [seg_offsets[s], seg_offsets[s+1]) of
// the rows of A, or (shared) one segment of all `rows` rows.
struct FfnProblem {
  const void* A;          // [rows, K1] act dtype
  const void* w13;        // [n_w, 2*Iw, K1]
  const void* w2;         // [n_w, K1, Iw]
  void* h;                // [rows, Iw] scratch
  void* y;                // [rows, K1] out
  const float* row_scale; // nullable, by row
  const int32_t* seg_offsets;  // nullable: shared problem = one segment
  const int32_t* seg_expert;
  const int32_t* a_rows;  // nullable: GEMM 1 reads row a_rows[r] of A for row r
  int32_t n_seg;          // segments (1 for shared)
  int32_t rows;           // rows of h / y (and of A unless a_rows gathers)
  int32_t max_seg_rows;   // no segment is longer (rows, or the tokens when every
                          // token has at most one row in a segment)
  int32_t n_w;            // experts in w13 / w2; segments of other experts are skipped
  int32_t Iw;             // intermediate size of this problem
  int32_t w_fp8;          // 1: w13 / w2 are E4M3 codes with the block scales below
  const float* w13_scale; // [n_w, 2*Iw/128, K1/128] (w_fp8 only)
  const float* w2_scale;  // [n_w, K1/128, Iw/128]
  // FP8 activations (w_fp8 too): A holds E4M3 codes with a_scale [A rows,
  // K1/128]; h is quantized into h_q [rows, Iw] / h_scale [rows, Iw/128]
  // between the two GEMMs
  int32_t a_fp8;
  const float* a_scale;
  uint8_t* h_q;
  float* h_scale;
  // FP8 activations on the decode tiles: scratch for A in bf16 [A rows, K1]
  // of a_deq_bytes (too small or null: the E4M3 decode tiles read the codes)
  void* a_deq;
  size_t a_deq_bytes;
};
void launch_grouped_ffn(const moe_config& c, const FfnProblem* probs, int n_probs,
                        hipStream_t s);
// FP8 weights: block-quantize n_mat bf16 matrices [rows, cols] (multiples of 128).
void launch_quantize_fp8(int n_mat, int rows, int cols, const void* src, uint8_t* q,
                         float* scale, hipStream_t s);
// FP8 activations: quantize bf16 rows [rows, cols] (cols a multiple of 128) in
// 1 x 128 pieces: codes [rows, cols] and scales [rows, cols / 128].
void launch_quantize_rows_fp8(int64_t rows, int cols, const void* src, uint8_t* q,
                              float* scale, hipStream_t s);
// bf16 dst = E4M3 codes q times their 1 x 128 scales (exact), [rows, cols].
void launch_dequantize_rows_fp8(int64_t rows, int cols, const uint8_t* q, const float* scale,
                                void* dst, hipStream_t s);
// bf16 rows rounded through E4M3 in place: each value becomes what the
// row quantizer's code and scale for it dequantize to.
void launch_fake_quant_rows_fp8(int64_t rows, int cols, void* data, hipStream_t s);
void launch_combine(const moe_config& c, const void* y_perm, const int32_t* a2r,
                    const float* w, const void* shared_y, void* out, hipStream_t s);

int device_cu_count();

}  // namespace moe
