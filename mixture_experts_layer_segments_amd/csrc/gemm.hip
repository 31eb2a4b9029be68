// Grouped SwiGLU expert MLP over ragged segments ("Serving Mixture-of-Experts
// Models", section "Follow one token through an MoE layer", step 3: one kernel
// runs every expert's segment as a matrix with its own row count; the MoE
// inference blog, "Optimized kernels for MoE": grouped GEMM).
//
//   GEMM 1: [g | u] = X_s . [W_gate[e] | W_up[e]],  h = silu(g) * u
//   GEMM 2: y = row_scale * (h . W_down[e])
//
// bf16 path: persistent MFMA kernels.  A device-side tile table (exclusive
// prefix of tiles per segment) is built from the segment offsets, so segment
// lengths never travel to the host.  Each workgroup walks the tile list with a
// fixed stride; tiles are ordered segment-major, then in groups of 8 row
// blocks that walk every column block, and the workgroup -> tile mapping is
// remapped so that consecutive tiles (which share weight slices and
// activation rows) land on the same XCD and therefore the same L2.  The K loop double-buffers LDS tiles; operands
// are XOR-swizzled in 16-byte chunks so that MFMA operand reads avoid bank
// conflicts.  fp32 path: a wave per output element (the fp32 layer is tiny).
#include <math.h>

#include <mutex>

#include "fp8_dev.h"
#include "moe_internal.h"
#include "wave_dev.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

struct GemmProblem {
  const uint16_t* A;        // [rows, K] bf16 bits
  const uint16_t* B;        // [n_w][NB, K]
  uint16_t* C;              // [rows, N]
  const float* scale;       // nullable, by row
  const int32_t* seg_offsets;  // nullable: one segment [0, rows)
  const int32_t* seg_expert;   // nullable: expert 0
  const int32_t* a_rows;       // nullable: row r of the problem is row a_rows[r] of A
  int32_t n_seg, rows, N, K;
  int32_t n_w;              // experts in B: a segment of another expert (padding) is skipped
  int32_t a_ld_rows;        // rows of the A allocation (bounds of the copy source)
  int32_t up_off;           // GEMM 1: row offset of W_up inside B
  int64_t b_stride;         // elements per expert in B
  const float* b_scale;     // FP8 weights: [n_w][NB/128][K/128] block scales (else unused)
  int64_t s_stride;         // floats per expert in b_scale
  const float* a_scale;     // FP8 activations: [A rows][K/128] scales of the A codes
  // FP8 activations, GEMM 1 on ring tiles: h leaves the tile as E4M3 codes
  // [rows, N] with one scale per 1 x 128 piece [rows, N/128] (C is unused)
  uint8_t* Cq;
  float* c_scale;
};

struct GemmArgs {
  GemmProblem p[2];
  int32_t n_probs;
  int32_t n_seg_total;
  // this launch's tiles: segments with min_len <= length < max_len, each cut
  // into ceil(length / tile_bm) x ceil(N / tile_ncols) tiles
  int32_t tile_bm, tile_ncols, min_len, max_len;
};

__device__ __forceinline__ void seg_range(const GemmProblem& P, int s, int& r0, int& len,
                                          int& e) {
  if (P.seg_offsets) {
    r0 = P.seg_offsets[s];
    len = P.seg_offsets[s + 1] - r0;
    e = P.seg_expert[s];
  } else {
    r0 = 0;
    len = P.rows;
    e = 0;
  }
}

// Row tiles that share a weight slice in the tile order (groups of 4, 16 or
// 32 measured 0.5-3% slower on the ragged layers).
constexpr int kGroupM = 8;
constexpr size_t kMaxLdsBytes = 160 * 1024;  // LDS per workgroup on gfx950

// Workgroup ids are dealt round-robin to the 8 XCDs; renumber them so that
// consecutive logical ids share an XCD (and its L2).  Measured 2-5% faster
// than the plain order on the ragged and DeepSeek-shaped layers.
__device__ __forceinline__ int xcd_logical(int bid, int G) {
  return (bid % 8) * (G / 8) + bid / 8;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)to_bf16(lo) | ((uint32_t)to_bf16(hi) << 16);
}

// Two E4M3 codes (the low or upper half-word of w) times a power-of-two
// scale, as two bf16 (exact: an E4M3 value times a power of two is a bf16
// value).
template <bool UPPER>
__device__ __forceinline__ uint32_t fp8x2_to_bf16(uint32_t w, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, UPPER));
}

// ---------------------------------------------------------------- tile tables
// Every workgroup of a grouped-GEMM launch builds the launch's tile table in
// its own LDS from the segment offsets at kernel start: tiles_l[g] = tiles of
// the segments before g (an exclusive prefix), tiles_l[n] = the total.  The
// lengths never leave the device, no separate planning launch runs, and the
// cost is one read of the offsets (L2-resident after the first workgroup)
// and a block scan.
// Tiles of segment g (over both problems) for a cover of tiles bm rows x
// ncols output columns over the segments of length in [min_len, max_len).
__device__ __forceinline__ int seg_tiles(const GemmArgs& a, int g, int bm, int ncols,
                                         int min_len, int max_len) {
  const int p = g < a.p[0].n_seg ? 0 : 1;
  const GemmProblem& P = a.p[p];
  const int s = g - (p ? a.p[0].n_seg : 0);
  const int len = P.seg_offsets ? P.seg_offsets[s + 1] - P.seg_offsets[s] : P.rows;
  if (len < min_len || len >= max_len) return 0;
  if (P.seg_offsets && (unsigned)P.seg_expert[s] >= (unsigned)P.n_w) return 0;
  return ((len + bm - 1) / bm) * ((P.N + ncols - 1) / ncols);
}

// `wsum`: NTHR / 64 + 1 ints of LDS scratch.  Ends with a barrier.
template <int NTHR>
__device__ void build_tile_table(const GemmArgs& a, int* tiles_l, int* wsum, int bm, int ncols,
                                 int min_len, int max_len) {
  constexpr int NW = NTHR / 64;
  const int n = a.n_seg_total, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n + NTHR - 1) / NTHR;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int g = lo; g < hi; ++g) sum += seg_tiles(a, g, bm, ncols, min_len, max_len);
  const int incl = wave_dev::incl_scan(sum);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int t = wsum[w];
      wsum[w] = run;
      run += t;
    }
    wsum[NW] = run;
  }
  __syncthreads();
  int run = wsum[wv] + incl - sum;
  for (int g = lo; g < hi; ++g) {
    tiles_l[g] = run;
    run += seg_tiles(a, g, bm, ncols, min_len, max_len);
  }
  if (tid == 0) tiles_l[n] = wsum[NW];
  __syncthreads();
}

// ---------------------------------------------------------------- bf16 MFMA tiles
// Segments of many rows.  Block tile BM x BN (weight rows) x 64 over NTHR/64
// waves laid out WAVES_M x WAVES_N, each wave a grid of 16x16x32 MFMAs with
// fp32 accumulators; 128 x 256 over 2 x 4 waves with a 3-stage ring for
// moderate segments (HBM-bound), 256 x 256 over 4 x 2 waves with 2 stages for
// large ones (half the operand traffic per flop).  LDS rows are 128-byte
// pieces of 8 chunks of 16 bytes, XOR-swizzled by row.
//
// MODE 0: GEMM 1 with the SwiGLU epilogue.  The B tile holds BN rows: the
//         first BN/2 are W_gate rows n0.., the rest W_up rows n0.. (BN/2
//         output columns per tile).  Each wave owns matching gate and up
//         columns, so silu(g) * u is formed in registers.
// MODE 1: GEMM 2 with the row-scale epilogue (BN output columns per tile).
//
// Global -> LDS copies go straight into a STAGES-deep LDS ring
// (global_load_lds_dwordx4: each wave instruction fills one contiguous 1 KiB
// block of 8 swizzled 128-byte row pieces), so the copies for the next
// STAGES-1 K stages stay in flight while the current one feeds the MFMAs,
// with no registers spent on staging.  Completion is tracked with explicit
// vmcnt waits: a wave waits until at most the copies it issued for later
// stages are outstanding, then a plain s_barrier (without the memory fence of
// __syncthreads, which would wait for every copy) makes the stage visible to
// all waves and frees the slot read one stage earlier.
//
// Inside a stage the MFMA operands are double-buffered in registers: the
// fragments of the second 32-deep K step are read from LDS while the MFMAs of
// the first run, one read slotted between every few MFMAs
// (sched_group_barrier), so a wave waits on LDS once per K step instead of
// once per fragment -- left to itself the compiler reloads one fragment at a
// time to save registers (measured 3-6% faster on the large tiles).
#define MOE_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most `later` stages of this wave's copies (LPW each) are in
// flight; vmcnt takes an immediate, so dispatch on the count.
template <int LPW, int J>
__device__ __forceinline__ void wait_stages(int later) {
  if constexpr (J <= 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= J) wait_vmcnt<J * LPW>();
    else wait_stages<LPW, J - 1>(later);
  }
}

// XOR swizzle of the 16-byte chunk index inside a row piece of KCH chunks,
// chosen so that the 16 lanes reading one MFMA operand column (16 rows, same
// logical chunk) hit distinct 16-byte bank groups of a 256-byte bank row
// (128-byte pieces: measured 3-9% faster than swizzling by row & 7; 256-byte
// pieces, the bf16 activations of 128-deep stages, every row a whole bank row:
// row & 15, 2-4% faster than row & 7).
template <int KCH>
__device__ __forceinline__ int swz(int row) {
  if constexpr (KCH == 16) return row & 15;
  else if constexpr (KCH == 8) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}

// Raw buffer resource over `bytes` bytes at `base` (word 3: the gfx9 raw
// buffer format; loads past `bytes` return zero instead of touching memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Copy K stage kt of this wave's LPI 1 KiB blocks into its ring slot: the
// wave's first A_IT blocks are A blocks i * NI + w (RPB rows of 128-byte
// pieces each), the rest B blocks (i - A_IT) * NI + w, starting at chunk A_CH
// of the slot (bf16 weights and the 128-deep stages' E4M3 codes: 128-byte
// row pieces; E4M3 codes of 64-deep stages: 64-byte pieces, 16 rows per
// block).  `voff` holds each lane's byte offset of its
// 16 bytes at k = 0; the stage's K offset goes in the scalar offset.
//
// K tail (bf16, K not a multiple of BK): in the last stage only the first
// `kval` 16-byte chunks of each row piece lie inside K; the lanes that copy
// a chunk past it take an offset past the buffer's range, so both operands
// hold zeros there and add nothing.  (KCH, KCHB: chunks per A / B row piece;
// RPB, RPBB: rows per 1 KiB block.)
template <int LPI, int NI, int STAGES, int STAGE_CH, int A_CH, int BK, int A_IT, int WB, int AB,
          int B_AUX = 0, int KCH = 8, int KCHB = 8, int BM = 0>
__device__ __forceinline__ void ring_issue(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                           const uint32_t* voff, u32x4* ring, int kt, int wv,
                                           int kval = 64) {
  u32x4* slot = ring + (kt % STAGES) * STAGE_CH;
  if (kval >= KCH && kval >= KCHB) {
#pragma unroll
    for (int i = 0; i < LPI; ++i) {
      if (i < A_IT)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MOE_LDS_PTR(slot + (i * NI + wv) * 64), 16,
                                                 voff[i], kt * BK * AB, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, MOE_LDS_PTR(slot + A_CH + ((i - A_IT) * NI + wv) * 64), 16, voff[i],
            kt * BK * WB, 0, B_AUX);
    }
  } else {
    const int lane = threadIdx.x & 63;
    constexpr int RPB = 64 / KCH, RPBB = 64 / KCHB;
#pragma unroll
    for (int i = 0; i < LPI; ++i) {
      if (i < A_IT) {
        const int row = (i * NI + wv) * RPB + lane / KCH;
        const int kc = (lane % KCH) ^ swz<KCH>(row);
        const uint32_t off = kc < kval ? voff[i] : 0xFFFFFFF0u - (uint32_t)(kt * BK * AB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MOE_LDS_PTR(slot + (i * NI + wv) * 64), 16,
                                                 off, kt * BK * AB, 0, 0);
      } else {
        const int br = ((i - A_IT) * NI + wv) * RPBB + lane / KCHB;
        const int kc = (lane % KCHB) ^ swz<KCHB>(BM + br);
        const uint32_t off = kc < kval ? voff[i] : 0xFFFFFFF0u - (uint32_t)(kt * BK * WB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, MOE_LDS_PTR(slot + A_CH + ((i - A_IT) * NI + wv) * 64), 16, off, kt * BK * WB,
            0, B_AUX);
      }
    }
  }
}

// 16-byte chunks of stage kt's row pieces that lie inside K (64, i.e. all of
// them, for a full stage).
// (KTAIL false: K is a multiple of BK and every stage is full -- the launches
// take the K-tail variant only when it is not.)
template <int BK, int AB, bool KTAIL>
__device__ __forceinline__ int ring_stage_chunks(int K, int kt) {
  if constexpr (!KTAIL) return 64;
  const int left = K - kt * BK;
  return left >= BK ? 64 : left * AB / 16;
}

// Ring-tile geometry shared by the per-tile body and the kernels that size
// the ring (WF = 1: the weight rows of a stage hold 1-byte E4M3 codes; WF = 2:
// the activation rows too).
template <int WF, int BM, int BN, int BK, int STAGES>
struct RingShape {
  static constexpr int AB = WF == 2 ? 1 : 2;              // bytes per activation element
  static constexpr int KCH = BK * AB / 16;                // A: 16-byte chunks per row piece
  static constexpr int KCHB = WF ? BK / 16 : BK / 8;      // B: 16-byte chunks per row piece
  static constexpr int A_CH = BM * KCH;                   // A chunks per stage
  static constexpr int STAGE_CH = A_CH + BN * KCHB;       // 16-byte chunks per stage
  static constexpr int RING_CH = STAGES * STAGE_CH;       // 16-byte chunks of the ring
};

// 8 E4M3 codes (byte j of word w = element 4w + j) times their block's
// power-of-two scale, as an MFMA operand of 8 bf16 (exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi, float sc) {
  return __builtin_bit_cast(bf16x8, u32x4{fp8x2_to_bf16<false>(lo, sc), fp8x2_to_bf16<true>(lo, sc),
                                          fp8x2_to_bf16<false>(hi, sc), fp8x2_to_bf16<true>(hi, sc)});
}

// Ring tiles.  A workgroup of the persistent grid takes tiles l, l + G,
// l + 2G, ...; each tile is set up (ring_setup), its block scales staged
// (ring_scales), its first stages issued (ring_prologue), its K loop run over
// the LDS ring (ring_kloop), and its output packed to bf16 (ring_pack) and
// written through the then idle ring (ring_store): every wave stages its rows
// there and writes them back as 16-byte row chunks, whole cache lines, instead
// of 8-byte pieces 16 rows apart (measured: the output writes had been ~40% of
// a 256 x 256 tile's time; the staged form is 5-10% faster overall).
//
// WF = 1: the weights are E4M3 codes with 128 x 128 block scales.  The codes
// travel into the ring as they are (half the bytes of bf16, so a ring of the
// same size holds more, or deeper, stages) and are dequantized when a wave reads its MFMA operand: an
// 8-byte LDS read and four conversions with the block's scale.  The tile's
// block scales (its two 128-row blocks of weights x K/128) are staged once
// per tile into `scl`, LDS beside the tile table.
// WF = 2: E4M3 activations too, one scaled FP8 MFMA K step per stage; the
// E8M0 exponents of the tile's activation rows' scales follow `scl`.
// Cache policy of the weight copies of a 128-row tile whose segment has no
// other row tile (its weights are read once): 2 = non-temporal (gfx950 "nt").
// Measured with bf16 weights: 2% faster on the prefill and DeepSeek-shaped
// layers (streaming the weights past L2 leaves it to the activations); with
// E4M3 weights on 128-deep stages 1%, with E4M3 activations too 2-4% (the
// 128-row launches).  Only where a stage's weight row piece is a whole
// 128-byte line: 64-byte pieces split every line over two stages, and a
// streamed line is fetched twice (6-7% slower).  A segment with several row
// tiles keeps the default policy, since its other row tiles read the same
// weights (streaming them too was 11% slower on prefill).
// Cache policy of the ring tiles' GEMM 2 output (y_perm) stores: 2 =
// non-temporal.  y_perm is written once and read once by the combine, and
// keeping it out of L2 leaves L2 to the tiles' operands: measured 1-2.5%
// faster grouped FFN on the bf16 prefill, DeepSeek-shaped and ragged layers.
constexpr int kAuxNT = 2;   // the gfx950 "nt" bit of a buffer access's aux operand
template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES>
struct RingCfg {
  using RS = RingShape<WF, BM, BN, BK, STAGES>;
  static constexpr int KCH = RS::KCH, KCHB = RS::KCHB, A_CH = RS::A_CH, STAGE_CH = RS::STAGE_CH;
  static constexpr int AB = RS::AB;            // bytes per activation element
  static constexpr int RPB = 64 / KCH;         // A rows per 1 KiB copy block
  static constexpr int RPBB = 64 / KCHB;       // B rows per 1 KiB copy block
  static constexpr int NW = NTHR / 64;
  static constexpr int WAVES_N = NW / WAVES_M;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;   // wave tile
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int WB = WF ? 1 : 2;        // bytes per weight
  // With 8 waves only one wave per SIMD (waves 0-3) issues the copies, so
  // that its partner never stalls behind the copy issue and keeps the SIMD's
  // matrix core fed.
  // (measured 2-5% faster than all eight waves issuing)
  static constexpr int NI = NW == 8 ? 4 : NW;   // issuing waves
  static constexpr int A_IT = BM / RPB / NI;   // A copies per issuing wave per stage
  static constexpr int LPI = A_IT + BN / RPBB / NI;   // all copies per issuing wave per stage
  // cache policy of the weight copies of single-row-tile segments (the
  // 128-row tiles whose weight row pieces are whole 128-byte lines, as above)
  static constexpr int B_AUX = (BM < 256 && BK * WB == 128) ? kAuxNT : 0;
  static_assert(WF == 2 ? BK == 128 : WF == 1 ? (BK == 64 || BK == 128) : (BK == 32 || BK == 64),
                "row pieces of 64, 128 or 256 bytes");
  static_assert((BM / RPB) % NI == 0 && (BN / RPBB) % NI == 0, "copy blocks per wave");
  static_assert(STAGES >= 2 && STAGES <= 6, "ring shape");
  static_assert(LPI * (STAGES - 2) < 64, "vmcnt range");
};

// Where one tile sits: its segment's rows, expert, output corner and the
// copy sources (voff: this lane's byte offset at k = 0 of each of the wave's
// copies; only the issuing waves fill it).
template <int LPI>
struct RingTileState {
  int r0, len, e, m0, n0;
  bool stream;   // the weight copies take the streaming cache policy
  const GemmProblem* P;
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t voff[LPI];
};

template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES>
__device__ __forceinline__ void ring_setup(const GemmArgs& args, const int* tiles_l, int tile,
                                           RingTileState<RingCfg<MODE, WF, BM, BN, BK, NTHR,
                                                                 WAVES_M, STAGES>::LPI>& t) {
  using C = RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>;
  const int lane = threadIdx.x & 63;
  const int wvs = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nst = args.n_seg_total;
  int lo = 0, hi = nst - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (tiles_l[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int gs = lo;
  const int pi = gs < args.p[0].n_seg ? 0 : 1;
  const GemmProblem& P = args.p[pi];
  t.P = &args.p[pi];
  seg_range(P, gs - (pi ? args.p[0].n_seg : 0), t.r0, t.len, t.e);
  const int mt = (t.len + BM - 1) / BM;
  // weights that no other row tile of the segment reads again
  t.stream = mt == 1;
  const int ncols = MODE == 0 ? BN / 2 : BN;
  const int nt = (P.N + ncols - 1) / ncols;
  const int local = tile - tiles_l[gs];
  const int grp = local / (kGroupM * nt);
  const int first_m = grp * kGroupM;
  const int gm = min(kGroupM, mt - first_m);
  const int lg = local - grp * kGroupM * nt;
  t.m0 = (first_m + lg % gm) * BM;
  t.n0 = (lg / gm) * ncols;
  const int K = P.K, N = P.N;
  const uint8_t* Bb = reinterpret_cast<const uint8_t*>(P.B) + (size_t)t.e * P.b_stride * C::WB;
  t.ra = buffer_rsrc(P.A, (uint32_t)((size_t)P.a_ld_rows * K * C::AB));
  t.rb = buffer_rsrc(Bb, (uint32_t)((size_t)(MODE == 0 ? 2 * N : N) * K * C::WB));
  if (wvs >= C::NI) return;
#pragma unroll
  for (int i = 0; i < C::LPI; ++i) {
    if (i < C::A_IT) {
      const int row = (i * C::NI + wvs) * C::RPB + lane / C::KCH;
      const int kc = (lane % C::KCH) ^ swz<C::KCH>(row);
      const int ar = t.r0 + min(t.m0 + row, t.len - 1);
      const int grow = P.a_rows ? P.a_rows[ar] : ar;
      t.voff[i] = (uint32_t)grow * (uint32_t)(K * C::AB) + kc * 16;
    } else {
      const int br = ((i - C::A_IT) * C::NI + wvs) * C::RPBB + lane / C::KCHB;  // weight-tile row
      const int kc = (lane % C::KCHB) ^ swz<C::KCHB>(BM + br);
      int grow;
      if (MODE == 0) {
        const int col = min(t.n0 + (br % (BN / 2)), N - 1);
        grow = br < BN / 2 ? col : P.up_off + col;
      } else {
        grow = min(t.n0 + br, N - 1);
      }
      t.voff[i] = (uint32_t)grow * (uint32_t)(K * C::WB) + kc * 16;
    }
  }
}

// The tile's block scales into LDS (WF >= 1); the ring and `scl` must be free.
template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES>
__device__ __forceinline__ void ring_scales(
    const RingTileState<RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>::LPI>& t,
    float* scl, int tid, int nthr) {
  if constexpr (WF >= 1) {
    const GemmProblem& P = *t.P;
    const int K = P.K, N = P.N, KB = K / 128;
    // group 0 / 1 = the tile's first / second 128 weight rows (GEMM 1: the
    // gate / up halves), x every K block
    const float* Sb = P.b_scale + (size_t)t.e * P.s_stride;
    const int nrb = (MODE == 0 ? 2 * N : N) / 128;
    for (int i = tid; i < 2 * KB; i += nthr) {
      const int g = i / KB, kb = i % KB;
      const int rb_ = MODE == 0 ? (g ? (P.up_off + t.n0) / 128 : t.n0 / 128)
                                : min(t.n0 / 128 + g, nrb - 1);
      scl[i] = Sb[rb_ * KB + kb];
    }
  }
}

// FP8 activations: the E8M0 exponents of the tile's BM activation rows'
// scales, a byte each, go into LDS after the weight-block scales.  TPR
// threads take one row (its source row looked up once) and a run of its KB
// scales each.  The first RUN of a thread's loads are issued together, with
// indices clamped into the run instead of branches, before the tile's first
// ring copies (act_scales_load); the bytes are written after them
// (act_scales_store), so the scale loads' latency overlaps the copies'.
// A run longer than RUN (K above RUN * TPR * 128) finishes in further passes.
template <int BM, int NTHR, int RUN>
struct ActScales {
  static constexpr int TPR = NTHR / BM;
  static_assert(NTHR % BM == 0, "threads per activation row");
  uint32_t v[RUN];
  const float* src;
  int k0, k1;
};

template <int BM, int NTHR, int RUN, typename TS>
__device__ __forceinline__ void act_scales_load(const TS& t, int KB, ActScales<BM, NTHR, RUN>& a) {
  constexpr int TPR = ActScales<BM, NTHR, RUN>::TPR;
  const GemmProblem& P = *t.P;
  const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
  const int per = (KB + TPR - 1) / TPR;
  a.k0 = min(KB, part * per);
  a.k1 = min(KB, a.k0 + per);
  const int ar = t.r0 + min(t.m0 + row, t.len - 1);
  const int grow = P.a_rows ? P.a_rows[ar] : ar;
  a.src = P.a_scale + (size_t)grow * KB;
  const int last = a.k1 - 1;   // >= 0 (KB >= 1); a thread past the row's end re-reads its last scale
#pragma unroll
  for (int i = 0; i < RUN; ++i) a.v[i] = __float_as_uint(a.src[min(a.k0 + i, last)]);
}

template <int BM, int NTHR, int RUN>
__device__ __forceinline__ void act_scales_store(ActScales<BM, NTHR, RUN>& a, uint8_t* ascl,
                                                 int KB) {
  constexpr int TPR = ActScales<BM, NTHR, RUN>::TPR;
  uint8_t* dst = ascl + (threadIdx.x / TPR) * KB;
  for (int base = a.k0;;) {
#pragma unroll
    for (int i = 0; i < RUN; ++i)
      if (base + i < a.k1) dst[base + i] = (uint8_t)(a.v[i] >> 23);
    base += RUN;
    if (base >= a.k1) break;
    const int last = a.k1 - 1;
#pragma unroll
    for (int i = 0; i < RUN; ++i) a.v[i] = __float_as_uint(a.src[min(base + i, last)]);
  }
}

constexpr int kActRun = 16;   // activation-scale loads in flight per thread

// The first STAGES - 1 stages of a tile's ring (issuing waves).
template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES,
          bool KTAIL>
__device__ __forceinline__ void ring_prologue(
    const RingTileState<RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>::LPI>& t,
    u32x4* ring) {
  using C = RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>;
  const int wvs = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = t.P->K, KT = KTAIL ? (K + BK - 1) / BK : K / BK;
  if (wvs >= C::NI) return;
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st) {
    if (st >= KT) break;
    const int kval = ring_stage_chunks<BK, C::AB, KTAIL>(K, st);
    if (C::B_AUX && t.stream)
      ring_issue<C::LPI, C::NI, STAGES, C::STAGE_CH, C::A_CH, BK, C::A_IT, C::WB, C::AB, C::B_AUX,
                 C::KCH, C::KCHB, BM>(t.ra, t.rb, t.voff, ring, st, wvs, kval);
    else
      ring_issue<C::LPI, C::NI, STAGES, C::STAGE_CH, C::A_CH, BK, C::A_IT, C::WB, C::AB, 0, C::KCH,
                 C::KCHB, BM>(t.ra, t.rb, t.voff, ring, st, wvs, kval);
  }
}

// The K loop of one tile into `acc`.
template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES,
          bool KTAIL>
__device__ __forceinline__ void ring_kloop(
    const RingTileState<RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>::LPI>& t,
    u32x4* ring, const float* scl,
    f32x4 (&acc)[RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>::TM]
               [RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>::TN]) {
  using C = RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>;
  constexpr int KCH = C::KCH, KCHB = C::KCHB, A_CH = C::A_CH, STAGE_CH = C::STAGE_CH;
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, WN = C::WN, LPI = C::LPI;
  int tid = threadIdx.x;
  // (FP8 activations: the lane's row addresses are computed per tile, not
  // kept live across the tile loop, where the quantizing epilogue needs the
  // registers)
  if constexpr (WF == 2) asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wv = tid >> 6;
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  const int wm = wv / C::WAVES_N, wn = wv % C::WAVES_N;
  int brow_of[TN];
#pragma unroll
  for (int ni = 0; ni < TN; ++ni) {
    if (MODE == 0)
      brow_of[ni] = (ni < TN / 2) ? wn * (WN / 2) + ni * 16
                                  : BN / 2 + wn * (WN / 2) + (ni - TN / 2) * 16;
    else
      brow_of[ni] = wn * WN + ni * 16;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int K = t.P->K;
  const int KT = KTAIL ? (K + BK - 1) / BK : K / BK;   // (KTAIL: the last stage is partial)
  const int KB = K / 128;               // WF: K blocks of the scales
  // WF: the scale group of this wave's weight fragments (GEMM 1: gate
  // fragments use group 0, up fragments group 1)
  const int g_down = MODE == 1 ? (wn * WN) / 128 : 0;
  // a wave whose rows all lie past the segment's end (the last row tile of a
  // segment) takes part in the copies and barriers only
  const bool rows_here = t.m0 + (wvs / C::WAVES_N) * WM < t.len;
  for (int kt = 0; kt < KT; ++kt) {
    // stage kt has landed once only the copies of later stages remain; the
    // waves that issue no copies (and write the output) have nothing to wait for
    if (wvs < C::NI) wait_stages<LPI, STAGES - 2>(min(STAGES - 2, KT - 1 - kt));
    if (WF) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the tile's scales are written
    raw_barrier();
    if (kt + STAGES - 1 < KT && wvs < C::NI) {
      const int kval = ring_stage_chunks<BK, C::AB, KTAIL>(K, kt + STAGES - 1);
      if (C::B_AUX && t.stream)
        ring_issue<LPI, C::NI, STAGES, STAGE_CH, A_CH, BK, C::A_IT, C::WB, C::AB, C::B_AUX, KCH,
                   KCHB, BM>(t.ra, t.rb, t.voff, ring, kt + STAGES - 1, wvs, kval);
      else
        ring_issue<LPI, C::NI, STAGES, STAGE_CH, A_CH, BK, C::A_IT, C::WB, C::AB, 0, KCH, KCHB,
                   BM>(t.ra, t.rb, t.voff, ring, kt + STAGES - 1, wvs, kval);
    }
    if (!rows_here) continue;
    const u32x4* slot = ring + (kt % STAGES) * STAGE_CH;
    if constexpr (WF == 2) {
      // E4M3 x E4M3: one 128-deep MFMA K step per stage.  Lane l supplies row
      // (or weight row) l % 16, chunks g and 4 + g (g = l / 16) of the 128-byte
      // piece, and its row's E8M0 scale (every lane of a row the same one: a
      // scale covers the whole 128-deep step).
      const uint8_t* ascl = reinterpret_cast<const uint8_t*>(scl + 2 * KB);
      const int g = lane >> 4;
      int sa[TM], sb[TN];
#pragma unroll
      for (int mi = 0; mi < TM; ++mi) sa[mi] = ascl[(wm * WM + mi * 16 + (lane & 15)) * KB + kt];
      const int e0 = (int)(__float_as_uint(scl[(MODE == 0 ? 0 : g_down) * KB + kt]) >> 23);
      const int e1 = (int)(__float_as_uint(scl[KB + kt]) >> 23);
#pragma unroll
      for (int ni = 0; ni < TN; ++ni) sb[ni] = (MODE == 0 && ni >= TN / 2) ? e1 : e0;
      i32x8 af[TM], bq[TN];
#pragma unroll
      for (int mi = 0; mi < TM; ++mi) {
        const int row = wm * WM + mi * 16 + (lane & 15);
        const u32x4 lo = slot[row * KCH + (g ^ swz<KCH>(row))];
        const u32x4 hi = slot[row * KCH + ((4 + g) ^ swz<KCH>(row))];
        af[mi] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int ni = 0; ni < TN; ++ni) {
        const int br = brow_of[ni] + (lane & 15);
        const u32x4* brow = slot + A_CH + br * KCHB;
        const u32x4 lo = brow[g ^ swz<KCHB>(BM + br)];
        const u32x4 hi = brow[(4 + g) ^ swz<KCHB>(BM + br)];
        bq[ni] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      // weights as the first operand: lane l gets output row l % 16 and
      // columns 4 (l / 16) .. +3 of each 16 x 16 piece (row-wise stores).
      // Weight fragment by weight fragment, so that the first MFMAs need only
      // the scales, the activation fragments and the first weight fragment;
      // the scheduler is told to place each later weight fragment's two reads
      // among the MFMAs of the one before.
#pragma unroll
      for (int ni = 0; ni < TN; ++ni)
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bq[ni], af[mi], acc[mi][ni], 0, 0, 0, sb[ni], 0, sa[mi]);
      constexpr int AHEAD = 2;   // weight fragments read ahead
      __builtin_amdgcn_sched_group_barrier(0x100, TM + (MODE == 0 ? 2 : 1) + 2 * TM + 2 * AHEAD, 0);
#pragma unroll
      for (int ni = 0; ni < TN; ++ni) {
        if (ni + AHEAD < TN) {
          __builtin_amdgcn_sched_group_barrier(0x008, TM / 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, TM - TM / 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, TM, 0);
        }
      }
    } else {
      float sc0 = 1.0f, sc1 = 1.0f;
      if (WF) {
        const int kb = kt * BK / 128;
        sc0 = scl[(MODE == 0 ? 0 : g_down) * KB + kb];
        sc1 = scl[KB + kb];
      }
      // Fragments of K step kk + 1 are read while the MFMAs of step kk run:
      // two register sets, and the scheduler is told to interleave the LDS
      // reads one by one among the MFMAs.  (WF: the weight fragment is read as
      // 8 codes and dequantized just before its MFMAs.)
      bf16x8 af[2][TM], bfr[2][TN];
      uint32_t b8[2][TN][2];
      auto load_frags = [&](int kk, bf16x8* a, bf16x8* b, uint32_t (*b8r)[2]) {
        const int ch = kk * 4 + (lane >> 4);
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) {
          const int row = wm * WM + mi * 16 + (lane & 15);
          a[mi] = __builtin_bit_cast(bf16x8, slot[row * KCH + (ch ^ swz<KCH>(row))]);
        }
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
          const int br = brow_of[ni] + (lane & 15);
          if (WF) {
            // codes of K kk*32 + q*8 .. +8: chunk 2*kk + q/2 of the row piece, half q % 2
            const int c = kk * 2 + ((lane >> 4) >> 1);
            const u32x2 v = reinterpret_cast<const u32x2*>(
                slot + A_CH + br * KCHB + (c ^ swz<KCHB>(BM + br)))[(lane >> 4) & 1];
            b8r[ni][0] = v.x;
            b8r[ni][1] = v.y;
          } else {
            const int row = BM + br;
            b[ni] = __builtin_bit_cast(bf16x8, slot[row * KCH + (ch ^ swz<KCH>(row))]);
          }
        }
      };
      load_frags(0, af[0], bfr[0], b8[0]);
#pragma unroll
      for (int kk = 0; kk < BK / 32; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < BK / 32) load_frags(kk + 1, af[cur ^ 1], bfr[cur ^ 1], b8[cur ^ 1]);
        if (WF) {
#pragma unroll
          for (int ni = 0; ni < TN; ++ni)
            bfr[cur][ni] = fp8x8_to_bf16(b8[cur][ni][0], b8[cur][ni][1],
                                         (MODE == 0 && ni >= TN / 2) ? sc1 : sc0);
        }
        if constexpr (WF == 0) {
          // weight fragment by weight fragment: the step's first MFMAs need
          // only its activation fragments and its first two weight fragments,
          // the rest of its reads (and the next step's) go among the MFMAs
#pragma unroll
          for (int ni = 0; ni < TN; ++ni)
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[cur][ni], af[cur][mi],
                                                                    acc[mi][ni], 0, 0, 0);
          constexpr int first = TM + 2;
          const int rest = (kk == 0 ? TN - 2 : 0) + (kk + 1 < BK / 32 ? TM + TN : 0);
          if (kk == 0) __builtin_amdgcn_sched_group_barrier(0x100, first, 0);
          if (rest > 0) {
            constexpr int R0 = TN - 2 + TM + TN;   // kk == 0 (BK / 32 > 1)
            constexpr int per0 = (TM * TN) / R0;
            static_assert(BK / 32 == 2, "two K steps per stage");
            if (kk == 0) {
#pragma unroll
              for (int i = 0; i < R0; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, per0, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              }
              __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - per0 * R0, 0);
            }
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
          }
        } else {
        // E4M3 weights: activation fragment by activation fragment, the
        // step's dequantized weight fragments all formed first
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
          for (int ni = 0; ni < TN; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[cur][ni], af[cur][mi],
                                                                  acc[mi][ni], 0, 0, 0);
        if (kk == 0) {
          // first: this step's own fragment reads
          __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
        }
        if (kk + 1 < BK / 32) {
          constexpr int per = (TM * TN) / (TM + TN);
#pragma unroll
          for (int i = 0; i < TM + TN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, per, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - per * (TM + TN), 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
        }
        }
      }
    }
  }
}

// The tile's output: lane l holds row l % 16 of each 16 x 16 piece and its
// columns 4 (l / 16) .. +3 (the weights are the MFMAs' first operand).
// ring_pack turns them into bf16 pairs (SwiGLU for GEMM 1; the rows' output
// scale `rsc` for GEMM 2) right after the K loop; ring_store stages each
// wave's rows in its own part of the idle ring and writes them as 16-byte
// row chunks, a row past the segment or columns past N getting an offset
// past the store's range (the largest range, 2^31 - 64 elements of 2 bytes,
// ends below it), so that they are dropped.
template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES>
__device__ __forceinline__ void ring_pack(
    const f32x4 (&acc)[RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>::TM]
                     [RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>::TN],
    const float* rsc, u32x2* out) {
  using C = RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>;
  constexpr int TM = C::TM, TN = C::TN, NPM = MODE == 0 ? TN / 2 : TN;
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NPM; ++ni) {
      if (MODE == 0) {
        const f32x4 g = acc[mi][ni], u = acc[mi][ni + TN / 2];
        out[mi * NPM + ni] = u32x2{pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]),
                                   pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3])};
      } else {
        const f32x4 y = acc[mi][ni];
        const float sc = rsc[mi];
        out[mi * NPM + ni] =
            u32x2{pack_bf16x2(y[0] * sc, y[1] * sc), pack_bf16x2(y[2] * sc, y[3] * sc)};
      }
    }
  }
}

template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES>
__device__ __forceinline__ void ring_store(
    const RingTileState<RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>::LPI>& t,
    const u32x2* out, u32x4* ring) {
  using C = RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>;
  constexpr int TM = C::TM, WM = C::WM, WN = C::WN, NPM = MODE == 0 ? C::TN / 2 : C::TN;
  constexpr int COUT = MODE == 0 ? WN / 2 : WN;   // output columns of a wave
  constexpr int CPR = COUT / 8;                   // 16-byte chunks per output row
  constexpr int LPR = CPR;                        // lanes reading one row
  constexpr int RPI = 64 / LPR;                   // rows per store instruction
  static_assert(CPR <= 16 && 64 % LPR == 0 && WM % RPI == 0, "output transpose shape");
  // (the lane number is made opaque here, so that the compiler computes these
  // lane-only addresses per tile instead of keeping them live through the K
  // loop, where the registers are all taken)
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wv = threadIdx.x >> 6;
  const int wm = wv / C::WAVES_N, wn = wv % C::WAVES_N;
  // this wave's region of the (idle) ring: WM rows of CPR chunks, chunk c of
  // row r at c ^ (r % CPR), so that the 16 rows one write instruction
  // touches and the chunks one read instruction touches hit distinct banks
  u32x4* reg = ring + (size_t)wv * WM * CPR;
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) {
    const int r = mi * 16 + (lane & 15);
#pragma unroll
    for (int ni = 0; ni < NPM; ++ni) {
      const int c = ni * 2 + ((lane >> 4) >> 1);        // 16-byte chunk of columns 4q..4q+3
      reinterpret_cast<u32x2*>(reg + r * CPR + (c ^ (r % CPR)))[(lane >> 4) & 1] =
          out[mi * NPM + ni];
    }
  }
  const GemmProblem& P = *t.P;
  const int N = P.N;
  const __amdgpu_buffer_rsrc_t rc =
      buffer_rsrc(P.C + (size_t)t.r0 * N, (uint32_t)((size_t)t.len * N * 2));
  const int col0 = t.n0 + wn * COUT;
#pragma unroll
  for (int it = 0; it < WM / RPI; ++it) {
    const int r = it * RPI + lane / LPR, c = lane % LPR;
    const u32x4 v = reg[r * CPR + (c ^ (r % CPR))];
    const int row = t.m0 + wm * WM + r, col = col0 + c * 8;
    // N % 64 == 0 for these tiles: the 8 columns are in or out together
    const uint32_t off = (row < t.len && col < N)
                             ? ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 2u
                             : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, MODE == 1 ? kAuxNT : 0);
  }
}

// GEMM 1 with E4M3 activations: a tile's BN / 2 = 128 h columns (n0 is a
// multiple of 128) are exactly one 1 x 128 piece of each of its rows, so the
// tile quantizes h itself and GEMM 2 reads the codes: no bf16 h round trip
// through HBM and no quantizer launch between the GEMMs.  The bf16 h values
// are staged as in ring_store; after a barrier, 8 lanes take one row (16
// columns each, two staged chunks), reduce the row's maximum with lane
// shuffles, and write its 128 codes as 16-byte pieces of one 128-byte line
// and its power-of-two scale.  The codes are those a separate quantizer would
// give on the bf16 h this tile would have written.
template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES>
__device__ __forceinline__ void ring_store_q(
    const RingTileState<RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>::LPI>& t,
    const u32x2* out, u32x4* ring) {
  using C = RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>;
  constexpr int TM = C::TM, WM = C::WM, WN = C::WN, NPM = C::TN / 2;
  constexpr int COUT = WN / 2;                    // h columns of a wave
  constexpr int CPR = COUT / 8;                   // 16-byte chunks per staged row
  constexpr int RPP = NTHR / 8;                   // rows per pass
  static_assert(MODE == 0 && WF == 2 && BN == 256, "one 1 x 128 piece per row of a tile");
  static_assert(BM % RPP == 0 && 16 % CPR == 0, "row pass shape");
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wv = threadIdx.x >> 6;
  u32x4* reg = ring + (size_t)wv * WM * CPR;
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) {
    const int r = mi * 16 + (lane & 15);
#pragma unroll
    for (int ni = 0; ni < NPM; ++ni) {
      const int c = ni * 2 + ((lane >> 4) >> 1);
      reinterpret_cast<u32x2*>(reg + r * CPR + (c ^ (r % CPR)))[(lane >> 4) & 1] =
          out[mi * NPM + ni];
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  raw_barrier();   // every wave's rows are staged
  const GemmProblem& P = *t.P;
  const int N = P.N;
  const __amdgpu_buffer_rsrc_t rq =
      buffer_rsrc(P.Cq + (size_t)t.r0 * N, (uint32_t)((size_t)t.len * N));
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int sub = tid & 7;
#pragma unroll
  for (int it = 0; it < BM / RPP; ++it) {
    const int R = it * RPP + (tid >> 3);          // row of the tile
    const int wm = R / WM, r = R % WM;
    u32x4 v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int cc = sub * 2 + j;                 // chunk of the row's 16
      const int wn = cc / CPR, c = cc % CPR;
      v[j] = ring[(size_t)(wm * C::WAVES_N + wn) * WM * CPR + r * CPR + (c ^ (r % CPR))];
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(v[j][w] << 16)),
                                 fabsf(__uint_as_float(v[j][w] & 0xffff0000u))));
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 8));
    const int sx = fp8_dev::block_exponent(amax);
    u32x4 codes;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t a = v[j][2 * w], b = v[j][2 * w + 1];
        codes[2 * j + w] = fp8_dev::e4m3x4(ldexpf(__uint_as_float(a << 16), -sx),
                                           ldexpf(__uint_as_float(a & 0xffff0000u), -sx),
                                           ldexpf(__uint_as_float(b << 16), -sx),
                                           ldexpf(__uint_as_float(b & 0xffff0000u), -sx));
      }
    const int row = t.m0 + R;
    const uint32_t off =
        row < t.len ? (uint32_t)row * (uint32_t)N + (uint32_t)(t.n0 + sub * 16) : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_buffer_store_b128(codes, rq, off, 0, 0);
    if (sub == 0 && row < t.len)
      P.c_scale[(size_t)(t.r0 + row) * (N / 128) + t.n0 / 128] = fp8_dev::pow2(sx);
  }
}

// One ring tile: set up, issue its first stages, run `after_issue` (every
// wave), the K loop, then the epilogue through the ring.  Starts with a
// barrier after which the ring and the scales are free (the previous tile's
// output is out).
template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES,
          bool KTAIL, typename Hook>
__device__ __forceinline__ void ring_tile(const GemmArgs& args, const int* tiles_l, int tile,
                                          u32x4* ring, float* scl, Hook after_issue) {
  using C = RingCfg<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv / C::WAVES_N;
  constexpr int NPM = MODE == 0 ? C::TN / 2 : C::TN;
  RingTileState<C::LPI> cur;
  ring_setup<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>(args, tiles_l, tile, cur);
  raw_barrier();
  ring_scales<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>(cur, scl, threadIdx.x, NTHR);
  if constexpr (WF == 2) {
    const int KB = cur.P->K / 128;
    ActScales<BM, NTHR, kActRun> as;
    act_scales_load(cur, KB, as);
    ring_prologue<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES, KTAIL>(cur, ring);
    act_scales_store(as, reinterpret_cast<uint8_t*>(scl + 2 * KB), KB);
  } else {
    ring_prologue<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES, KTAIL>(cur, ring);
  }
  after_issue();
  u32x2 outv[C::TM * NPM];
  {
    f32x4 acc[C::TM][C::TN];
    ring_kloop<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES, KTAIL>(cur, ring, scl, acc);
    // this tile's output scales (GEMM 2)
    float rsc[C::TM];
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi) {
      const int row = cur.m0 + wm * C::WM + mi * 16 + (lane & 15);
      rsc[mi] = (MODE == 1 && cur.P->scale) ? cur.P->scale[cur.r0 + min(row, cur.len - 1)] : 1.0f;
    }
    ring_pack<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>(acc, rsc, outv);
  }
  raw_barrier();   // every wave is done reading the ring: it takes the output
  if constexpr (MODE == 0 && WF == 2)
    ring_store_q<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>(cur, outv, ring);
  else
    ring_store<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES>(cur, outv, ring);
}

// Persistent schedule: workgroup l (XCD-remapped) takes tiles l, l + G, ...
// KTAIL: some problem's K is not a multiple of BK (bf16 only).
template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES, int OCC,
          bool KTAIL>
__global__ __launch_bounds__(NTHR, OCC) void gemm_ring_kernel(GemmArgs args) {
  // The ring and the tile table are this kernel's only LDS objects: with a
  // third one the compiler can no longer tell the operand reads from the
  // in-flight ring copies and waits for every copy before each stage's first
  // read (measured 15-30% slower).  The table build's scan scratch therefore
  // borrows the ring, which is idle until the first tile.
  // (WF: the dynamic LDS also holds a tile's block scales, after the table.)
  __shared__ __attribute__((aligned(1024))) u32x4 ring[RingShape<WF, BM, BN, BK, STAGES>::RING_CH];
  extern __shared__ int tiles_l[];
  build_tile_table<NTHR>(args, tiles_l, reinterpret_cast<int*>(ring), args.tile_bm,
                         args.tile_ncols, args.min_len, args.max_len);
  const int total = tiles_l[args.n_seg_total];
  float* scl = reinterpret_cast<float*>(tiles_l + args.n_seg_total + 1);
  const int G = gridDim.x;
  for (int tile = xcd_logical(blockIdx.x, G); tile < total; tile += G)
    ring_tile<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES, KTAIL>(args, tiles_l, tile, ring,
                                                                   scl, [] {});
}

// Ring-tile shapes: BM, BN, BK, threads, waves along M, ring stages.  "big"
// for segments of at least kBigRows rows, "mid" for the rest.
constexpr int kBigRows = 256;

template <int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES>
struct TileCfg {
  static constexpr int kRingBytes = RingShape<WF, BM, BN, BK, STAGES>::RING_CH * 16;
  static constexpr int kThreads = NTHR;
  static constexpr int kBM = BM, kBN = BN, kBK = BK, kWM = WAVES_M, kStages = STAGES;
};
// tile shapes per operand format
template <int WF> struct Tiles;
// kSmallRows: segments shorter than this take the Small shape in a launch of
// their own (0: no such launch).
template <> struct Tiles<0> {                              // bf16
  using Mid = TileCfg<0, 128, 256, 64, 512, 2, 3>;         // 2 x 4 waves of 64 x 64
  using Big = TileCfg<0, 256, 256, 64, 512, 4, 2>;         // 4 x 2 waves of 64 x 128
  using Small = Mid;
  static constexpr int kSmallRows = 0;
};
// E4M3 weights: the weight rows of a stage take half the bytes.  The
// 128-row tile takes 128-deep stages (two), so that a stage's weight row
// piece is a whole 128-byte line rather than half of one (the other half
// fetched again a stage later): 4-6% faster on its launches than four
// 64-deep stages.  The 256-row tile keeps 64-deep stages, one more than
// bf16 (128-deep ones would not fit twice), and 2 x 4 waves of 128 x 64
// rather than bf16's 4 x 2 of 64 x 128: every wave dequantizes the weight
// fragments it reads, so half as many weight columns per wave halves the
// conversions (for 25% more activation reads): 4-9% faster on its launches.
// (With bf16 weights the two layouts read the same LDS bytes and time the
// same.)  Two 128-deep stages of the 128-row tile keep one stage of weights
// in flight per CU, which holds its weight stream to 3.4-3.8 TB/s, where the
// bf16 tile's three stages reach 5.7-6.6.  Segments of fewer than 64 rows
// (most of the DeepSeek-shaped layer's) take a 64-row tile instead, whose
// 48 KiB stages fit three times: 12-23% faster on those launches.  The
// longer ones stay on the 128-row tile: as two 64-row tiles the prefill
// layer's 100-260-row segments ran 10-22% slower.
template <> struct Tiles<1> {
  using Mid = TileCfg<1, 128, 256, 128, 512, 2, 2>;
  using Big = TileCfg<1, 256, 256, 64, 512, 2, 3>;   // 2 x 4 waves of 128 x 64
  using Small = TileCfg<1, 64, 256, 128, 512, 2, 3>;  // 2 x 4 waves of 32 x 64
  static constexpr int kSmallRows = 64;
};
// E4M3 activations and weights: 128-deep stages (128-byte row pieces, as the
// bf16 tiles' 64-deep ones), one scaled FP8 MFMA K step each.
template <> struct Tiles<2> {
  using Mid = TileCfg<2, 128, 256, 128, 512, 2, 3>;
  using Big = TileCfg<2, 256, 256, 128, 512, 4, 2>;
  using Small = Mid;
  static constexpr int kSmallRows = 0;
};



// ---------------------------------------------------------------- fp32 path
// GEMM 1 writes h, GEMM 2 writes y.
__device__ int find_segment(const int32_t* off, int n, int r) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// fp32 grouped GEMMs (the fp32 layer is tiny: a few rows per expert): one
// wave per output element.  Its lanes stride K, so every load instruction
// reads consecutive elements of an A row and of a weight row, and the wave
// sums the 64 partial dot products in registers.
template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B,
                                                       float* __restrict__ C,
                                                       const float* __restrict__ scale,
                                                       const int32_t* __restrict__ seg_offsets,
                                                       const int32_t* __restrict__ seg_expert,
                                                       const int32_t* __restrict__ a_rows,
                                                       int n_seg, int rows, int N, int K,
                                                       int up_off, int64_t b_stride, int n_w) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int row = (int)(w / N), col = (int)(w % N);
  // (every exit below is taken by the whole wave: its row and column are
  // the wave's)
  if (row >= rows) return;
  int e = 0;
  if (seg_offsets) {
    if (row >= seg_offsets[n_seg]) return;
    e = seg_expert[find_segment(seg_offsets, n_seg, row)];
    if ((unsigned)e >= (unsigned)n_w) return;   // padding segment
  }
  const float* a = A + (size_t)(a_rows ? a_rows[row] : row) * K;
  const float* b = B + (size_t)e * b_stride;
  if (MODE == 0) {
    const float* bg = b + (size_t)col * K;
    const float* bu = b + (size_t)(up_off + col) * K;
    float g = 0.f, u = 0.f;
    for (int kk = lane; kk < K; kk += 64) {
      const float x = a[kk];
      g = fmaf(x, bg[kk], g);
      u = fmaf(x, bu[kk], u);
    }
    g = wave_dev::sum(g);
    u = wave_dev::sum(u);
    if (lane == 0) C[(size_t)row * N + col] = silu(g) * u;
  } else {
    const float* bd = b + (size_t)col * K;
    float y = 0.f;
    for (int kk = lane; kk < K; kk += 64) y = fmaf(a[kk], bd[kk], y);
    y = wave_dev::sum(y);
    if (lane == 0) C[(size_t)row * N + col] = y * (scale ? scale[row] : 1.0f);
  }
}

// ---------------------------------------------------------------- bf16 decode tiles
// Segments of a few rows (decode): the FFN is bound by reading each active
// expert's weights once, and HBM only reaches its practical rate with many
// waves per CU each keeping loads in flight.  So the tile is small -- 16
// activation rows x BN weight rows -- and so is its footprint: one LDS stage
// holds the BN x BK weight slice (loaded coalesced, whole rows, and
// XOR-swizzled), the next stage is prefetched in registers while the current
// one is consumed, and activation fragments come straight from L2 into MFMA
// registers (rows past the segment end are never loaded).  The four waves
// split each stage's K and reduce their partial sums through LDS at the end
// of the tile, so every wave issues MFMAs even on one-row segments.
// Waves per SIMD of the decode tiles (their register budgets keep the K loop
// free of spills): bf16 6 (8 spilled, 6% slower); E4M3 weights 5 (codes in
// LDS); E4M3 weights and activations 4.
constexpr int kDecodeWaves = 6, kDecodeWavesF8 = 5, kDecodeWavesW8A8 = 4;
// One activation fragment of the decode tiles, 8 consecutive K elements of
// row `arow` starting at element offset `off` (K index k), as loaded: bf16,
// or (WF = 2) 8 E4M3 codes in .x/.y with their 1 x 128 piece scale's bits in
// .z.  decode_a_bf16 turns a loaded fragment into the MFMA operand (codes
// times scale, exact); loads and conversions are apart so that the
// one-stage-ahead prefetch does not wait for its own loads.
// Weight chunks of the decode tiles are read once per layer call, so they
// are loaded non-temporal: measured 7% faster on the bf16 decode layer (6.4
// against 6.0 TB/s), 10% with E4M3 weights, bit-identical results.
// E4M3 weights in the decode tiles: the codes go into LDS as they are and are
// dequantized at the operand read, so a 512-deep stage takes 16 KiB of LDS
// (as a bf16 256-deep one) instead of 32 KiB of dequantized bf16, which had
// held a CU to 4 workgroups.  Measured with the waves per SIMD above: FP8-weight
// decode FFN 7% faster, W8A8 6%, bit-identical.
// A weight chunk of the decode tiles (non-temporal, as above).
__device__ __forceinline__ u32x4 decode_w_chunk(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
template <int WF>
__device__ __forceinline__ u32x4 decode_a_frag(const GemmProblem& P, bool ok, uint32_t off,
                                               int arow, int k) {
  if (!ok) return u32x4{0u, 0u, 0u, 0u};
  if constexpr (WF == 2) {
    const u32x2 c = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(P.A) + off);
    const float sc = P.a_scale[(size_t)arow * (P.K / 128) + k / 128];
    return u32x4{c.x, c.y, __float_as_uint(sc), 0u};
  } else {
    return *reinterpret_cast<const u32x4*>(P.A + off);
  }
}
template <int WF>
__device__ __forceinline__ u32x4 decode_a_bf16(u32x4 f) {
  if constexpr (WF == 2) return __builtin_bit_cast(u32x4, fp8x8_to_bf16(f.x, f.y, __uint_as_float(f.z)));
  else return f;
}

// WF = 1: E4M3 weights with 128 x 128 block scales, loaded as 16-byte chunks
// of 16 codes, kept as codes in LDS and dequantized (exactly) to bf16 at the
// operand read.  WF = 2: E4M3 activations too (see decode_a_frag).
template <int MODE, int WF, int BN, int BK, int MT, int WAVES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WAVES)))
void gemm_decode_kernel(GemmArgs args) {
  constexpr int BM = 16 * MT;                    // rows per tile (MT subtiles of 16)
  constexpr int KCH = BK / 8;                    // 16-byte bf16 chunks per row
  constexpr int LCH = WF ? BK / 16 : KCH;        // 16-byte chunks per row as loaded
  constexpr int B_CH = BN * LCH / 256;           // loaded chunks per thread per stage
  constexpr int WB = WF ? 1 : 2;                 // bytes per weight
  constexpr int AB = WF == 2 ? 1 : 2;            // bytes per activation element
  constexpr int KPW = BK / 32 / 4;               // MFMA K steps per wave per stage
  constexpr int TN = BN / 16;                    // n subtiles
  static_assert(KPW >= 1 && B_CH >= 1, "tile shape");
  // E4M3 weights stay codes in LDS (LDS_CH chunks of 16 codes per row) and
  // are dequantized at the operand read, so a stage takes as much LDS as a
  // bf16 one and as many workgroups fit per CU
  constexpr bool F8LDS = WF >= 1;
  constexpr int LDS_CH = LCH;
  static_assert(!F8LDS || KPW * 32 == 128, "a wave's K steps of a stage share one scale block");
  __shared__ __attribute__((aligned(1024))) u32x4 Bs[BN * LDS_CH];   // swizzled rows: keep banks
  extern __shared__ int tiles_l[];
  f32x4 (*red)[TN][64] = reinterpret_cast<f32x4 (*)[TN][64]>(&Bs[0]);  // after the K loop
  static_assert(sizeof(f32x4) * 4 * TN * 64 <= sizeof(u32x4) * BN * LDS_CH, "reduction fits");

  __shared__ int wsum[256 / 64 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nst = args.n_seg_total;
  build_tile_table<256>(args, tiles_l, wsum, args.tile_bm, args.tile_ncols, args.min_len,
                        args.max_len);
  const int total = tiles_l[nst];
  const int G = gridDim.x;
  const int logical = xcd_logical(blockIdx.x, G);
  const int r = lane & 15, q = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  for (int tile = logical; tile < total; tile += G) {
    int lo = 0, hi = nst - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (tiles_l[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int gs = lo;
    const int pi = gs < args.p[0].n_seg ? 0 : 1;
    const GemmProblem& P = args.p[pi];
    int r0, len, e;
    seg_range(P, gs - (pi ? args.p[0].n_seg : 0), r0, len, e);
    const int mt = (len + BM - 1) / BM;
    const int local = tile - tiles_l[gs];
    const int m0 = (local % mt) * BM;
    const int n0 = (local / mt) * (MODE == 0 ? BN / 2 : BN);
    const int K = P.K, N = P.N;
    const uint8_t* Bb = reinterpret_cast<const uint8_t*>(P.B) + (size_t)e * P.b_stride * WB;
    const float* Sb = WF ? P.b_scale + (size_t)e * P.s_stride : nullptr;

    // byte offsets (within this expert's matrix) of this thread's chunks
    uint32_t b_off[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + 256 * i, row = c / LCH, kc = c % LCH;
      int brow;
      if (MODE == 0) {
        const int col = min(n0 + (row % (BN / 2)), N - 1);
        brow = row < BN / 2 ? col : P.up_off + col;
      } else {
        brow = min(n0 + row, N - 1);
      }
      b_off[i] = ((uint32_t)brow * (uint32_t)K + kc * (16 / WB)) * WB;
    }
    // this lane's activation row and its K offsets inside a stage (WF = 2:
    // E4M3 codes, dequantized with their 1 x 128 scale on the way to the MFMA)
    // WF: the scale index at k = 0 of each 16-row group's 128-row block
    // (GEMM 1: the gate rows n0.., the up rows up_off + n0..; GEMM 2: rows
    // n0 + 16 j.., all in one block since n0 is a multiple of BN and N of
    // 128); wave wv reads K block wv of every stage.  Uniform over the wave,
    // so the scales are scalar loads.
    int g_sc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row0 = MODE == 0 ? (j < TN / 2 ? n0 : P.up_off + n0) : n0 + j * 16;
      g_sc[j] = __builtin_amdgcn_readfirstlane((row0 / 128) * (K / 128) + wv);
    }
    bool a_ok[MT];
    uint32_t a_off[MT];
    int a_row[MT];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      a_ok[mi] = m0 + mi * 16 + r < len;
      const int ar = r0 + min(m0 + mi * 16 + r, len - 1);
      a_row[mi] = P.a_rows ? P.a_rows[ar] : ar;
      a_off[mi] = (uint32_t)a_row[mi] * (uint32_t)K + (wv * KPW * 32 + q * 8);
    }
    (void)AB;

    f32x4 acc[MT][TN];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[mi][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 rb[B_CH], ra[MT][KPW];
    float gsc[TN];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = decode_w_chunk(Bb + b_off[i]);
    if constexpr (F8LDS) {
#pragma unroll
      for (int j = 0; j < TN; ++j) gsc[j] = Sb[g_sc[j]];
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int jj = 0; jj < KPW; ++jj)
        ra[mi][jj] = decode_a_frag<WF>(P, a_ok[mi], a_off[mi] + jj * 32, a_row[mi],
                                       wv * KPW * 32 + jj * 32);

    const int KT = K / BK;
    for (int kt = 0; kt < KT; ++kt) {
      __syncthreads();  // everyone done with the previous stage (or tile)
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + 256 * i, row = c / LCH, kc = c % LCH;
        Bs[row * LDS_CH + (kc ^ (row & 7))] = rb[i];
      }
      __syncthreads();
      float sc[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) sc[j] = F8LDS ? gsc[j] : 1.0f;
      u32x4 ac[MT][KPW];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int jj = 0; jj < KPW; ++jj) ac[mi][jj] = decode_a_bf16<WF>(ra[mi][jj]);
      if (kt + 1 < KT) {
        const int koff = (kt + 1) * BK;
#pragma unroll
        for (int i = 0; i < B_CH; ++i) rb[i] = decode_w_chunk(Bb + b_off[i] + koff * WB);
        if constexpr (F8LDS) {
#pragma unroll
          for (int j = 0; j < TN; ++j) gsc[j] = Sb[g_sc[j] + koff / 128];
        } else {
#pragma unroll
          for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int jj = 0; jj < KPW; ++jj)
              ra[mi][jj] = decode_a_frag<WF>(P, a_ok[mi], a_off[mi] + koff + jj * 32,
                                             a_row[mi], koff + wv * KPW * 32 + jj * 32);
        }
      }
#pragma unroll
      for (int jj = 0; jj < KPW; ++jj) {
        const int ch = (wv * KPW + jj) * 4 + q;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = j * 16 + r;
          bf16x8 b;
          if constexpr (F8LDS) {
            // codes of bf16 chunk ch: half ch % 2 of code chunk ch / 2
            const int cc = ch >> 1;
            const u32x2 v = reinterpret_cast<const u32x2*>(&Bs[row * LDS_CH + (cc ^ (row & 7))])[ch & 1];
            b = fp8x8_to_bf16(v.x, v.y, sc[j]);
          } else {
            b = __builtin_bit_cast(bf16x8, Bs[row * KCH + (ch ^ (row & 7))]);
          }
#pragma unroll
          for (int mi = 0; mi < MT; ++mi)
            acc[mi][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, ac[mi][jj]), b, acc[mi][j], 0, 0, 0);
        }
        // (E4M3: one K step's fragments at a time, so that the converted
        // operands of later steps do not all stay live)
        if constexpr (F8LDS) __builtin_amdgcn_sched_barrier(0);
      }
      // E4M3: the next stage's activation fragments are fetched after this
      // stage's MFMAs, when its own are dead (they are L2 hits, and the next
      // stage first waits for its weight chunks anyway)
      if constexpr (F8LDS) {
        if (kt + 1 < KT) {
          const int koff = (kt + 1) * BK;
#pragma unroll
          for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int jj = 0; jj < KPW; ++jj)
              ra[mi][jj] = decode_a_frag<WF>(P, a_ok[mi], a_off[mi] + koff + jj * 32,
                                             a_row[mi], koff + wv * KPW * 32 + jj * 32);
        }
      }
    }

    // split-K reduction over the four waves, one 16-row subtile at a time,
    // then the epilogue on wave 0
    uint16_t* Cb = P.C + (size_t)r0 * N;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      if (m0 + mi * 16 >= len) break;  // uniform over the workgroup
      __syncthreads();
#pragma unroll
      for (int j = 0; j < TN; ++j) red[wv][j][lane] = acc[mi][j];
      __syncthreads();
      if (wv == 0) {
        f32x4 v[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) v[j] = acc[mi][j] + red[1][j][lane] + red[2][j][lane] + red[3][j][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m0 + mi * 16 + q * 4 + i;
          if (row >= len) continue;
          if (MODE == 0) {
#pragma unroll
            for (int j = 0; j < TN / 2; ++j) {
              const int col = n0 + j * 16 + r;
              if (col < N) Cb[(size_t)row * N + col] = to_bf16(silu(v[j][i]) * v[j + TN / 2][i]);
            }
          } else {
            const float sc = P.scale ? P.scale[r0 + row] : 1.0f;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int col = n0 + j * 16 + r;
              if (col < N) Cb[(size_t)row * N + col] = to_bf16(v[j][i] * sc);
            }
          }
        }
      }
    }
  }
}

// decode tiles: GEMM 1 32 weight rows (16 h columns) x K 256; GEMM 2 32 rows x K 256
// (512-deep bf16 stages measured 0.5% slower)
constexpr int DBN1 = 32, DBK1 = 256, DBN2 = 32, DBK2 = 256;
// E4M3 weights: twice the K per stage, so that a stage moves as many bytes
// (and keeps as many in flight) as with bf16 weights (256-deep: 4% slower)
constexpr int kDbkF8 = 512;
template <int WF> constexpr int decode_bk1() { return WF ? kDbkF8 : DBK1; }
template <int WF> constexpr int decode_bk2() { return WF ? kDbkF8 : DBK2; }

// Persistent grid: as many workgroups as can be resident at once (a larger
// grid would run its excess only after others finish), a multiple of 8 so
// that the XCD remap is a bijection.  The occupancy query's own error (it
// refuses some large-LDS kernels that launch fine) is cleared so that it is
// not reported as a launch failure; `fallback` workgroups per CU are used
// then.  Results are cached per kernel and LDS size.
// (The cache is shared by every host thread that calls the library: guarded.)
template <typename Kern>
int persistent_grid(Kern kernel, size_t dyn_lds, int fallback, int threads = 256) {
  struct Entry { const void* k; size_t lds; int dev; int per_cu; };
  static Entry cache[64];
  static int n_cache = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const void* key = reinterpret_cast<const void*>(kernel);
  int per_cu = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cache; ++i)
      if (cache[i].k == key && cache[i].lds == dyn_lds && cache[i].dev == dev) per_cu = cache[i].per_cu;
  }
  if (per_cu == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, dyn_lds) != hipSuccess ||
        per_cu < 1) {
      (void)hipGetLastError();
      per_cu = fallback;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (n_cache < 64) cache[n_cache++] = Entry{key, dyn_lds, dev, per_cu};
  }
  const int g = device_cu_count() * per_cu / 8 * 8;
  return g > 8 ? g : 8;
}

// Dynamic LDS of a ring launch: the tile table, and (E4M3 weights) a tile's
// block scales: 2 groups x K/128 floats for the longest K of the problems.
// Dynamic LDS of a ring launch: the tile table, then (FP8 weights) a tile's
// two groups of weight block scales, then (FP8 activations) the E8M0 bytes
// of its BM rows' scales.
inline size_t ring_dyn_lds(const GemmArgs& g, int wf, int bm) {
  int kmax = 0;
  for (int p = 0; p < g.n_probs; ++p) kmax = g.p[p].K > kmax ? g.p[p].K : kmax;
  const size_t kb = (size_t)(kmax / 128);
  return (size_t)(g.n_seg_total + 1) * sizeof(int) + (wf ? 2 * kb * 4 : 0) +
         (wf == 2 ? (size_t)bm * kb : 0);
}

template <int MODE, int WF, int BM, int BN, int BK, int NTHR, int WAVES_M, int STAGES>
void launch_ring(const GemmArgs& g, hipStream_t s) {
  const size_t dyn = ring_dyn_lds(g, WF, BM);
  bool tail = false;
  for (int p = 0; p < g.n_probs; ++p) tail = tail || g.p[p].K % BK != 0;
  if constexpr (WF == 0) {
    if (tail) {
      auto k = gemm_ring_kernel<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES, 1, true>;
      k<<<persistent_grid(k, dyn, 1, NTHR), NTHR, dyn, s>>>(g);
      return;
    }
  }
  auto k = gemm_ring_kernel<MODE, WF, BM, BN, BK, NTHR, WAVES_M, STAGES, 1, false>;
  k<<<persistent_grid(k, dyn, 1, NTHR), NTHR, dyn, s>>>(g);
}

}  // namespace

namespace {

constexpr int kAll = 0x7fffffff;

GemmArgs cover(GemmArgs g, int bm, int ncols, int min_len, int max_len) {
  g.tile_bm = bm;
  g.tile_ncols = ncols;
  g.min_len = min_len;
  g.max_len = max_len;
  return g;
}

// Between the two GEMMs of an FP8-activation pair: h of every problem, as
// GEMM 1 wrote it in bf16, quantized in 1 x 128 pieces for GEMM 2.
template <int WF>
void quantize_h(const FfnProblem* probs, int n_probs, hipStream_t s) {
  if constexpr (WF == 2) {
    for (int p = 0; p < n_probs; ++p)
      launch_quantize_rows_fp8(probs[p].rows, probs[p].Iw, probs[p].h, probs[p].h_q,
                               probs[p].h_scale, s);
  }
}

// FP8 activations on the decode tiles: the activation codes are dequantized
// to bf16 once (E4M3 value times its power-of-two scale, exact), h is
// rounded through E4M3 in place between the launches, and the FP8-weight
// decode tiles run on them.  Those are the bf16 operands the E4M3-activation
// decode tiles form fragment by fragment, in the same K order, so the
// results are the same bit for bit; the FP8-weight tiles read 16-byte
// activation fragments without per-fragment scale loads (measured ~10%
// faster).  Needs the a_deq scratch and one activation matrix for all
// problems (the layer's routed and shared problems both read x); returns
// false otherwise, and the E4M3-activation decode tiles run.
bool w8a8_on_fp8w_decode(const moe_config& c, const FfnProblem* probs, int n_probs,
                         const GemmArgs& g1, const GemmArgs& g2, size_t lds_tiles,
                         hipStream_t s) {
  if (!probs[0].a_deq) return false;
  for (int p = 1; p < n_probs; ++p)
    if (probs[p].A != probs[0].A || probs[p].a_scale != probs[0].a_scale) return false;
  int64_t a_rows = 0;
  for (int p = 0; p < n_probs; ++p)
    a_rows = g1.p[p].a_ld_rows > a_rows ? g1.p[p].a_ld_rows : a_rows;
  if ((size_t)a_rows * c.H * 2 > probs[0].a_deq_bytes) return false;
  launch_dequantize_rows_fp8(a_rows, c.H, (const uint8_t*)probs[0].A, probs[0].a_scale,
                             probs[0].a_deq, s);
  GemmArgs d1 = g1, d2 = g2;
  for (int p = 0; p < n_probs; ++p) {
    d1.p[p].A = (const uint16_t*)probs[0].a_deq;
    d1.p[p].a_scale = nullptr;
    d2.p[p].A = (const uint16_t*)probs[p].h;
    d2.p[p].a_scale = nullptr;
  }
  auto k1 = gemm_decode_kernel<0, 1, DBN1, decode_bk1<1>(), 1, kDecodeWavesF8>;
  auto k2 = gemm_decode_kernel<1, 1, DBN2, decode_bk2<1>(), 1, kDecodeWavesF8>;
  k1<<<persistent_grid(k1, lds_tiles, 4), 256, lds_tiles, s>>>(cover(d1, 16, DBN1 / 2, 1, kAll));
  for (int p = 0; p < n_probs; ++p)
    launch_fake_quant_rows_fp8(probs[p].rows, probs[p].Iw, probs[p].h, s);
  k2<<<persistent_grid(k2, lds_tiles, 4), 256, lds_tiles, s>>>(cover(d2, 16, DBN2, 1, kAll));
  MOE_DBG("grouped gemms (W8A8 on the FP8-weight decode tiles)");
  return true;
}

// The GEMM pair for operand format WF (0: bf16; 1: E4M3 weights with block
// scales, bf16 activations; 2: E4M3 weights and activations).
template <int WF>
void launch_mfma_pair(const moe_config& c, const FfnProblem* probs, int n_probs,
                      const GemmArgs& g1, const GemmArgs& g2, hipStream_t s) {
  const int H = c.H, nst = g1.n_seg_total;
  constexpr int BK1 = decode_bk1<WF>(), BK2 = decode_bk2<WF>();
  int max_rows = 0;
  bool k_ok = H % BK1 == 0;
  for (int p = 0; p < n_probs; ++p) {
    max_rows += probs[p].rows;
    k_ok = k_ok && probs[p].Iw % BK2 == 0;
  }
  const size_t lds_tiles = (size_t)(nst + 1) * sizeof(int);
  // Few rows per segment on average: weight streaming with 16-row tiles.
  if (k_ok && uses_decode_tiles(max_rows, nst)) {
    if constexpr (WF == 2) {
      if (w8a8_on_fp8w_decode(c, probs, n_probs, g1, g2, lds_tiles, s)) return;
    }
    constexpr int DW = WF == 0 ? kDecodeWaves : WF == 1 ? kDecodeWavesF8 : kDecodeWavesW8A8;
    auto k1 = gemm_decode_kernel<0, WF, DBN1, BK1, 1, DW>;
    auto k2 = gemm_decode_kernel<1, WF, DBN2, BK2, 1, DW>;
    k1<<<persistent_grid(k1, lds_tiles, 4), 256, lds_tiles, s>>>(cover(g1, 16, DBN1 / 2, 1, kAll));
    quantize_h<WF>(probs, n_probs, s);
    k2<<<persistent_grid(k2, lds_tiles, 4), 256, lds_tiles, s>>>(cover(g2, 16, DBN2, 1, kAll));
    MOE_DBG("grouped gemms");
    return;
  }
  // Segments of kBigRows rows or more take 256 x 256 tiles (half the weight
  // re-reads of their many row tiles), the rest 128 x 256 tiles: one launch
  // per shape, each covering its own segments.  The mid ring is cut to 2
  // stages if the 3-stage one leaves no room for the tile table (and the
  // scales), and the mid tiles take the long segments too if the big ring
  // does not fit beside them.  The big launches are skipped when no segment
  // can reach kBigRows rows (each problem states the longest a segment of it
  // can be).  With E4M3 weights the segments shorter than kSmallRows take
  // a launch of 64-row tiles of their own.
  using MT = typename Tiles<WF>::Mid;
  using BG = typename Tiles<WF>::Big;
  using SM = typename Tiles<WF>::Small;
  constexpr int kSmall = Tiles<WF>::kSmallRows;
  constexpr size_t kMargin = 64;
  const bool big_fits = ring_dyn_lds(g1, WF, BG::kBM) + BG::kRingBytes + kMargin <= kMaxLdsBytes &&
                        ring_dyn_lds(g2, WF, BG::kBM) + BG::kRingBytes + kMargin <= kMaxLdsBytes;
  const int mid_hi = big_fits ? kBigRows : kAll;
  const int mid_lo = kSmall > 0 ? kSmall : 1;
  const GemmArgs m1 = cover(g1, MT::kBM, MT::kBN / 2, mid_lo, mid_hi);
  const GemmArgs m2 = cover(g2, MT::kBM, MT::kBN, mid_lo, mid_hi);
  const GemmArgs s1 = cover(g1, SM::kBM, SM::kBN / 2, 1, mid_lo);
  const GemmArgs s2 = cover(g2, SM::kBM, SM::kBN, 1, mid_lo);
  const GemmArgs b1 = cover(g1, BG::kBM, BG::kBN / 2, kBigRows, kAll);
  const GemmArgs b2 = cover(g2, BG::kBM, BG::kBN, kBigRows, kAll);
  const bool deep1 = ring_dyn_lds(g1, WF, MT::kBM) + MT::kRingBytes + kMargin <= kMaxLdsBytes;
  const bool deep2 = ring_dyn_lds(g2, WF, MT::kBM) + MT::kRingBytes + kMargin <= kMaxLdsBytes;
  const bool sdeep1 = ring_dyn_lds(g1, WF, SM::kBM) + SM::kRingBytes + kMargin <= kMaxLdsBytes;
  const bool sdeep2 = ring_dyn_lds(g2, WF, SM::kBM) + SM::kRingBytes + kMargin <= kMaxLdsBytes;
  int longest = 0;
  for (int p = 0; p < n_probs; ++p)
    longest = probs[p].max_seg_rows > longest ? probs[p].max_seg_rows : longest;
  const bool any_big = big_fits && longest >= kBigRows;
  // (a 2-stage ring of the mid and small shapes always fits beside the
  // largest table)
  if constexpr (kSmall > 0) {
    if (sdeep1) launch_ring<0, WF, SM::kBM, SM::kBN, SM::kBK, SM::kThreads, SM::kWM, SM::kStages>(s1, s);
    else launch_ring<0, WF, SM::kBM, SM::kBN, SM::kBK, SM::kThreads, SM::kWM, 2>(s1, s);
  }
  if (deep1) launch_ring<0, WF, MT::kBM, MT::kBN, MT::kBK, MT::kThreads, MT::kWM, MT::kStages>(m1, s);
  else launch_ring<0, WF, MT::kBM, MT::kBN, MT::kBK, MT::kThreads, MT::kWM, 2>(m1, s);
  if (any_big) launch_ring<0, WF, BG::kBM, BG::kBN, BG::kBK, BG::kThreads, BG::kWM, BG::kStages>(b1, s);
  // (FP8 activations: the ring tiles of GEMM 1 wrote h quantized)
  if constexpr (kSmall > 0) {
    if (sdeep2) launch_ring<1, WF, SM::kBM, SM::kBN, SM::kBK, SM::kThreads, SM::kWM, SM::kStages>(s2, s);
    else launch_ring<1, WF, SM::kBM, SM::kBN, SM::kBK, SM::kThreads, SM::kWM, 2>(s2, s);
  }
  if (deep2) launch_ring<1, WF, MT::kBM, MT::kBN, MT::kBK, MT::kThreads, MT::kWM, MT::kStages>(m2, s);
  else launch_ring<1, WF, MT::kBM, MT::kBN, MT::kBK, MT::kThreads, MT::kWM, 2>(m2, s);
  if (any_big) launch_ring<1, WF, BG::kBM, BG::kBN, BG::kBK, BG::kThreads, BG::kWM, BG::kStages>(b2, s);
  MOE_DBG("grouped gemms");
}

}  // namespace

void launch_grouped_ffn(const moe_config& c, const FfnProblem* probs, int n_probs,
                        hipStream_t s) {
  const int H = c.H;
  if (c.act_dtype == MOE_DT_F32) {
    for (int p = 0; p < n_probs; ++p) {
      const FfnProblem& P = probs[p];
      const int Iw = P.Iw;
      int64_t n1 = (int64_t)P.rows * Iw, n2 = (int64_t)P.rows * H;
      gemm_f32_kernel<0><<<(unsigned)((n1 + 3) / 4), 256, 0, s>>>(
          (const float*)P.A, (const float*)P.w13, (float*)P.h, nullptr, P.seg_offsets,
          P.seg_expert, P.a_rows, P.n_seg, P.rows, Iw, H, Iw, (int64_t)2 * Iw * H, P.n_w);
      gemm_f32_kernel<1><<<(unsigned)((n2 + 3) / 4), 256, 0, s>>>(
          (const float*)P.h, (const float*)P.w2, (float*)P.y, P.row_scale, P.seg_offsets,
          P.seg_expert, nullptr, P.n_seg, P.rows, H, Iw, 0, (int64_t)H * Iw, P.n_w);
    }
    return;
  }
  GemmArgs g1{}, g2{};
  int nst = 0;
  for (int p = 0; p < n_probs; ++p) {
    const FfnProblem& P = probs[p];
    GemmProblem& a = g1.p[p];
    a.A = (const uint16_t*)P.A;
    a.B = (const uint16_t*)P.w13;
    a.C = (uint16_t*)P.h;
    a.scale = nullptr;
    a.seg_offsets = P.seg_offsets;
    a.seg_expert = P.seg_expert;
    a.a_rows = P.a_rows;
    a.n_seg = P.n_seg;
    a.rows = P.rows;
    a.n_w = P.n_w;
    a.a_ld_rows = P.a_rows ? c.T : P.rows;   // gathered rows come from x
    a.N = P.Iw;
    a.K = H;
    a.up_off = P.Iw;
    a.b_stride = (int64_t)2 * P.Iw * H;
    a.b_scale = P.w13_scale;
    a.s_stride = (int64_t)(2 * P.Iw / 128) * (H / 128);
    a.a_scale = P.a_scale;
    a.Cq = P.h_q;
    a.c_scale = P.h_scale;
    GemmProblem& b = g2.p[p];
    b = a;
    b.A = (const uint16_t*)(P.a_fp8 ? (const void*)P.h_q : P.h);
    b.a_scale = P.h_scale;
    b.Cq = nullptr;
    b.c_scale = nullptr;
    b.a_rows = nullptr;
    b.a_ld_rows = P.rows;
    b.B = (const uint16_t*)P.w2;
    b.C = (uint16_t*)P.y;
    b.scale = P.row_scale;
    b.N = H;
    b.K = P.Iw;
    b.up_off = 0;
    b.b_stride = (int64_t)H * P.Iw;
    b.b_scale = P.w2_scale;
    b.s_stride = (int64_t)(H / 128) * (P.Iw / 128);
    nst += P.n_seg;
  }
  g1.n_probs = g2.n_probs = n_probs;
  g1.n_seg_total = g2.n_seg_total = nst;
  if (probs[0].a_fp8) launch_mfma_pair<2>(c, probs, n_probs, g1, g2, s);
  else if (probs[0].w_fp8) launch_mfma_pair<1>(c, probs, n_probs, g1, g2, s);
  else launch_mfma_pair<0>(c, probs, n_probs, g1, g2, s);
}

}  // namespace moe
