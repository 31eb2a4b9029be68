// C ABI of libmoe: argument checks, workspace layout and launch order.
// Every check runs on the host before any HIP call, so a bad call returns a
// status without touching the GPU (and can be tested on a machine without
// one).
#include <string.h>

#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace moe {

int32_t num_segments(const moe_config& c) {
  if (c.capacity_factor_permille > 0) return 2 * c.E;
  if (c.n_hot_split > 0 && c.split_ways > 1)
    return c.E + (c.n_hot_split < c.E ? c.n_hot_split : c.E) * (c.split_ways - 1);
  return c.E;
}

Layout make_layout(const moe_config& c) {
  Layout L{};
  const size_t A = (size_t)c.T * c.k;
  const size_t R = (size_t)num_rows(c);
  const size_t eb = c.act_dtype == MOE_DT_F32 ? 4 : 2;
  const size_t nbins = (size_t)c.E * bin_ways(c);
  const size_t nb = (size_t)chunk_stride((int64_t)A);
  const size_t S = (size_t)num_segments(c);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.cnt_bin = take(nbins * nb * 4);
  L.blk_off = take(S * nb * 4);
  L.seg_of_bin = take(nbins * 4);
  L.p_end = o;
  L.h = take(R * c.I * eb);
  L.shared_h = take((size_t)c.T * c.shared_I * eb);
  const size_t ib = ((size_t)c.I + 127) / 128, sb = ((size_t)c.shared_I + 127) / 128;
  L.h_q = take(R * c.I);
  L.h_s = take(R * ib * 4);
  L.shared_hq = take((size_t)c.T * c.shared_I);
  L.shared_hs = take((size_t)c.T * sb * 4);
  {
    // bf16 copy of FP8 activations for the decode tiles: x (T rows) in the
    // layer, x_perm (R rows) in the grouped FFN, when the launch takes them
    const int64_t rows = (int64_t)R + (c.shared_I > 0 ? c.T : 0);
    const int64_t segs = (int64_t)S + (c.shared_I > 0 ? 1 : 0);
    const bool dec = c.act_dtype == MOE_DT_BF16 && uses_decode_tiles(rows, segs);
    L.a_deq = take(dec ? std::max((size_t)c.T, R) * c.H * 2 : 0);
  }
  L.g_end = o;
  L.y_perm = take(R * c.H * eb);
  L.shared_y = take(c.shared_I > 0 ? (size_t)c.T * c.H * eb : 0);
  L.seg_offsets = take((S + 1) * 4);
  L.seg_expert = take(S * 4);
  L.assign_to_row = take(A * 4);
  L.row_to_token = take(R * 4);
  L.row_w = take(R * 4);
  L.x_q = take((size_t)c.T * c.H);
  L.x_s = take((size_t)c.T * (((size_t)c.H + 127) / 128) * 4);
  L.l_end = o;
  return L;
}

int device_cu_count() {
  static std::atomic<int> cache[64];   // per device; any thread may fill it (same value)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

moe_status check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->H <= 0 || c->E <= 0 || c->k <= 0 || c->I <= 0) return MOE_ERR_INVALID_ARG;
  if (c->E > kMaxE || c->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (c->k > c->E) return MOE_ERR_INVALID_ARG;
  if (c->act_dtype != MOE_DT_F32 && c->act_dtype != MOE_DT_BF16) return MOE_ERR_INVALID_ARG;
  if (c->score != MOE_SCORE_SOFTMAX && c->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (c->n_group <= 0 || c->E % c->n_group != 0) return MOE_ERR_INVALID_ARG;
  if (c->n_group > 64) return MOE_ERR_UNSUPPORTED;
  if (c->n_group > 1) {
    if (c->score != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
    const int per = c->E / c->n_group;
    if (c->topk_group <= 0 || c->topk_group > c->n_group) return MOE_ERR_INVALID_ARG;
    if ((int64_t)c->topk_group * per < c->k) return MOE_ERR_INVALID_ARG;
    if (c->group_score_topn <= 0 || c->group_score_topn > per) return MOE_ERR_INVALID_ARG;
  }
  if (c->n_hot_split < 0 || c->split_ways < 1) return MOE_ERR_INVALID_ARG;
  if (c->split_ways > kMaxWays) return MOE_ERR_UNSUPPORTED;
  if (c->split_mode != MOE_SPLIT_PARITY && c->split_mode != MOE_SPLIT_BOUNDED)
    return MOE_ERR_INVALID_ARG;
  if (c->split_c_permille < 0 || c->split_c_permille > 100000) return MOE_ERR_INVALID_ARG;
  if (c->capacity_factor_permille < 0 || c->capacity_factor_permille > 1000000)
    return MOE_ERR_INVALID_ARG;
  if (c->capacity_factor_permille > 0 && c->n_hot_split > 0 && c->split_ways > 1)
    return MOE_ERR_UNSUPPORTED;
  if (c->shared_I < 0) return MOE_ERR_INVALID_ARG;
  if ((int64_t)c->T * c->k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  // the kernels address each activation and weight matrix with 32-bit byte
  // offsets: keep every one below 2^31 elements
  const int64_t lim = (int64_t)1 << 31, A = (int64_t)c->T * c->k, R = num_rows(*c);
  if (R > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  if (A * c->H >= lim || A * c->I >= lim || (int64_t)c->T * c->shared_I >= lim ||
      R * c->H >= lim || R * c->I >= lim ||
      (int64_t)2 * c->I * c->H >= lim || (int64_t)2 * c->shared_I * c->H >= lim)
    return MOE_ERR_UNSUPPORTED;
  if (c->act_dtype == MOE_DT_BF16) {
    // rows of 16-byte chunks (the GEMM copies, gather and combine move 8 bf16)
    if (c->H % 8 || c->I % 8 || c->shared_I % 8) return MOE_ERR_UNSUPPORTED;
  } else {
    if (c->H % 4) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace {

// Expert weights of one call: bf16 (scales NULL), or E4M3 codes with 128 x 128
// block scales.
struct Weights {
  const void* w13;
  const void* w2;
  const float* w13_scale;
  const float* w2_scale;
  bool fp8;
  bool acts_fp8 = false;   // with fp8: E4M3 activations too (W8A8)
};

// Extra requirements of FP8 weights: bf16 activations, 128-multiples, scales.
moe_status check_fp8(const moe_config* cfg, const Weights& w) {
  if (!w.fp8) return MOE_OK;
  if (cfg->act_dtype != MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
  if (cfg->H % 128 || cfg->I % 128 || cfg->shared_I % 128) return MOE_ERR_UNSUPPORTED;
  if (!w.w13_scale || !w.w2_scale) return MOE_ERR_INVALID_ARG;
  if (!aligned(w.w13_scale, 4) || !aligned(w.w2_scale, 4)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status grouped_ffn(const moe_config* cfg, const void* x_perm, const float* x_perm_scale,
                       const int32_t* seg_offsets, const int32_t* seg_expert, const Weights& w,
                       const float* row_scale, void* y_perm, void* workspace,
                       size_t workspace_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!w.w13 || !w.w2) return MOE_ERR_INVALID_ARG;
  if ((st = check_fp8(cfg, w)) != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!x_perm || !seg_offsets || !seg_expert || !y_perm || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (w.acts_fp8 && (!x_perm_scale || !aligned(x_perm_scale, 4))) return MOE_ERR_INVALID_ARG;
  if (!aligned(x_perm, 16) || !aligned(w.w13, 16) || !aligned(w.w2, 16) ||
      !aligned(y_perm, 16) || !aligned(workspace, kAlign) || !aligned(seg_offsets, 4) ||
      !aligned(seg_expert, 4) || (row_scale && !aligned(row_scale, 4)))
    return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(*cfg);
  if (workspace_bytes < L.g_end) return MOE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  FfnProblem p{};
  p.A = x_perm;
  p.w13 = w.w13;
  p.w2 = w.w2;
  p.w_fp8 = w.fp8;
  p.w13_scale = w.w13_scale;
  p.w2_scale = w.w2_scale;
  p.h = ws + L.h;
  p.y = y_perm;
  p.row_scale = row_scale;
  p.seg_offsets = seg_offsets;
  p.seg_expert = seg_expert;
  p.n_seg = num_segments(*cfg);
  p.rows = (int32_t)num_rows(*cfg);
  p.max_seg_rows = p.rows;   // any segment lengths (ids may repeat within a token)
  p.n_w = cfg->E;
  p.Iw = cfg->I;
  p.a_fp8 = w.acts_fp8;
  p.a_scale = x_perm_scale;
  p.h_q = (uint8_t*)(ws + L.h_q);
  p.h_scale = (float*)(ws + L.h_s);
  p.a_deq = ws + L.a_deq;
  p.a_deq_bytes = L.g_end - L.a_deq;
  launch_grouped_ffn(*cfg, &p, 1, (hipStream_t)stream);
  return launch_status();
}

moe_status layer_forward(const moe_config* cfg, const float* logits, const void* x,
                         const Weights& w, const Weights& sw, void* out, int32_t* topk_ids,
                         float* topk_w, int32_t* counts, float* balancedness, void* workspace,
                         size_t workspace_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const bool shared = cfg->shared_I > 0;
  if (!w.w13 || !w.w2 || (shared && (!sw.w13 || !sw.w2))) return MOE_ERR_INVALID_ARG;
  if ((st = check_fp8(cfg, w)) != MOE_OK) return st;
  if (shared && (st = check_fp8(cfg, sw)) != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!logits || !x || !out || !topk_ids || !topk_w || !counts || !balancedness || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w.w13, 16) || !aligned(w.w2, 16) || !aligned(out, 16) ||
      (shared && (!aligned(sw.w13, 16) || !aligned(sw.w2, 16))) ||
      !aligned(workspace, kAlign) || !aligned(logits, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4) || !aligned(counts, 4) || !aligned(balancedness, 4))
    return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(*cfg);
  if (workspace_bytes < L.l_end) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int32_t* seg_offsets = (int32_t*)(ws + L.seg_offsets);
  int32_t* seg_expert = (int32_t*)(ws + L.seg_expert);
  int32_t* a2r = (int32_t*)(ws + L.assign_to_row);
  int32_t* r2t = (int32_t*)(ws + L.row_to_token);
  float* row_w = (float*)(ws + L.row_w);

  MOE_DBG("layer entry");
  // FP8 activations: x is quantized before dispatch (1 x 128 pieces)
  const void* xa = x;
  const float* xs = nullptr;
  if (w.acts_fp8) {
    launch_quantize_rows_fp8(cfg->T, cfg->H, x, (uint8_t*)(ws + L.x_q), (float*)(ws + L.x_s), s);
    xa = ws + L.x_q;
    xs = (const float*)(ws + L.x_s);
  }
  // no x_perm: GEMM 1 gathers its rows from x through row_to_token
  if (cfg->T * cfg->k <= kSmallA) {
    launch_route_permute_small(*cfg, logits, topk_ids, topk_w, counts, seg_offsets, seg_expert,
                               a2r, r2t, row_w, balancedness, s);
  } else {
    launch_route(*cfg, logits, topk_ids, topk_w, s);
    launch_permute(*cfg, x, topk_ids, nullptr, seg_offsets, seg_expert, a2r, r2t, counts,
                   balancedness, topk_w, row_w, ws, L, s);
  }
  MOE_DBG("route + permute");
  FfnProblem p[2]{};
  p[0].A = xa;
  p[0].a_fp8 = w.acts_fp8;
  p[0].a_scale = xs;
  p[0].h_q = (uint8_t*)(ws + L.h_q);
  p[0].h_scale = (float*)(ws + L.h_s);
  p[0].a_deq = ws + L.a_deq;
  p[0].a_deq_bytes = L.g_end - L.a_deq;
  p[0].a_rows = r2t;
  p[0].w13 = w.w13;
  p[0].w2 = w.w2;
  p[0].w_fp8 = w.fp8;
  p[0].w13_scale = w.w13_scale;
  p[0].w2_scale = w.w2_scale;
  p[0].h = ws + L.h;
  p[0].y = ws + L.y_perm;
  p[0].row_scale = row_w;
  p[0].seg_offsets = seg_offsets;
  p[0].seg_expert = seg_expert;
  p[0].n_seg = num_segments(*cfg);
  p[0].rows = (int32_t)num_rows(*cfg);
  // routing gives every token k distinct experts: a segment holds at most one
  // row per token
  p[0].max_seg_rows = p[0].rows < cfg->T ? p[0].rows : cfg->T;
  p[0].n_w = cfg->E;
  p[0].Iw = cfg->I;
  if (shared) {
    p[1].A = xa;
    p[1].a_fp8 = w.acts_fp8;
    p[1].a_scale = xs;
    p[1].h_q = (uint8_t*)(ws + L.shared_hq);
    p[1].h_scale = (float*)(ws + L.shared_hs);
    p[1].a_deq = ws + L.a_deq;
    p[1].a_deq_bytes = L.g_end - L.a_deq;
    p[1].w13 = sw.w13;
    p[1].w2 = sw.w2;
    p[1].w_fp8 = sw.fp8;
    p[1].w13_scale = sw.w13_scale;
    p[1].w2_scale = sw.w2_scale;
    p[1].h = ws + L.shared_h;
    p[1].y = ws + L.shared_y;
    p[1].row_scale = nullptr;
    p[1].seg_offsets = nullptr;
    p[1].seg_expert = nullptr;
    p[1].n_seg = 1;
    p[1].rows = cfg->T;
    p[1].max_seg_rows = cfg->T;
    p[1].n_w = 1;
    p[1].Iw = cfg->shared_I;
  }
  launch_grouped_ffn(*cfg, p, shared ? 2 : 1, s);
  launch_combine(*cfg, ws + L.y_perm, a2r, nullptr, shared ? ws + L.shared_y : nullptr, out,
                 s);
  return launch_status();
}

// ---- the entry point that allocates nothing ----
// Its workspace is this file-scope device array.  Each GPU the library runs
// on holds its own copy at its own address from the time the code object is
// loaded there until the process ends.  In host code the name `scratch` is
// only a host-side stand-in: its device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept in static_scratch_base.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_WORKSPACE_BYTES];

// Device address of `scratch` on the current device, nullptr if it cannot be
// had (status in *err).
void* static_scratch_base(moe_status* err) {
  static std::mutex mu;
  static void* base[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    *err = MOE_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      *err = MOE_ERR_HIP;
      return nullptr;
    }
    base[dev] = p;
  }
  return base[dev];
}

}  // namespace

extern "C" {

moe_status moe_layer_forward_static(const moe_config* cfg, const float* logits, const void* x,
                                    const void* w13, const void* w2, const void* shared_w13,
                                    const void* shared_w2, void* out, int32_t* topk_ids,
                                    float* topk_w, int32_t* counts, float* balancedness,
                                    void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  // sizes beyond the static array: refused before anything touches the GPU
  if (make_layout(*cfg).l_end > (size_t)MOE_STATIC_WORKSPACE_BYTES) return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  void* ws = static_scratch_base(&st);
  if (!ws) return st;
  return layer_forward(cfg, logits, x, Weights{w13, w2, nullptr, nullptr, false},
                       Weights{shared_w13, shared_w2, nullptr, nullptr, false}, out, topk_ids,
                       topk_w, counts, balancedness, ws, (size_t)MOE_STATIC_WORKSPACE_BYTES,
                       stream);
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t moe_num_segments(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return -1;
  return num_segments(*cfg);
}

int32_t moe_num_rows(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return -1;
  return (int32_t)num_rows(*cfg);
}

size_t moe_workspace_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return make_layout(*cfg).l_end;
}

moe_status moe_layer_plan_offsets(const moe_config* cfg, size_t offsets[4]) {
  const moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(*cfg);
  offsets[0] = L.seg_offsets;
  offsets[1] = L.seg_expert;
  offsets[2] = L.assign_to_row;
  offsets[3] = L.row_to_token;
  return MOE_OK;
}

moe_status moe_route_topk(const moe_config* cfg, const float* logits, int32_t* topk_ids,
                          float* topk_w, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return MOE_ERR_INVALID_ARG;
  launch_route(*cfg, logits, topk_ids, topk_w, (hipStream_t)stream);
  return launch_status();
}

moe_status moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_ids,
                       void* x_perm, int32_t* seg_offsets, int32_t* seg_expert,
                       int32_t* assign_to_row, int32_t* row_to_token, int32_t* counts,
                       float* balancedness, void* workspace, size_t workspace_bytes,
                       void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !topk_ids || !x_perm || !seg_offsets || !seg_expert || !assign_to_row ||
      !row_to_token || !counts || !balancedness || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(x_perm, 16) || !aligned(workspace, kAlign) ||
      !aligned(topk_ids, 4) || !aligned(seg_offsets, 4) || !aligned(seg_expert, 4) ||
      !aligned(assign_to_row, 4) || !aligned(row_to_token, 4) || !aligned(counts, 4) ||
      !aligned(balancedness, 4))
    return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(*cfg);
  if (workspace_bytes < L.p_end) return MOE_ERR_WORKSPACE;
  launch_permute(*cfg, x, topk_ids, x_perm, seg_offsets, seg_expert, assign_to_row,
                 row_to_token, counts, balancedness, nullptr, nullptr, (char*)workspace, L,
                 (hipStream_t)stream);
  return launch_status();
}


moe_status moe_grouped_ffn(const moe_config* cfg, const void* x_perm,
                           const int32_t* seg_offsets, const int32_t* seg_expert,
                           const void* w13, const void* w2, const float* row_scale,
                           void* y_perm, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return grouped_ffn(cfg, x_perm, nullptr, seg_offsets, seg_expert,
                     Weights{w13, w2, nullptr, nullptr, false}, row_scale, y_perm, workspace,
                     workspace_bytes, stream);
}

moe_status moe_grouped_ffn_fp8w(const moe_config* cfg, const void* x_perm,
                                const int32_t* seg_offsets, const int32_t* seg_expert,
                                const uint8_t* w13_q, const float* w13_scale,
                                const uint8_t* w2_q, const float* w2_scale,
                                const float* row_scale, void* y_perm, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return grouped_ffn(cfg, x_perm, nullptr, seg_offsets, seg_expert,
                     Weights{w13_q, w2_q, w13_scale, w2_scale, true}, row_scale, y_perm,
                     workspace, workspace_bytes, stream);
}

moe_status moe_grouped_ffn_w8a8(const moe_config* cfg, const uint8_t* x_perm_q,
                                const float* x_perm_scale, const int32_t* seg_offsets,
                                const int32_t* seg_expert, const uint8_t* w13_q,
                                const float* w13_scale, const uint8_t* w2_q,
                                const float* w2_scale, const float* row_scale, void* y_perm,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return grouped_ffn(cfg, x_perm_q, x_perm_scale, seg_offsets, seg_expert,
                     Weights{w13_q, w2_q, w13_scale, w2_scale, true, true}, row_scale, y_perm,
                     workspace, workspace_bytes, stream);
}

moe_status moe_unpermute_combine(const moe_config* cfg, const void* y_perm,
                                 const int32_t* assign_to_row, const float* topk_w,
                                 const void* shared_y, void* out, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T == 0) return MOE_OK;
  if (!y_perm || !assign_to_row || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(y_perm, 16) || !aligned(out, 16) || (shared_y && !aligned(shared_y, 16)) ||
      !aligned(assign_to_row, 4) || (topk_w && !aligned(topk_w, 4)))
    return MOE_ERR_INVALID_ARG;
  launch_combine(*cfg, y_perm, assign_to_row, topk_w, shared_y, out, (hipStream_t)stream);
  return launch_status();
}

moe_status moe_layer_forward(const moe_config* cfg, const float* logits, const void* x,
                             const void* w13, const void* w2, const void* shared_w13,
                             const void* shared_w2, void* out, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, float* balancedness,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return layer_forward(cfg, logits, x, Weights{w13, w2, nullptr, nullptr, false},
                       Weights{shared_w13, shared_w2, nullptr, nullptr, false}, out, topk_ids,
                       topk_w, counts, balancedness, workspace, workspace_bytes, stream);
}

moe_status moe_layer_forward_fp8w(const moe_config* cfg, const float* logits, const void* x,
                                  const uint8_t* w13_q, const float* w13_scale,
                                  const uint8_t* w2_q, const float* w2_scale,
                                  const uint8_t* shared_w13_q, const float* shared_w13_scale,
                                  const uint8_t* shared_w2_q, const float* shared_w2_scale,
                                  void* out, int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  float* balancedness, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return layer_forward(cfg, logits, x, Weights{w13_q, w2_q, w13_scale, w2_scale, true},
                       Weights{shared_w13_q, shared_w2_q, shared_w13_scale, shared_w2_scale, true},
                       out, topk_ids, topk_w, counts, balancedness, workspace, workspace_bytes,
                       stream);
}

moe_status moe_layer_forward_w8a8(const moe_config* cfg, const float* logits, const void* x,
                                  const uint8_t* w13_q, const float* w13_scale,
                                  const uint8_t* w2_q, const float* w2_scale,
                                  const uint8_t* shared_w13_q, const float* shared_w13_scale,
                                  const uint8_t* shared_w2_q, const float* shared_w2_scale,
                                  void* out, int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  float* balancedness, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return layer_forward(
      cfg, logits, x, Weights{w13_q, w2_q, w13_scale, w2_scale, true, true},
      Weights{shared_w13_q, shared_w2_q, shared_w13_scale, shared_w2_scale, true, true}, out,
      topk_ids, topk_w, counts, balancedness, workspace, workspace_bytes, stream);
}

moe_status moe_quantize_act_fp8(int32_t rows, int32_t cols, const void* src, uint8_t* q,
                                float* scale, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 128) return MOE_ERR_INVALID_ARG;
  if ((int64_t)rows * cols >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!src || !q || !scale || !aligned(src, 16) || !aligned(q, 16) || !aligned(scale, 4))
    return MOE_ERR_INVALID_ARG;
  launch_quantize_rows_fp8(rows, cols, src, q, scale, (hipStream_t)stream);
  return launch_status();
}

moe_status moe_quantize_fp8(int32_t n_mat, int32_t rows, int32_t cols, const void* src,
                            uint8_t* q, float* scale, void* stream) {
  if (n_mat < 0 || rows <= 0 || cols <= 0 || rows % 128 || cols % 128)
    return MOE_ERR_INVALID_ARG;
  if ((int64_t)rows * cols >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (n_mat == 0) return MOE_OK;
  if (!src || !q || !scale || !aligned(src, 16) || !aligned(q, 16) || !aligned(scale, 4))
    return MOE_ERR_INVALID_ARG;
  launch_quantize_fp8(n_mat, rows, cols, src, q, scale, (hipStream_t)stream);
  return launch_status();
}

}  // extern "C"
