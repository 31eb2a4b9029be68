/*
 * moe.h -- C ABI of libmoe: the forward pass of one Mixture-of-Experts layer on
 * one AMD Instinct MI355X (gfx950), as hand-written HIP kernels.
 *
 * The layer follows the four runtime steps of "Serving Mixture-of-Experts
 * Models" (section "Follow one token through an MoE layer"), minus the network
 * send: (1) the router's top-k expert ids and weights per token; (2) a
 * histogram / prefix-sum permutation that packs token rows into contiguous
 * per-expert segments; (3) every expert's segment through its SwiGLU MLP as a
 * grouped matrix multiplication; (4) the inverse permutation with a
 * router-weighted sum.  It also reports balancedness = mean / max tokens per
 * expert (same chapter, section "The slowest expert sets the pace").
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host".  The caller allocates
 *    and frees every buffer, including the workspace; the library never
 *    allocates, frees or synchronises, and keeps no state between calls other
 *    than a per-device cache of the compute-unit count.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  Calls on different streams may run concurrently if they use
 *    different workspaces and outputs.
 *  - Argument checks run on the host before anything is launched and return a
 *    negative status synchronously; nothing is written then.  A failed launch
 *    returns MOE_ERR_HIP.  Faults inside kernels surface at the caller's next
 *    synchronisation, as for any asynchronous GPU API.
 *  - Device index arrays are int32, row-major.  Assignment a = t*k + j is slot
 *    j of token t.  Activations x, weights and outputs share one element type
 *    (cfg->act_dtype): fp32 or bf16; arithmetic accumulates in fp32.
 *  - T == 0 is an empty batch: every call returns MOE_OK and touches nothing.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment */
  MOE_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels handle */
  MOE_ERR_WORKSPACE = -3,   /* workspace_bytes too small */
  MOE_ERR_HIP = -4          /* a HIP launch failed */
} moe_status;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_SCORE_SOFTMAX = 0, /* flat top-k, softmax weights */
  MOE_SCORE_SIGMOID = 1  /* group-limited top-k on sigmoid scores */
} moe_score;

/* Replica split of the hot experts.
 *  MOE_SPLIT_PARITY:  replica p holds the assignments of tokens t with
 *                     t mod split_ways == p.
 *  MOE_SPLIT_BOUNDED: the relaxed balance constraint of the Zepp paper
 *                     (section 4.1, Eq. 1) on one GPU, with the integer
 *                     rounding and greedy water-filling of its section 5
 *                     ("Routing"): for an expert with d assignments,
 *                     q = d / split_ways and C = split_c_permille / 1000,
 *                     every replica load lies in
 *                     [floor(q (1 - C)), ceil(q (1 + C))]; replicas are
 *                     filled in order, each as far as the upper bound allows
 *                     while the later replicas can still reach their lower
 *                     bound, and replica p takes the next consecutive run of
 *                     the expert's assignments in increasing a.  With C = 0
 *                     the loads differ by at most one, larger ones first.
 *                     All replicas share the one GPU, so the pages' cost
 *                     term is the same for every feasible split. */
typedef enum { MOE_SPLIT_PARITY = 0, MOE_SPLIT_BOUNDED = 1 } moe_split_mode;

/* Layer description, a host struct read by every call (never retained). */
typedef struct moe_config {
  int32_t T;  /* tokens in the batch (>= 0) */
  int32_t H;  /* hidden size */
  int32_t E;  /* routed (logical) experts, 1..1024 */
  int32_t k;  /* experts per token, 1..min(E, 32) */
  int32_t I;  /* expert intermediate size */
  int32_t score;            /* moe_score */
  int32_t n_group;          /* expert groups (contiguous, E % n_group == 0); 1 = flat */
  int32_t topk_group;       /* groups kept per token (sigmoid mode) */
  int32_t group_score_topn; /* a group's score = sum of its best n member scores */
  int32_t renormalize;      /* 1: the k weights are renormalised to sum to 1 */
  int32_t n_hot_split;      /* hottest experts given replica segments (0 = none) */
  int32_t split_ways;       /* replicas per hot expert (1..4) */
  int32_t shared_I;         /* 0, or the shared expert's intermediate size */
  int32_t act_dtype;        /* moe_dtype of x, weights, x_perm, y_perm, out */
  int32_t split_mode;       /* moe_split_mode: how a hot expert's assignments
                             * are spread over its replicas */
  int32_t split_c_permille; /* MOE_SPLIT_BOUNDED: relaxation ratio C of the
                             * load bounds in 1/1000 (0..100000); ignored
                             * otherwise */
  int32_t capacity_factor_permille; /* 0: dropless, packed segments.  > 0
                             * (up to 1000000): the fixed-capacity layout
                             * below, factor f = value / 1000; needs
                             * n_hot_split = 0 */
} moe_config;
/* Fixed-capacity layout (the book's "Capacity, padding, and the drop
 * decision"; the fixed-size masked layout of the MoE inference blog's
 * "Prefill and decode kernel layouts"): every expert gets
 * cap = ceil(f * T*k / E) slots, expert e owning rows [e*cap, (e+1)*cap) of
 * x_perm / y_perm.  Its assignments, in increasing a = t*k + j, fill those
 * rows in order; the ones that find them full are dropped (assign_to_row =
 * -1, no contribution to out: their output for the layer is zero).  There
 * are S = 2E segments: segment 2e holds expert e's kept rows, segment 2e+1
 * the rest of its slots, with seg_expert = -1 (padding: no expert computes
 * it, row_to_token = -1 there).  Routing counts and balancedness are those
 * of the routed ids, before any drop. */
/* Size limits (MOE_ERR_UNSUPPORTED beyond them): T*k <= 2^30; each of
 * T*k*H, T*k*I, T*shared_I, 2*I*H and 2*shared_I*H below 2^31 elements (the
 * kernels address every matrix with 32-bit byte offsets); bf16 needs H, I
 * and shared_I to be multiples of 8, fp32 needs H % 4 == 0. */

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status s);

/* Number of segments S = E + min(n_hot_split, E) * (split_ways - 1)
 * (split_ways > 1 only), or 2E in the fixed-capacity layout; -1 if cfg is
 * NULL or invalid. */
int32_t moe_num_segments(const moe_config* cfg);

/* Rows R of x_perm, y_perm and row_to_token: T*k, or E * cap in the
 * fixed-capacity layout; -1 if cfg is NULL or invalid. */
int32_t moe_num_rows(const moe_config* cfg);

/* Bytes of device workspace that suffices for every call below with this
 * configuration (moe_layer_forward needs all of it; moe_permute and
 * moe_grouped_ffn need a leading part of it and accept any size at least
 * that large).  0 if cfg is invalid. */
size_t moe_workspace_size(const moe_config* cfg);

/* Step 1 -- top-k gating ("Follow one token through an MoE layer": the router
 * picks each token's experts and their weights; the MoE inference blog's
 * "MoE architecture recap": top-k experts, or a few expert groups first and
 * then the top experts inside them).
 *   logits   [T, E] fp32, finite.
 *   topk_ids [T, k] out: expert ids in descending logit order; an exact tie
 *            goes to the lower id.
 *   topk_w   [T, k] out, fp32: softmax mode -- softmax over the k winners
 *            (renormalize = 1) or the full-E softmax of each winner;
 *            sigmoid mode -- groups are scored by the sum of their best
 *            group_score_topn sigmoid scores (fp32), the topk_group best
 *            groups are kept (lower group id on a tie), the k largest logits
 *            of the kept groups win, and weights are s_j / sum(s)
 *            (renormalize = 1) or s_j.  Weights are computed in fp64 and
 *            rounded once to fp32. */
moe_status moe_route_topk(const moe_config* cfg, const float* logits,
                          int32_t* topk_ids, float* topk_w, void* stream);

/* Step 2 -- histogram / prefix-sum permutation into contiguous per-expert
 * segments ("Follow one token through an MoE layer", step 1), or into the
 * fixed-capacity layout when capacity_factor_permille > 0.  R =
 * moe_num_rows(cfg).
 *   x             [T, H]  act_dtype.
 *   topk_ids      [T, k]  ids in [0, E); an id outside is dropped (its
 *                          assign_to_row is -1 and it joins no segment).
 *   x_perm        [R, H]  out: x_perm[r] = x[row_to_token[r]] byte for byte,
 *                          for r < seg_offsets[S] with row_to_token[r] >= 0;
 *                          other rows untouched.
 *   seg_offsets   [S+1]   out: exclusive prefix sum of segment lengths.
 *   seg_expert    [S]     out: logical expert of each segment.  Segments are
 *                          in ascending expert order; a hot expert (one of the
 *                          n_hot_split largest counts, lower id on a tie) has
 *                          split_ways adjacent replica segments, filled as
 *                          split_mode says (replicas keep the logical
 *                          selection and weights, Zepp section 4.1).  Empty
 *                          segments stay listed.
 *   assign_to_row [T*k]   out: row of each assignment (-1 if dropped).
 *   row_to_token  [R]     out: token of each row (rows < seg_offsets[S];
 *                          -1 on padding rows).
 *   counts        [E]     out: assignments per logical expert.
 *   balancedness  [1]     out, fp32: (sum(counts) / E) / max(counts), from
 *                          exact integers by one fp64 division ("The slowest
 *                          expert sets the pace"); 0 if every id was dropped.
 * Rows of a segment are its assignments in increasing a (a stable counting
 * sort), so every output is deterministic.  H * element size must be a
 * multiple of 16 bytes and x / x_perm 16-byte aligned. */
moe_status moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_ids,
                       void* x_perm, int32_t* seg_offsets, int32_t* seg_expert,
                       int32_t* assign_to_row, int32_t* row_to_token, int32_t* counts,
                       float* balancedness, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Step 3 -- every segment through its expert as one grouped matrix
 * multiplication ("Follow one token through an MoE layer", step 3; the MoE
 * inference blog's "Optimized kernels for MoE": one kernel over many experts
 * with different token counts).  Per row r of segment s, e = seg_expert[s]:
 *   h = silu(x_perm[r] . W_gate[e]) * (x_perm[r] . W_up[e])   (fp32, rounded
 *       to act_dtype), y_perm[r] = row_scale[r] * (h . W_down[e]).
 * A segment whose seg_expert lies outside [0, E) is skipped (its rows of
 * y_perm are left untouched): the padding of the fixed-capacity layout.
 *   x_perm      [R, H]  rows as produced by moe_permute (R = moe_num_rows).
 *   seg_offsets [S+1], seg_expert [S] as produced by moe_permute (read on the
 *               device; the host never needs the counts).
 *   w13         [E, 2I, H] act_dtype, K-contiguous: rows 0..I-1 of expert e
 *               are W_gate[e]^T, rows I..2I-1 are W_up[e]^T.
 *   w2          [E, H, I]  act_dtype, W_down[e]^T.
 *   row_scale   [R] fp32 indexed by row, or NULL for 1.0.
 *   y_perm      [R, H] out (rows of computed segments).
 * bf16 needs H and I multiples of 8; all pointers 16-byte aligned. */
moe_status moe_grouped_ffn(const moe_config* cfg, const void* x_perm,
                           const int32_t* seg_offsets, const int32_t* seg_expert,
                           const void* w13, const void* w2, const float* row_scale,
                           void* y_perm, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Step 4 -- inverse permutation and router-weighted sum ("Follow one token
 * through an MoE layer", step 4):
 *   out[t] = sum_{j<k} w[t,j] * y_perm[assign_to_row[t*k+j]] (+ shared_y[t]),
 * accumulated in fp32 in slot order j = 0..k-1 and rounded once.
 *   topk_w    [T, k] fp32, or NULL when y_perm rows are already scaled.
 *   shared_y  [T, H] or NULL (the shared expert, added with weight 1).
 *   out       [T, H] out.  A dropped slot (assign_to_row -1) adds nothing. */
moe_status moe_unpermute_combine(const moe_config* cfg, const void* y_perm,
                                 const int32_t* assign_to_row, const float* topk_w,
                                 const void* shared_y, void* out, void* stream);

/* The whole layer: steps 1-4 plus the shared expert (if cfg->shared_I > 0;
 * "MoE architecture recap": shared experts process every token), with no host
 * synchronisation between steps (segment lengths never leave the device).
 *   logits [T, E] fp32; x [T, H]; w13 [E, 2I, H]; w2 [E, H, I];
 *   shared_w13 [2*shared_I, H] and shared_w2 [H, shared_I] (NULL if none);
 *   out [T, H] out; topk_ids [T, k], topk_w [T, k], counts [E],
 *   balancedness [1] out (as in the step calls).
 *   workspace: at least moe_workspace_size(cfg) bytes, 256-byte aligned. */
moe_status moe_layer_forward(const moe_config* cfg, const float* logits, const void* x,
                             const void* w13, const void* w2, const void* shared_w13,
                             const void* shared_w2, void* out, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, float* balancedness,
                             void* workspace, size_t workspace_bytes, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same layer, the same kernels and the same results bit for
 * bit, but the workspace is a device array inside the library, of
 * MOE_STATIC_WORKSPACE_BYTES, one per GPU, held from the time the library's
 * code is loaded on that GPU until the process ends.  The call allocates
 * nothing: no hipMalloc, hipFree or allocating library routine.  The caller
 * still passes every input and output, as for moe_layer_forward.
 *   Returns MOE_ERR_WORKSPACE, before touching the GPU, when the layer needs
 *   more workspace than that (moe_workspace_size(cfg) >
 *   MOE_STATIC_WORKSPACE_BYTES: about T*k*(H + I)*2 bytes in bf16, so
 *   decode-sized batches fit, e.g. 64 tokens at H = 8192 top-2 take ~6 MB);
 *   MOE_ERR_HIP if the array's device address cannot be had.
 *   Nothing in the array needs to start at zero (every kernel writes what it
 *   later reads), and it keeps the last call's contents.  All calls on one
 *   GPU share it: calls that overlap in time on one GPU (on different
 *   streams or host threads) race and must be serialized by the caller. */
#define MOE_STATIC_WORKSPACE_BYTES (64u * 1024u * 1024u)
moe_status moe_layer_forward_static(const moe_config* cfg, const float* logits, const void* x,
                                    const void* w13, const void* w2, const void* shared_w13,
                                    const void* shared_w2, void* out, int32_t* topk_ids,
                                    float* topk_w, int32_t* counts, float* balancedness,
                                    void* stream);

/* Where moe_layer_forward (and its _fp8w and _w8a8 forms) leave the
 * permutation they built inside their workspace, as byte offsets from its
 * start: offsets[0] seg_offsets [S+1], offsets[1] seg_expert [S],
 * offsets[2] assign_to_row [T*k], offsets[3] row_to_token [R] (int32, the
 * contents and meaning of the moe_permute outputs of the same names).  They
 * hold the last call's values once it has completed, until the workspace is
 * used again.  MOE_ERR_INVALID_ARG for an invalid cfg or a NULL offsets. */
moe_status moe_layer_plan_offsets(const moe_config* cfg, size_t offsets[4]);

/* ------------------------------------------------------------------------
 * FP8 expert weights (the MoE inference blog, "Communication pressure", its
 * optimized MoE kernels: a low-precision GEMM kernel uses FP8 to cut memory
 * and compute cost).  Format of one expert matrix W [R, C] (W13[e]: R = 2I,
 * C = H; W2[e]: R = H, C = I):
 *   q     [R, C] uint8, OCP E4M3 codes (OFP8: bias 7, subnormals m * 2^-9,
 *         no infinity, largest finite 448);
 *   scale [R/128, C/128] fp32, one power of two per 128 x 128 block;
 *   W[r][c] = E4M3(q[r][c]) * scale[r/128][c/128].
 * The layer then computes exactly as with bf16 weights equal to these values
 * (they are exact in bf16); activations, h, y_perm and out stay bf16.  The
 * FP8 calls need act_dtype bf16 and H, I, shared_I multiples of 128.
 * ------------------------------------------------------------------------ */

/* Quantize n_mat bf16 matrices [n_mat, rows, cols] (rows, cols multiples of
 * 128) to the format above: per 128 x 128 block, scale = 2^s with s the
 * smallest integer such that max|block| <= 448 * 2^s (s = 0 for an all-zero
 * block), q = round-to-nearest-even E4M3 of w / 2^s (sign kept, so -0 -> 0x80).
 *   src [n_mat, rows, cols] bf16; q [n_mat, rows, cols] out; scale
 *   [n_mat, rows/128, cols/128] out.  16-byte aligned pointers.
 * MOE_ERR_INVALID_ARG for bad sizes or pointers; asynchronous on `stream`. */
moe_status moe_quantize_fp8(int32_t n_mat, int32_t rows, int32_t cols, const void* src,
                            uint8_t* q, float* scale, void* stream);

/* moe_grouped_ffn with FP8 expert weights: w13_q [E, 2I, H] + w13_scale
 * [E, 2I/128, H/128]; w2_q [E, H, I] + w2_scale [E, H/128, I/128].  Other
 * arguments, outputs and errors as moe_grouped_ffn. */
moe_status moe_grouped_ffn_fp8w(const moe_config* cfg, const void* x_perm,
                                const int32_t* seg_offsets, const int32_t* seg_expert,
                                const uint8_t* w13_q, const float* w13_scale,
                                const uint8_t* w2_q, const float* w2_scale,
                                const float* row_scale, void* y_perm, void* workspace,
                                size_t workspace_bytes, void* stream);

/* moe_layer_forward with FP8 expert weights (routed as in
 * moe_grouped_ffn_fp8w; shared_w13_q [2*shared_I, H] + shared_w13_scale
 * [2*shared_I/128, H/128], shared_w2_q [H, shared_I] + shared_w2_scale
 * [H/128, shared_I/128], all NULL when shared_I == 0). */
moe_status moe_layer_forward_fp8w(const moe_config* cfg, const float* logits, const void* x,
                                  const uint8_t* w13_q, const float* w13_scale,
                                  const uint8_t* w2_q, const float* w2_scale,
                                  const uint8_t* shared_w13_q, const float* shared_w13_scale,
                                  const uint8_t* shared_w2_q, const float* shared_w2_scale,
                                  void* out, int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  float* balancedness, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------
 * FP8 activations as well (W8A8; the MoE inference blog, "Communication
 * pressure": token activations may be quantized to FP8 before dispatch, and
 * the low-precision expert GEMM).  An activation matrix X [R, C] (C a
 * multiple of 128) is held as
 *   q     [R, C] uint8 E4M3 codes;
 *   scale [R, C/128] fp32, one power of two per 1 x 128 piece of a row;
 *   X[r][c] = E4M3(q[r][c]) * scale[r][c/128].
 * Scales follow the weights' rule (the smallest s with max|piece| <= 448 * 2^s,
 * 0 for an all-zero piece), with s kept in [-127, 127] -- the range of the
 * 8-bit power-of-two scales of the FP8 matrix instructions -- in the weights'
 * quantizer too.  In the layer, x is quantized before dispatch; GEMM 1
 * multiplies E4M3 x and weights with fp32 accumulation, h = silu(g) * u is
 * rounded to bf16 and quantized the same way, and GEMM 2 multiplies E4M3 h
 * and W2; y_perm and out stay bf16.
 * ------------------------------------------------------------------------ */

/* Quantize bf16 rows src [rows, cols] (cols a multiple of 128; 16-byte
 * aligned src and q) into q [rows, cols] and scale [rows, cols/128] as
 * above.  MOE_ERR_INVALID_ARG for bad sizes or pointers; asynchronous. */
moe_status moe_quantize_act_fp8(int32_t rows, int32_t cols, const void* src, uint8_t* q,
                                float* scale, void* stream);

/* moe_grouped_ffn_fp8w with FP8 activations: x_perm_q [R, H] codes and
 * x_perm_scale [R, H/128] (the rows of moe_permute's x_perm, quantized with
 * moe_quantize_act_fp8).  Other arguments, outputs and errors as
 * moe_grouped_ffn_fp8w. */
moe_status moe_grouped_ffn_w8a8(const moe_config* cfg, const uint8_t* x_perm_q,
                                const float* x_perm_scale, const int32_t* seg_offsets,
                                const int32_t* seg_expert, const uint8_t* w13_q,
                                const float* w13_scale, const uint8_t* w2_q,
                                const float* w2_scale, const float* row_scale, void* y_perm,
                                void* workspace, size_t workspace_bytes, void* stream);

/* moe_layer_forward_fp8w with FP8 activations: x [T, H] bf16 is quantized
 * inside the call (into the workspace) before dispatch.  Arguments, outputs
 * and errors as moe_layer_forward_fp8w. */
moe_status moe_layer_forward_w8a8(const moe_config* cfg, const float* logits, const void* x,
                                  const uint8_t* w13_q, const float* w13_scale,
                                  const uint8_t* w2_q, const float* w2_scale,
                                  const uint8_t* shared_w13_q, const float* shared_w13_scale,
                                  const uint8_t* shared_w2_q, const float* shared_w2_scale,
                                  void* out, int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  float* balancedness, void* workspace, size_t workspace_bytes,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
