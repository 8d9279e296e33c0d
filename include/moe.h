/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer hot path.
 *
 * The layer that follows attention in a Mixture-of-Experts transformer, in the
 * five steps of the MoE FlashAttention page (http://www.framerc.cn/news/2508843/,
 * section "FlashAttention 在 MoE 模型里的位置"): the attention output is given;
 * each token is routed to its top-k experts, tokens are grouped by expert, each
 * expert runs its FFN on its own tokens, and the expert outputs are merged
 * weighted by the route weights.
 *
 * Page references used below:
 *   [FA-MoE]  http://www.framerc.cn/news/2508843/  (MoE layer, fusions, fused call)
 *   [Router]  https://2048ai.net/6a1268d0662f9a54cb76af71.html  (router, dispatch, capacity)
 *   [LightOP] https://adg.csdn.net/6a3a2e8f10ee7a33f281154b.html (fused gate/top-k,
 *             MoE Align, MoE Sum, W8A8)
 *
 * Conventions for every entry point
 *   - Memory: every pointer argument is DEVICE memory owned by the caller
 *     unless stated otherwise.  The library never allocates or frees device
 *     memory; scratch comes from a caller-provided workspace whose minimum
 *     size the matching *_workspace_size() returns (workspace pointers must be
 *     256-byte aligned; tensor pointers 16-byte aligned).
 *   - Layout: row-major, densely packed; bf16 is the IEEE bfloat16 bit pattern.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  Calls
 *     enqueue kernels and return at once; they never synchronise the device and
 *     never copy device data to the host.  Kernel faults surface at the
 *     caller's next synchronisation, as usual in HIP.
 *   - Errors: every call returns a moe_status and throws nothing.  Argument
 *     checks run on the host before any launch, so an error return means
 *     nothing was enqueued.  moe_last_error() gives a thread-local message.
 *     An unsupported shape or dtype is an error, never a slower fallback.
 *   - T == 0 is a valid no-op returning MOE_OK.
 *   - Values: NaN/Inf inputs are not supported and not checked.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null required pointer, negative size, k < 1, k > E, ... */
  MOE_ERR_UNSUPPORTED = 2, /* dtype combination or shape the kernels do not implement */
  MOE_ERR_WORKSPACE = 3,   /* workspace too small or misaligned */
  MOE_ERR_HIP = 4          /* a HIP call or kernel launch failed */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_I8 = 2,
  MOE_I4 = 3,  /* int4 codes packed two per byte (see moe_pack_int4); weights only */
  MOE_I4A8 = 4 /* the same packed int4 weights, run with int8 activations (W4A8) */
} moe_dtype;

/* Limits shared by all entry points: 1 <= E <= 256, 1 <= k <= min(E, 8),
 * H % 64 == 0, I % 64 == 0, T * k < 2^31. */

/* ---------------------------------------------------------------- route --
 * Gate, softmax, top-k and renormalisation in one pass over x
 * ([Router] section on the router as a small network; [LightOP] section 3.1,
 * fused gate + softmax + top-k), optionally with the per-token int8
 * quantisation of x ([LightOP] section 4.1, per-token int8 quantisation).
 *
 *   x        [T, H]  x_dtype (MOE_F32 or MOE_BF16): attention output
 *   wg       [E, H]  wg_dtype (MOE_F32 or MOE_BF16): gate weight (Linear(H, E))
 *   bias     [E] fp32 or NULL: added to the logits before the softmax
 *   topk_ids [T, k] int32 out: expert ids, most probable first; equal
 *            probabilities go to the lower id
 *   topk_w   [T, k] fp32 out: selected probabilities divided by their sum
 *   topk_p   [T, k] fp32 out or NULL: selected softmax probabilities
 *   xq, xs   [T, H] int8 and [T] fp32 out, both or neither: per-token codes
 *            round-half-even(x / s) clamped to [-128, 127] with
 *            s = absmax(x row) / 127 (1 for an all-zero row); fp32 IEEE
 *            arithmetic, bit-exact to that definition
 * Logits, the softmax and the selection are fp32.  Supported: E <= 16 with
 * any x/wg dtype; 16 < E <= 256 (E % 16 == 0) with bf16 x and bf16 wg.
 */
size_t moe_route_workspace_size(int64_t T, int32_t H, int32_t E, int32_t k);
moe_status moe_route(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                     const float* bias, int64_t T, int32_t H, int32_t E, int32_t k,
                     int32_t* topk_ids, float* topk_w, float* topk_p, int8_t* xq, float* xs,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Group-limited routing ([LightOP] section 3.1, Moe Fuse Gate: groups are
 * picked first, each group's Top1/Top2 kept).  The page gives no formula;
 * this is the reading implemented:
 *   the E experts form n_group contiguous groups of E / n_group experts;
 *   a group's score is the sum of its two largest softmax probabilities (its
 *   only one when groups have one expert);
 *   the topk_group highest-scoring groups are kept (equal scores: the lower
 *   group index first), and top-k runs over their experts only, ordered and
 *   renormalised exactly as in moe_route; topk_p holds the probabilities of
 *   the full softmax over all E experts.
 * topk_group == n_group gives moe_route's result.
 * Arguments as in moe_route (same workspace size), plus:
 *   n_group     in [1, 64], divides E;  topk_group in [1, n_group];
 *   k <= topk_group * E / n_group, else MOE_ERR_INVALID_ARG.
 * Supported: 16 < E <= 256, E % 16 == 0, bf16 x and bf16 wg (the MFMA
 * logits path); other shapes return MOE_ERR_UNSUPPORTED. */
moe_status moe_route_grouped(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                             const float* bias, int64_t T, int32_t H, int32_t E, int32_t k,
                             int32_t n_group, int32_t topk_group, int32_t* topk_ids, float* topk_w,
                             float* topk_p, int8_t* xq, float* xs, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------- capacity -----
 * Per-expert capacity C = ceil(factor * T * k / E) ([Router] section on
 * communication/computation overlap, capacity limit, with the load counted as
 * the T*k assignments).  factor <= 0 means no limit and returns 0.
 * The factor is taken as the fraction p/q nearest to it with q <= 2^20 (its
 * continued-fraction best approximation), so a decimal factor such as 1.1 or
 * 1.25 counts as the decimal (11/10, 5/4) and not as the double just above
 * or below it; C is then ceil(p*T*k / (q*E)) in integers.  Factors outside
 * [2^-20, 2^30] return -1 (not a capacity: check before passing it on, since
 * moe_align treats any capacity <= 0 as no limit).  Host only.
 */
int64_t moe_capacity(int64_t T, int32_t k, int32_t E, double factor);

/* ------------------------------------------------------------- align -----
 * Group the T*k (token, choice) assignments by expert: per-expert histogram,
 * capacity cut, exclusive prefix sum, expert-sorted slot list and the GEMM
 * row-tile list ([Router] section on token dispatch, counting per
 * destination; [LightOP] section 3.2, MoE Align: prefix sum, hierarchical
 * atomics, fused map/mask/fill).
 *
 * Slot s = t*k + j is token t's j-th choice.  rank(s) = number of slots
 * before s (in slot order) routed to the same expert.  s is kept iff
 * capacity <= 0 or rank(s) < capacity; dropped slots take the residual path.
 *   topk_ids    [T, k] int32 in, each in [0, E) (an id outside is dropped)
 *   counts      [E] int32 out: assignments per expert before the cut
 *   offsets     [E+1] int32 out: exclusive prefix sum of min(counts, C);
 *               offsets[E] = N = kept assignments
 *   sorted_slot [T*k] int32 out: sorted_slot[offsets[e] + rank] = slot for
 *               kept slots, in slot order within each expert; -1 at [N, T*k)
 *   pos         [T*k] int32 out: sorted row of each slot, -1 if dropped
 *   tiles       [moe_align_max_tiles(...)][4] int32 out: (expert, first
 *               sorted row, row count, 0) for row tiles of at most block_m
 *               rows, one expert each, in expert order; unused entries are
 *               (-1, 0, 0, 0)
 *   num_tiles   [1] int32 out;  num_dropped [1] int32 out: T*k - N
 * Every output is deterministic and bit-exact to that definition.
 * block_m in {16, 32, 64, 128, 256}.
 */
size_t moe_align_workspace_size(int64_t T, int32_t k, int32_t E);
int64_t moe_align_max_tiles(int64_t T, int32_t k, int32_t E, int32_t block_m);
moe_status moe_align(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                     int64_t capacity, int32_t block_m, int32_t* counts, int32_t* offsets,
                     int32_t* sorted_slot, int32_t* pos, int32_t* tiles, int32_t* num_tiles,
                     int32_t* num_dropped, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ------------------------------------------------------ route + align -----
 * moe_route followed by moe_align, in one launch where one workgroup can
 * take every token (the route step's own workgroup for E <= 16 and T <= 16;
 * the top-k workgroup for E > 16 and T <= 64: decode-sized batches), which
 * then aligns the T*k slots it has just routed (the MoE FlashAttention page's
 * first fusion, routing fused with grouping by expert, [FA-MoE] "融合一").
 * Larger batches run two launches: where the route kernel takes every
 * expert of its tokens (E <= 64), each of its workgroups also publishes its
 * per-expert selection counts and a single align launch takes them
 * (per-expert bases and offsets from integer sums of the counts, then the
 * stable ranking), instead of histogramming the ids again; otherwise the
 * route step is followed by moe_align.  Arguments, outputs and errors are
 * those of moe_route and moe_align (capacity, block_m and the align outputs
 * as in moe_align); every output equals what the two calls give.
 * moe_last_dispatch() names the path taken.  The workspace
 * (moe_route_align_workspace_size bytes) serves both steps.  The one-launch
 * form saves the host one launch; on the GPU it is no faster (one workgroup
 * takes every token's top-k), so moe_layer uses the two-launch forms. */
size_t moe_route_align_workspace_size(int64_t T, int32_t H, int32_t E, int32_t k);
moe_status moe_route_align(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype, const float* bias,
                           int64_t T, int32_t H, int32_t E, int32_t k, int64_t capacity, int32_t block_m,
                           int32_t* topk_ids, float* topk_w, float* topk_p, int8_t* xq, float* xs,
                           int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* pos, int32_t* tiles,
                           int32_t* num_tiles, int32_t* num_dropped, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ---------------------------------------------------------- expert FFN ---
 * Per-expert SwiGLU on the expert-sorted rows as a grouped GEMM pair
 * ([FA-MoE] step 4 and its fused call with stacked expert weights and
 * activation "silu"; [LightOP] sections 4.1 and 4.3, W16A16 and W8A8 MoE):
 *   for sorted row r of expert e with slot s = sorted_slot[r], t = s / k:
 *     h[r]  = silu(W1[e] a_t) * (W3[e] a_t),    silu(z) = z / (1 + exp(-z))
 *     Y[r]  = w * (W2[e] h[r]),  w = topk_w[s] (1 if topk_w is NULL)
 *   act_dtype MOE_F32 / MOE_BF16: a_t = x[t] (w_dtype must equal act_dtype)
 *   act_dtype MOE_I8 (W8A8, w_dtype MOE_I8): a_t = xq[t] with scale xs[t];
 *     int32 accumulation, dequantised by xs[t] * s13[e][n]; h, rounded to
 *     bf16, is quantised per row with the per-token rule before the second
 *     GEMM, whose int32 result is scaled by that row scale * s2[e][n]
 *     ([LightOP] section 4.1)
 *   act_dtype MOE_BF16 with w_dtype MOE_I4 (W4A16, [LightOP] section 4.3):
 *     a_t = x[t]; each weight is its int4 code (in [-8, 7]) times the
 *     per-output-channel scale s13[e][n] or s2[e][n]; bf16 MFMA with fp32
 *     accumulation, the channel scale applied to the sum (before SwiGLU in
 *     the up GEMM); h is bf16 as in W16A16
 *   act_dtype MOE_I8 with w_dtype MOE_I4A8 (W4A8, [LightOP] section 4.3):
 *     the W8A8 rule above with the packed int4 codes as the int8 weights
 *   x        [T, H] act_dtype;  xs [T] fp32 (act_dtype MOE_I8 only, else NULL)
 *   w13      [E, 2I, H] w_dtype: rows 0..I-1 are W1[e], rows I..2I-1 W3[e]
 *            (MOE_I4, MOE_I4A8: [E, 2I, H/2] bytes as written by moe_pack_int4)
 *   w2       [E, H, I] w_dtype (MOE_I4, MOE_I4A8: [E, H, I/2] packed bytes)
 *   s13, s2  [E, 2I], [E, H] fp32 per-output-channel scales (MOE_I8,
 *            MOE_I4 and MOE_I4A8 only)
 *   sorted_slot, tiles, num_tiles: from moe_align with the same block_m;
 *   block_m must equal moe_ffn_block_m() for this shape
 *   y_sorted [T*k, H] y_dtype out (MOE_F32 for f32 activations, else
 *            MOE_BF16): rows >= N are not written
 */
int32_t moe_ffn_block_m(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t w_dtype);

/* Offline weight preparation for W4A16: packs int4 codes, given one per int8
 * ([rows, K], each in [-8, 7]; other values are stored modulo 16), two per
 * byte along K: packed byte j of a row holds code 2j in its low nibble and
 * code 2j+1 in its high nibble (two's complement nibbles).  [rows, K/2]
 * bytes out.  K % 64 == 0; both pointers 16-byte aligned; device memory. */
moe_status moe_pack_int4(const int8_t* codes, int64_t rows, int32_t K, uint8_t* packed, void* stream);
size_t moe_ffn_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                              int32_t w_dtype);
moe_status moe_expert_ffn(const void* x, int32_t act_dtype, const float* xs, const void* w13,
                          const void* w2, int32_t w_dtype, const float* s13, const float* s2,
                          const int32_t* sorted_slot, const int32_t* tiles,
                          const int32_t* num_tiles, int32_t block_m, const float* topk_w,
                          int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, void* y_sorted,
                          int32_t y_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/* The two halves of moe_expert_ffn as separate launches (the up GEMM with
 * its SwiGLU epilogue, and the down GEMM with its route-weight epilogue, each
 * one step of the layer).  The workspace (moe_ffn_workspace_size bytes)
 * carries h from moe_ffn_up to moe_ffn_down: pass the same workspace, with
 * nothing else writing it in between, on the same stream.  Arguments as in
 * moe_expert_ffn; for W8A8 the down call quantises h per row first. */
moe_status moe_ffn_up(const void* x, int32_t act_dtype, const float* xs, const void* w13,
                      int32_t w_dtype, const float* s13, const int32_t* sorted_slot,
                      const int32_t* tiles, const int32_t* num_tiles, int32_t block_m, int64_t T,
                      int32_t H, int32_t I, int32_t E, int32_t k, void* workspace,
                      size_t workspace_bytes, void* stream);
moe_status moe_ffn_down(const void* w2, int32_t w_dtype, const float* s2,
                        const int32_t* sorted_slot, const int32_t* tiles,
                        const int32_t* num_tiles, int32_t block_m, const float* topk_w, int64_t T,
                        int32_t H, int32_t I, int32_t E, int32_t k, void* y_sorted, int32_t y_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ combine ----
 * Route-weighted merge of each token's kept expert rows ([FA-MoE] step 5 and
 * its fusion of weighting into accumulation; [LightOP] section 3.2, MoE Sum):
 *   out[t] = sum over j with pos[t*k+j] >= 0 of  w * y_sorted[pos[t*k+j]]
 *   w = topk_w[t*k+j], or 1 when topk_w is NULL (rows already weighted)
 * A token with every slot dropped gets 0.  fp32 accumulation in slot order.
 *   y_sorted [*, H] y_dtype (MOE_F32 / MOE_BF16);  out [T, H] out_dtype.
 */
moe_status moe_combine(const void* y_sorted, int32_t y_dtype, const int32_t* pos,
                       const float* topk_w, int64_t T, int32_t k, int32_t H, void* out,
                       int32_t out_dtype, void* stream);

/* moe_combine plus the shared expert's term and a bias, fused into the same
 * single write ([LightOP] section 3.2, MoE Sum: shared-expert factor and bias
 * add):
 *   out[t, h] = ((sum as in moe_combine) + shared_factor * shared[t, h]) + bias[h]
 * each step rounded in fp32, then one rounding to out_dtype.
 *   shared [T, H] in out_dtype (the shared expert's output), or NULL for none;
 *     it may be the same buffer as out (an in-place update), but must not
 *     otherwise overlap it.
 *   bias [H] fp32, 16-byte aligned, or NULL for none.
 * Other arguments and errors as in moe_combine; a non-finite shared_factor
 * is MOE_ERR_INVALID_ARG.  With shared and bias both NULL the result equals
 * moe_combine's. */
moe_status moe_combine_shared(const void* y_sorted, int32_t y_dtype, const int32_t* pos,
                              const float* topk_w, int64_t T, int32_t k, int32_t H,
                              const void* shared, float shared_factor, const float* bias,
                              void* out, int32_t out_dtype, void* stream);

/* -------------------------------------------------------------- layer ----
 * The whole MoE branch (route, align, expert FFN, combine) enqueued on one
 * stream with no host synchronisation ([FA-MoE] fused MoE call: attention
 * output, router weight, stacked expert weights, expert count, top-k, silu).
 *   x [T, H] (MOE_F32 or MOE_BF16), wg [E, H], bias [E] or NULL,
 *   w13/w2/s13/s2 as in moe_expert_ffn, capacity as in moe_align
 *   (<= 0: none), out [T, H] with out_dtype == x_dtype.
 *   w_dtype MOE_I8 quantises x per token inside the route step (W8A8);
 *   w_dtype MOE_I4 (packed int4 weights, with s13/s2) needs bf16 x (W4A16);
 *   w_dtype MOE_I4A8 (the same weights) quantises x per token (W4A8).
 * aux (host struct, may be NULL; each member may be NULL) names device
 * buffers the layer writes its intermediates to instead of the workspace:
 * topk_ids/topk_w/topk_p [T,k], counts [E], offsets [E+1], sorted_slot and
 * pos [T*k], num_dropped [1], xq [T,H] int8 and xs [T] (W8A8 only).
 * aux->stage_events (each entry may be NULL) are hipEvent_t handles the
 * caller created; the layer records them on its stream before the route
 * step and after each of its five steps (route, align, up GEMM, down GEMM
 * with the W8A8 quantisation of h, combine), so the caller can time every
 * step inside a layer call.  They are checked (hipEventQuery) before the
 * first launch; the layer only records them.
 * The layer returns the MoE branch only: the caller adds the residual, which
 * is where dropped assignments go.
 */
typedef struct moe_layer_aux {
  int32_t* topk_ids;
  float* topk_w;
  float* topk_p;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slot;
  int32_t* pos;
  int32_t* num_dropped;
  int8_t* xq;
  float* xs;
  void* stage_events[6];
} moe_layer_aux;

size_t moe_layer_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                int32_t x_dtype, int32_t w_dtype);
moe_status moe_layer(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                     const float* bias, const void* w13, const void* w2, int32_t w_dtype,
                     const float* s13, const float* s2, int64_t T, int32_t H, int32_t I,
                     int32_t E, int32_t k, int64_t capacity, void* out, int32_t out_dtype,
                     const moe_layer_aux* aux, void* workspace, size_t workspace_bytes,
                     void* stream);

/* moe_layer with the gate and sum variants of [LightOP] section 3 folded in:
 * group-limited routing (section 3.1, Moe Fuse Gate; as in
 * moe_route_grouped) and the shared expert's term plus a bias merged into
 * the combine (section 3.2, MoE Sum; as in moe_combine_shared).
 *   options (host struct, may be NULL = moe_layer):
 *     n_group      0: plain top-k; else group-limited routing with
 *                  topk_group kept groups (limits and supported shapes as in
 *                  moe_route_grouped: 16 < E <= 256, bf16 x and wg);
 *     shared       [T, H] device buffer in out_dtype, 16-byte aligned, or
 *                  NULL; it may be out itself (read before the write) but
 *                  must not otherwise overlap it;
 *     shared_factor  finite, scales shared;
 *     out_bias     [H] fp32 device buffer, 16-byte aligned, or NULL.
 * Workspace size as moe_layer_workspace_size; all other arguments and
 * errors as in moe_layer.  An invalid option is MOE_ERR_INVALID_ARG (an
 * unsupported routing shape MOE_ERR_UNSUPPORTED) before anything is
 * enqueued. */
typedef struct moe_layer_options {
  int32_t n_group;
  int32_t topk_group;
  const void* shared;
  float shared_factor;
  const float* out_bias;
} moe_layer_options;

moe_status moe_layer_ex(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                        const float* bias, const void* w13, const void* w2, int32_t w_dtype,
                        const float* s13, const float* s2, int64_t T, int32_t H, int32_t I,
                        int32_t E, int32_t k, int64_t capacity, void* out, int32_t out_dtype,
                        const moe_layer_aux* aux, const moe_layer_options* options, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ------------------------------------------------ allocation-free layer --
 * For callers that cannot allocate device memory or hand the library a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  moe_layer_noalloc is moe_layer with the workspace
 * taken from a scratch array the library itself holds on each GPU it runs on
 * (MOE_NOALLOC_SCRATCH_BYTES, for the life of the process); the caller still
 * passes x, the weights, out and, if it wants them, the aux buffers.  It
 * calls no allocating routine.  Shapes whose moe_layer_workspace_size
 * exceeds MOE_NOALLOC_SCRATCH_BYTES (16 MiB: decode-sized batches, e.g. up
 * to 128 tokens at H = 4096, E = 256, k = 8, I = 1024) return
 * MOE_ERR_UNSUPPORTED before anything is enqueued.  Arguments, outputs and
 * the other errors are moe_layer's; every output equals moe_layer's.
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (two host threads, or two streams
 * not ordered by the caller) race.  Calls on one stream are ordered. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
moe_status moe_layer_noalloc(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                             const float* bias, const void* w13, const void* w2, int32_t w_dtype,
                             const float* s13, const float* s2, int64_t T, int32_t H, int32_t I,
                             int32_t E, int32_t k, int64_t capacity, void* out, int32_t out_dtype,
                             const moe_layer_aux* aux, void* stream);

/* ------------------------------------------------------- diagnostics -----
 * moe_last_error: message of this thread's last failed call ("" if none).
 * moe_last_dispatch: kernel variants this thread's last successful call
 * enqueued (never a silent fallback: an unsupported case is an error).
 * Both return thread-local storage valid until the thread's next call.
 */
const char* moe_last_error(void);
const char* moe_last_dispatch(void);
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
