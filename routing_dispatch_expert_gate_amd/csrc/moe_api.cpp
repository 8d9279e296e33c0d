// C ABI of the MoE layer hot path: argument validation, workspace carving and
// kernel dispatch.  Every check runs on the host before the first launch, so
// an error return means nothing was enqueued; unsupported cases are errors,
// never a slower path.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <mutex>
#include <string>

#include "moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_err;
thread_local std::string g_dispatch;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

moe_status ok(const std::string& d) {
  g_err.clear();
  g_dispatch = d;
  return MOE_OK;
}

bool al(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t a256(size_t b) { return (b + 255) & ~(size_t)255; }
bool is_act(int d) { return d == MOE_F32 || d == MOE_BF16; }

// Shape checks shared by every entry point.
moe_status check_dims(int64_t T, int32_t H, int32_t E, int32_t k) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1 (got %d)", E);
  if (k < 1) return fail(MOE_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "k (%d) must be <= E (%d)", k, E);
  if (H < 1) return fail(MOE_ERR_INVALID_ARG, "H must be >= 1 (got %d)", H);
  if (E > moe::kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E > %d is not supported (got %d)", moe::kMaxE, E);
  if (k > moe::kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k > %d is not supported (got %d)", moe::kMaxK, k);
  if (H % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "H must be a multiple of 64 (got %d)", H);
  if (T * (int64_t)k >= (int64_t)1 << 31) return fail(MOE_ERR_UNSUPPORTED, "T*k must be < 2^31");
  return MOE_OK;
}

moe_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL; %zu bytes needed", need);
  if (!al(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  return MOE_OK;
}

#define MOE_TRY(expr)              \
  do {                             \
    moe_status st_ = (expr);       \
    if (st_ != MOE_OK) return st_; \
  } while (0)

#define MOE_NONNULL(p)                                                            \
  do {                                                                            \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "required pointer " #p " is NULL"); \
  } while (0)

#define MOE_ALIGNED(p, a)                                                              \
  do {                                                                                 \
    if ((p) && !al((p), (a)))                                                          \
      return fail(MOE_ERR_INVALID_ARG, "pointer " #p " must be %d-byte aligned", (int)(a)); \
  } while (0)

moe_status route_checks(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype, int64_t T,
                        int32_t H, int32_t E, int32_t k, int32_t* ids, float* w, int8_t* xq,
                        float* xs, moe::RoutePlan* plan, bool fused_ok = true) {
  MOE_TRY(check_dims(T, H, E, k));
  if (!is_act(x_dtype)) return fail(MOE_ERR_UNSUPPORTED, "x dtype must be MOE_F32 or MOE_BF16");
  if (!is_act(wg_dtype)) return fail(MOE_ERR_UNSUPPORTED, "wg dtype must be MOE_F32 or MOE_BF16");
  if ((xq == nullptr) != (xs == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "xq and xs must both be given or both be NULL");
  *plan = moe::plan_route(T, H, E, k, x_dtype, wg_dtype, fused_ok);
  if (plan->kind < 0)
    return fail(MOE_ERR_UNSUPPORTED,
                "route: E=%d with x/wg dtypes %d/%d and H=%d is not implemented (E<=8 with H<=8192 or "
                "E<=16 with H<=4096, any dtype; or E%%16==0, E<=256 with bf16 x and bf16 wg)",
                E, x_dtype, wg_dtype, H);
  if (T == 0) return MOE_OK;
  MOE_NONNULL(x);
  MOE_NONNULL(wg);
  MOE_NONNULL(ids);
  MOE_NONNULL(w);
  MOE_ALIGNED(x, 16);
  MOE_ALIGNED(wg, 16);
  MOE_ALIGNED(xq, 8);
  return MOE_OK;
}

std::string route_name(const moe::RoutePlan& p) {
  char b[160];
  if (p.kind == 0)
    snprintf(b, sizeof b, "route_fma_kernel(tokens/wg=%d,waves=%d)", p.bt, p.nw);
  else if (p.kind == 3)
    snprintf(b, sizeof b, "route_fused_kernel(tokens/wg=%d,parts=%d)", p.bt, p.ks);
  else
    snprintf(b, sizeof b, "route_gemm_kernel(tokens/wg=%d,experts/wg=%d,ksplit=%d)+route_topk_kernel", p.bt,
             p.be, p.ks);
  return b;
}

moe_status ffn_checks(int32_t act_dtype, int32_t w_dtype, int32_t y_dtype, int64_t T, int32_t H,
                      int32_t I, int32_t E, int32_t k) {
  MOE_TRY(check_dims(T, H, E, k));
  if (I < 1) return fail(MOE_ERR_INVALID_ARG, "I must be >= 1 (got %d)", I);
  if (I % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "I must be a multiple of 64 (got %d)", I);
  const bool ok_combo = (act_dtype == MOE_F32 && w_dtype == MOE_F32 && y_dtype == MOE_F32) ||
                        (act_dtype == MOE_BF16 && w_dtype == MOE_BF16 && y_dtype == MOE_BF16) ||
                        (act_dtype == MOE_I8 && w_dtype == MOE_I8 && y_dtype == MOE_BF16) ||
                        (act_dtype == MOE_BF16 && w_dtype == MOE_I4 && y_dtype == MOE_BF16) ||
                        (act_dtype == MOE_I8 && w_dtype == MOE_I4A8 && y_dtype == MOE_BF16);
  if (!ok_combo)
    return fail(MOE_ERR_UNSUPPORTED,
                "expert FFN dtypes (act %d, w %d, y %d) not implemented: use f32/f32/f32, "
                "bf16/bf16/bf16, i8/i8/bf16, bf16/i4/bf16 or i8/i4a8/bf16",
                act_dtype, w_dtype, y_dtype);
  if ((w_dtype == MOE_I8 || w_dtype == MOE_I4A8) && (H % 128 != 0 || I % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "W8A8 and W4A8 need H and I multiples of 128 (got %d, %d)", H, I);
  // the GEMM kernels address activations and one expert's weights with
  // 32-bit byte offsets
  const int64_t eb = act_dtype == MOE_F32 ? 4 : (act_dtype == MOE_BF16 ? 2 : 1);
  if (T * H * eb >= ((int64_t)1 << 32) || 2 * (int64_t)I * H * eb >= ((int64_t)1 << 32))
    return fail(MOE_ERR_UNSUPPORTED, "activations (T*H) and each expert's weights (2*I*H) must be < 4 GiB");
  return MOE_OK;
}

bool valid_block_m(int32_t b) { return b == 16 || b == 32 || b == 64 || b == 128 || b == 256; }

// Layout of the fused layer's workspace.
struct LayerCarve {
  size_t ids, w, p, counts, offsets, sorted_slot, pos, tiles, num_tiles, num_dropped, xq, xs, y,
      scratch, total;
  moe::RoutePlan rp;
  moe::AlignPlan ap;
  moe::FfnPlan fp;
};

// grouped: the group-limited router (never the fused kind).  The scratch
// covers the two-kernel router either way, so one workspace size serves
// moe_layer and moe_layer_ex with any options.
LayerCarve carve_layer(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t x_dtype,
                       int32_t wg_dtype, int32_t w_dtype, bool grouped = false) {
  LayerCarve c{};
  const int64_t n = T * k;
  c.rp = moe::plan_route(T, H, E, k, x_dtype, wg_dtype, !grouped);
  const moe::RoutePlan rp2 = moe::plan_route(T, H, E, k, x_dtype, wg_dtype, false);
  c.ap = moe::plan_align(T, k, E);
  c.fp = moe::plan_ffn(T, H, I, E, k, w_dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += a256(bytes);
    return o;
  };
  c.ids = take(n * 4);
  c.w = take(n * 4);
  c.p = take(n * 4);
  c.counts = take((size_t)E * 4);
  c.offsets = take((size_t)(E + 1) * 4);
  c.sorted_slot = take(n * 4);
  c.pos = take(n * 4);
  c.tiles = take((size_t)c.fp.max_tiles * 16);
  c.num_tiles = take(4);
  c.num_dropped = take(4);
  const bool a8 = w_dtype == MOE_I8 || w_dtype == MOE_I4A8;
  c.xq = take(a8 ? (size_t)T * H : 0);
  c.xs = take(a8 ? (size_t)T * 4 : 0);
  c.y = take(n * (size_t)H * (w_dtype == MOE_F32 ? 4 : 2));
  size_t scratch = c.rp.ws_bytes > rp2.ws_bytes ? c.rp.ws_bytes : rp2.ws_bytes;
  if (c.ap.ws_bytes > scratch) scratch = c.ap.ws_bytes;
  // the route step's per-workgroup counts, read by the align step (after
  // the route step's own workspace, which the align step does not use)
  const size_t whist = moe::route_hist_bytes(c.rp, T, k, E);
  if (whist > scratch) scratch = whist;
  if (c.fp.ws_bytes > scratch) scratch = c.fp.ws_bytes;
  c.scratch = take(scratch);
  c.total = off;
  return c;
}

// ------------------------------------------------------------- capacity --
// A capacity factor such as 1.1 has no exact double: the stored value lies a
// little above or below the decimal, and ceil(factor * load / E) can then
// land one off when the decimal quotient is an integer.  The factor is
// therefore taken as the fraction p/q nearest to it with q <= 2^20 (the
// continued-fraction best approximation, ties to the convergent), which
// recovers every decimal of up to six places, and the ceiling is taken in
// integers.
typedef unsigned __int128 u128;
constexpr double kCapFactorMin = 0x1p-20, kCapFactorMax = 0x1p30;
constexpr uint64_t kCapDenMax = 1u << 20;

// a * b as a 192-bit value (hi, lo) for a < 2^128, b < 2^64
struct U192 {
  uint64_t hi;
  u128 lo;
};
U192 mul_u128_u64(u128 a, uint64_t b) {
  const u128 lo = (u128)(uint64_t)a * b;
  const u128 mid = (u128)(uint64_t)(a >> 64) * b + (lo >> 64);
  return U192{(uint64_t)(mid >> 64), (mid << 64) | (u128)(uint64_t)lo};
}
bool le192(const U192& a, const U192& b) { return a.hi != b.hi ? a.hi < b.hi : a.lo <= b.lo; }

// The fraction nearest to f (in [2^-20, 2^30]) with denominator <= dmax.
void nearest_fraction(double f, uint64_t dmax, uint64_t* p_out, uint64_t* q_out) {
  // f = N / D exactly, in lowest terms (D a power of two)
  int ex = 0;
  const double mant = std::frexp(f, &ex);
  uint64_t m = (uint64_t)std::ldexp(mant, 53);
  int e = ex - 53;
  while ((m & 1) == 0 && e < 0) {
    m >>= 1;
    ++e;
  }
  const u128 N = e >= 0 ? (u128)m << e : (u128)m;
  const u128 D = e >= 0 ? (u128)1 : (u128)1 << (-e);
  if (D <= dmax) {
    *p_out = (uint64_t)N;
    *q_out = (uint64_t)D;
    return;
  }
  // convergents p1/q1 of N/D while their denominator stays <= dmax
  u128 p0 = 0, q0 = 1, p1 = 1, q1 = 0, n = N, d = D;
  for (;;) {
    const u128 a = n / d;
    const u128 q2 = q0 + a * q1;
    if (q2 > dmax) break;
    const u128 p2 = p0 + a * p1;
    p0 = p1;
    q0 = q1;
    p1 = p2;
    q1 = q2;
    const u128 r = n - a * d;
    n = d;
    d = r;
  }
  // the best semiconvergent below the bound, against the last convergent
  const u128 kk = (dmax - q0) / q1;
  const u128 pb = p0 + kk * p1, qb = q0 + kk * q1;
  // |p1/q1 - N/D| <= |pb/qb - N/D|  <=>  |p1 D - N q1| qb <= |pb D - N qb| q1
  auto absdiff = [](u128 a, u128 b) { return a > b ? a - b : b - a; };
  const U192 lhs = mul_u128_u64(absdiff(p1 * D, N * q1), (uint64_t)qb);
  const U192 rhs = mul_u128_u64(absdiff(pb * D, N * qb), (uint64_t)q1);
  if (le192(lhs, rhs)) {
    *p_out = (uint64_t)p1;
    *q_out = (uint64_t)q1;
  } else {
    *p_out = (uint64_t)pb;
    *q_out = (uint64_t)qb;
  }
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }
const char* moe_last_dispatch(void) { return g_dispatch.c_str(); }
const char* moe_version(void) { return "moe-gfx950 0.1.0"; }

int64_t moe_capacity(int64_t T, int32_t k, int32_t E, double factor) {
  if (!(factor > 0.0) || E < 1 || T < 0 || k < 1) return 0;
  if (!(factor >= kCapFactorMin && factor <= kCapFactorMax)) return -1;
  uint64_t p, q;
  nearest_fraction(factor, kCapDenMax, &p, &q);
  // ceil(p * T * k / (q * E)) in integers: p < 2^51, T * k < 2^31
  const u128 num = (u128)p * (u128)(T * (int64_t)k), den = (u128)q * (u128)E;
  return (int64_t)((num + den - 1) / den);
}

size_t moe_route_workspace_size(int64_t T, int32_t H, int32_t E, int32_t k) {
  // the two-kernel plan's (the fused kind needs none): the same size serves
  // moe_route_grouped
  return moe::plan_route(T, H, E, k, MOE_BF16, MOE_BF16, false).ws_bytes;
}

moe_status moe_route(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                     const float* bias, int64_t T, int32_t H, int32_t E, int32_t k,
                     int32_t* topk_ids, float* topk_w, float* topk_p, int8_t* xq, float* xs,
                     void* workspace, size_t workspace_bytes, void* stream) {
  moe::RoutePlan plan;
  MOE_TRY(route_checks(x, x_dtype, wg, wg_dtype, T, H, E, k, topk_ids, topk_w, xq, xs, &plan));
  if (T == 0) return ok("none (T=0)");
  MOE_TRY(check_ws(workspace, workspace_bytes, plan.ws_bytes));
  hipError_t e = moe::launch_route(plan, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, topk_ids, topk_w,
                                   topk_p, xq, xs, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_route launch");
  return ok(route_name(plan));
}

moe_status moe_route_grouped(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                             const float* bias, int64_t T, int32_t H, int32_t E, int32_t k,
                             int32_t n_group, int32_t topk_group, int32_t* topk_ids, float* topk_w,
                             float* topk_p, int8_t* xq, float* xs, void* workspace,
                             size_t workspace_bytes, void* stream) {
  MOE_TRY(check_dims(T, H, E, k));
  if (n_group < 1 || n_group > 64 || E % n_group != 0)
    return fail(MOE_ERR_INVALID_ARG, "n_group (%d) must divide E (%d) and be in [1, 64]", n_group, E);
  if (topk_group < 1 || topk_group > n_group)
    return fail(MOE_ERR_INVALID_ARG, "topk_group (%d) must be in [1, n_group=%d]", topk_group, n_group);
  if ((int64_t)k > (int64_t)topk_group * (E / n_group))
    return fail(MOE_ERR_INVALID_ARG, "k (%d) exceeds the %d experts of the kept groups", k,
                topk_group * (E / n_group));
  moe::RoutePlan plan;
  MOE_TRY(route_checks(x, x_dtype, wg, wg_dtype, T, H, E, k, topk_ids, topk_w, xq, xs, &plan, false));
  if (plan.kind != 2)
    return fail(MOE_ERR_UNSUPPORTED,
                "group-limited routing needs 16 < E <= 256, E %% 16 == 0, bf16 x and bf16 wg (got E=%d)", E);
  if (T == 0) return ok("none (T=0)");
  MOE_TRY(check_ws(workspace, workspace_bytes, plan.ws_bytes));
  hipError_t e = moe::launch_route_grouped(plan, x, wg, bias, T, H, E, k, n_group, topk_group, topk_ids,
                                           topk_w, topk_p, xq, xs, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_route_grouped launch");
  return ok(route_name(plan) + "<grouped>");
}

size_t moe_align_workspace_size(int64_t T, int32_t k, int32_t E) {
  return moe::plan_align(T, k, E).ws_bytes;
}

int64_t moe_align_max_tiles(int64_t T, int32_t k, int32_t E, int32_t block_m) {
  if (T < 0 || k < 1 || E < 1 || block_m < 1) return 0;
  return moe::align_max_tiles(T, k, E, block_m);
}

moe_status moe_align(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int64_t capacity,
                     int32_t block_m, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                     int32_t* pos, int32_t* tiles, int32_t* num_tiles, int32_t* num_dropped,
                     void* workspace, size_t workspace_bytes, void* stream) {
  MOE_TRY(check_dims(T, 64, E, k));
  if (!valid_block_m(block_m))
    return fail(MOE_ERR_INVALID_ARG, "block_m must be 16, 32, 64, 128 or 256 (got %d)", block_m);
  if (T == 0) return ok("none (T=0)");
  MOE_NONNULL(topk_ids);
  MOE_NONNULL(counts);
  MOE_NONNULL(offsets);
  MOE_NONNULL(sorted_slot);
  MOE_NONNULL(pos);
  MOE_NONNULL(tiles);
  MOE_NONNULL(num_tiles);
  MOE_NONNULL(num_dropped);
  MOE_ALIGNED(tiles, 16);
  const moe::AlignPlan plan = moe::plan_align(T, k, E);
  MOE_TRY(check_ws(workspace, workspace_bytes, plan.ws_bytes));
  const int64_t mt = moe::align_max_tiles(T, k, E, block_m);
  hipError_t e = moe::launch_align(plan, topk_ids, T, k, E, capacity, block_m, mt, counts, offsets,
                                   sorted_slot, pos, tiles, num_tiles, num_dropped, workspace,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_align launch");
  char b[128];
  if (plan.nblocks == 0)
    snprintf(b, sizeof b, "align_one_block_kernel(slots=%lld)", (long long)(T * k));
  else
    snprintf(b, sizeof b, "align_hist+align_scan+align_scatter(blocks=%d,slots/block=%d)", plan.nblocks,
             plan.slots_per_block);
  return ok(b);
}

size_t moe_route_align_workspace_size(int64_t T, int32_t H, int32_t E, int32_t k) {
  // the two steps run one after the other and share the workspace; route
  // kinds that publish per-workgroup counts put them there for the align
  const size_t r = moe_route_workspace_size(T, H, E, k), a = moe_align_workspace_size(T, k, E);
  size_t need = r > a ? r : a;
  for (int xd = MOE_F32; xd <= MOE_BF16; ++xd)
    for (int wd = MOE_F32; wd <= MOE_BF16; ++wd) {
      const moe::RoutePlan p = moe::plan_route(T, H, E, k, xd, wd);
      const size_t h = E > 0 ? moe::route_hist_bytes(p, T, k, E) : 0;
      if (p.kind >= 0 && h > need) need = h;
    }
  return need;
}

moe_status moe_route_align(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype, const float* bias,
                           int64_t T, int32_t H, int32_t E, int32_t k, int64_t capacity, int32_t block_m,
                           int32_t* topk_ids, float* topk_w, float* topk_p, int8_t* xq, float* xs,
                           int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* pos, int32_t* tiles,
                           int32_t* num_tiles, int32_t* num_dropped, void* workspace, size_t workspace_bytes,
                           void* stream) {
  moe::RoutePlan plan;
  MOE_TRY(route_checks(x, x_dtype, wg, wg_dtype, T, H, E, k, topk_ids, topk_w, xq, xs, &plan));
  if (!valid_block_m(block_m))
    return fail(MOE_ERR_INVALID_ARG, "block_m must be 16, 32, 64, 128 or 256 (got %d)", block_m);
  if (T == 0) return ok("none (T=0)");
  MOE_NONNULL(counts);
  MOE_NONNULL(offsets);
  MOE_NONNULL(sorted_slot);
  MOE_NONNULL(pos);
  MOE_NONNULL(tiles);
  MOE_NONNULL(num_tiles);
  MOE_NONNULL(num_dropped);
  MOE_ALIGNED(tiles, 16);
  MOE_TRY(check_ws(workspace, workspace_bytes, moe_route_align_workspace_size(T, H, E, k)));
  const int64_t mt = moe::align_max_tiles(T, k, E, block_m);
  const int64_t cap = capacity > 0 ? capacity : 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (moe::route_align_fusable(plan, T, k)) {
    e = moe::launch_route_align_fused(plan, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, topk_ids, topk_w, topk_p,
                                      xq, xs, workspace, cap, block_m, mt, counts, offsets, sorted_slot, pos,
                                      tiles, num_tiles, num_dropped, s);
    if (e != hipSuccess) return hip_fail(e, "moe_route_align launch");
    moe::RoutePlan named = plan;
    if (named.kind == 0) named.bt = (int)T;   // one workgroup takes every token
    return ok(route_name(named) + "+align (one launch)");
  }
  if (moe::route_publishes_hist(plan, T, k)) {
    // the route step publishes each workgroup's counts; one align launch
    // takes them (the layer's path for these route kinds)
    int32_t* whist = (int32_t*)((uint8_t*)workspace + moe::route_hist_offset(plan));
    e = moe::launch_route(plan, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, topk_ids, topk_w, topk_p, xq, xs,
                          workspace, s, whist);
    if (e != hipSuccess) return hip_fail(e, "moe_route_align route launch");
    e = moe::launch_align_from_route(topk_ids, whist, moe::route_hist_groups(plan, T, k),
                                     moe::route_hist_tokens(plan, k), T, k, E, cap, block_m,
                                     mt, counts, offsets, sorted_slot, pos, tiles, num_tiles, num_dropped, s);
    if (e != hipSuccess) return hip_fail(e, "moe_route_align align launch");
    return ok(route_name(plan) + " | align(from route counts, one launch)");
  }
  e = moe::launch_route(plan, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, topk_ids, topk_w, topk_p, xq, xs,
                        workspace, s);
  if (e != hipSuccess) return hip_fail(e, "moe_route_align route launch");
  const moe::AlignPlan ap = moe::plan_align(T, k, E);
  e = moe::launch_align(ap, topk_ids, T, k, E, cap, block_m, mt, counts, offsets, sorted_slot, pos, tiles,
                        num_tiles, num_dropped, workspace, s);
  if (e != hipSuccess) return hip_fail(e, "moe_route_align align launch");
  return ok(route_name(plan) + " | align");
}

moe_status moe_pack_int4(const int8_t* codes, int64_t rows, int32_t K, uint8_t* packed, void* stream) {
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
  if (K < 1 || K % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "K must be a positive multiple of 64 (got %d)", K);
  if (rows == 0) return ok("none (rows=0)");
  MOE_NONNULL(codes);
  MOE_NONNULL(packed);
  MOE_ALIGNED(codes, 16);
  MOE_ALIGNED(packed, 16);
  hipError_t e = moe::launch_pack_i4(codes, rows * (int64_t)K, packed, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_pack_int4 launch");
  return ok("pack_i4_kernel");
}

int32_t moe_ffn_block_m(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t w_dtype) {
  if (w_dtype < MOE_F32 || w_dtype > MOE_I4A8) return -1;
  return moe::plan_ffn(T, H, I, E, k, w_dtype).block_m;
}

size_t moe_ffn_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t w_dtype) {
  if (w_dtype < MOE_F32 || w_dtype > MOE_I4A8) return 0;
  return moe::plan_ffn(T, H, I, E, k, w_dtype).ws_bytes;
}

namespace {
// Checks shared by the FFN entry points; fills the plan.
moe_status ffn_prologue(int32_t act_dtype, int32_t w_dtype, int32_t y_dtype, int32_t block_m,
                        int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                        const int32_t* sorted_slot, const int32_t* tiles,
                        const int32_t* num_tiles, void* workspace, size_t workspace_bytes,
                        moe::FfnPlan* plan) {
  MOE_TRY(ffn_checks(act_dtype, w_dtype, y_dtype, T, H, I, E, k));
  *plan = moe::plan_ffn(T, H, I, E, k, w_dtype);
  if (block_m != plan->block_m)
    return fail(MOE_ERR_INVALID_ARG,
                "block_m %d does not match the FFN tile height %d for this shape "
                "(use moe_ffn_block_m)",
                block_m, plan->block_m);
  if (T == 0) return MOE_OK;
  MOE_NONNULL(sorted_slot);
  MOE_NONNULL(tiles);
  MOE_NONNULL(num_tiles);
  MOE_ALIGNED(tiles, 16);
  return MOE_OK;
}

moe_status up_checks(const void* x, const float* xs, const void* w13, int32_t w_dtype,
                     const float* s13) {
  MOE_NONNULL(x);
  MOE_NONNULL(w13);
  if (w_dtype == MOE_I8 || w_dtype == MOE_I4A8) MOE_NONNULL(xs);
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16) MOE_NONNULL(s13);
  MOE_ALIGNED(x, 16);
  MOE_ALIGNED(w13, 16);
  return MOE_OK;
}

moe_status down_checks(const void* w2, int32_t w_dtype, const float* s2, void* y) {
  MOE_NONNULL(w2);
  MOE_NONNULL(y);
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16) MOE_NONNULL(s2);
  MOE_ALIGNED(w2, 16);
  MOE_ALIGNED(y, 16);
  return MOE_OK;
}

int32_t y_dtype_of(int32_t w_dtype) { return w_dtype == MOE_F32 ? MOE_F32 : MOE_BF16; }
}  // namespace

moe_status moe_ffn_up(const void* x, int32_t act_dtype, const float* xs, const void* w13,
                      int32_t w_dtype, const float* s13, const int32_t* sorted_slot,
                      const int32_t* tiles, const int32_t* num_tiles, int32_t block_m, int64_t T,
                      int32_t H, int32_t I, int32_t E, int32_t k, void* workspace,
                      size_t workspace_bytes, void* stream) {
  moe::FfnPlan plan;
  MOE_TRY(ffn_prologue(act_dtype, w_dtype, y_dtype_of(w_dtype), block_m, T, H, I, E, k, sorted_slot,
                       tiles, num_tiles, workspace, workspace_bytes, &plan));
  if (T == 0) return ok("none (T=0)");
  MOE_TRY(up_checks(x, xs, w13, w_dtype, s13));
  MOE_TRY(check_ws(workspace, workspace_bytes, plan.ws_bytes));
  hipError_t e = moe::launch_ffn_up(plan, x, xs, w13, w_dtype, s13, sorted_slot, tiles, num_tiles, T,
                                    H, I, k, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_ffn_up launch");
  return ok(plan.up_name);
}

moe_status moe_ffn_down(const void* w2, int32_t w_dtype, const float* s2,
                        const int32_t* sorted_slot, const int32_t* tiles,
                        const int32_t* num_tiles, int32_t block_m, const float* topk_w, int64_t T,
                        int32_t H, int32_t I, int32_t E, int32_t k, void* y_sorted, int32_t y_dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  moe::FfnPlan plan;
  // the activation dtype the up launch used (W4A16: bf16, W4A8: int8)
  const int32_t act = w_dtype == MOE_I4 ? MOE_BF16 : (w_dtype == MOE_I4A8 ? MOE_I8 : w_dtype);
  MOE_TRY(ffn_prologue(act, w_dtype, y_dtype, block_m, T, H, I, E, k, sorted_slot, tiles, num_tiles,
                       workspace, workspace_bytes, &plan));
  if (T == 0) return ok("none (T=0)");
  MOE_TRY(down_checks(w2, w_dtype, s2, y_sorted));
  MOE_TRY(check_ws(workspace, workspace_bytes, plan.ws_bytes));
  hipError_t e = moe::launch_ffn_down(plan, w2, w_dtype, s2, sorted_slot, tiles, num_tiles, topk_w, T,
                                      H, I, k, y_sorted, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_ffn_down launch");
  return ok(plan.down_name);
}

moe_status moe_expert_ffn(const void* x, int32_t act_dtype, const float* xs, const void* w13,
                          const void* w2, int32_t w_dtype, const float* s13, const float* s2,
                          const int32_t* sorted_slot, const int32_t* tiles,
                          const int32_t* num_tiles, int32_t block_m, const float* topk_w,
                          int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, void* y_sorted,
                          int32_t y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  moe::FfnPlan plan;
  MOE_TRY(ffn_prologue(act_dtype, w_dtype, y_dtype, block_m, T, H, I, E, k, sorted_slot, tiles,
                       num_tiles, workspace, workspace_bytes, &plan));
  if (T == 0) return ok("none (T=0)");
  MOE_TRY(up_checks(x, xs, w13, w_dtype, s13));
  MOE_TRY(down_checks(w2, w_dtype, s2, y_sorted));
  MOE_TRY(check_ws(workspace, workspace_bytes, plan.ws_bytes));
  hipError_t e = moe::launch_ffn_up(plan, x, xs, w13, w_dtype, s13, sorted_slot, tiles, num_tiles, T,
                                    H, I, k, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn up launch");
  e = moe::launch_ffn_down(plan, w2, w_dtype, s2, sorted_slot, tiles, num_tiles, topk_w, T, H, I, k,
                           y_sorted, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_expert_ffn down launch");
  return ok(std::string(plan.up_name) + "+" + plan.down_name);
}

moe_status moe_combine(const void* y_sorted, int32_t y_dtype, const int32_t* pos,
                       const float* topk_w, int64_t T, int32_t k, int32_t H, void* out,
                       int32_t out_dtype, void* stream) {
  MOE_TRY(check_dims(T, H, moe::kMaxE, k));
  if (!is_act(y_dtype) || !is_act(out_dtype))
    return fail(MOE_ERR_UNSUPPORTED, "combine dtypes must be MOE_F32 or MOE_BF16");
  if (T == 0) return ok("none (T=0)");
  MOE_NONNULL(y_sorted);
  MOE_NONNULL(pos);
  MOE_NONNULL(out);
  MOE_ALIGNED(y_sorted, 16);
  MOE_ALIGNED(out, 16);
  hipError_t e = moe::launch_combine(y_sorted, y_dtype, pos, topk_w, T, k, H, out, out_dtype,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_combine launch");
  return ok(topk_w ? "combine_kernel<weighted>" : "combine_kernel<pre-weighted>");
}

moe_status moe_combine_shared(const void* y_sorted, int32_t y_dtype, const int32_t* pos,
                              const float* topk_w, int64_t T, int32_t k, int32_t H,
                              const void* shared, float shared_factor, const float* bias,
                              void* out, int32_t out_dtype, void* stream) {
  MOE_TRY(check_dims(T, H, moe::kMaxE, k));
  if (!is_act(y_dtype) || !is_act(out_dtype))
    return fail(MOE_ERR_UNSUPPORTED, "combine dtypes must be MOE_F32 or MOE_BF16");
  if (!std::isfinite(shared_factor))
    return fail(MOE_ERR_INVALID_ARG, "shared_factor must be finite");
  if (T == 0) return ok("none (T=0)");
  MOE_NONNULL(y_sorted);
  MOE_NONNULL(pos);
  MOE_NONNULL(out);
  MOE_ALIGNED(y_sorted, 16);
  MOE_ALIGNED(out, 16);
  if (shared) MOE_ALIGNED(shared, 16);
  if (bias) MOE_ALIGNED(bias, 16);
  if (shared && shared != out) {
    // partial overlap would let one thread's write land on another's input
    const size_t bytes = (size_t)T * (size_t)H * (out_dtype == MOE_BF16 ? 2 : 4);
    const char *a = (const char*)shared, *b = (const char*)out;
    if (a < b + bytes && b < a + bytes)
      return fail(MOE_ERR_INVALID_ARG, "shared overlaps out without being out");
  }
  hipError_t e = moe::launch_combine_shared(y_sorted, y_dtype, pos, topk_w, T, k, H, shared,
                                            shared_factor, bias, out, out_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_combine_shared launch");
  return ok(topk_w ? "combine_kernel<weighted,shared+bias>" : "combine_kernel<pre-weighted,shared+bias>");
}

size_t moe_layer_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                int32_t x_dtype, int32_t w_dtype) {
  if (T < 0 || k < 1 || E < 1 || H < 1 || I < 1) return 0;
  const int32_t wgd = E <= 16 ? x_dtype : MOE_BF16;
  return carve_layer(T, H, I, E, k, x_dtype, wgd, w_dtype).total;
}

}  // extern "C"

// ------------------------------------------------ allocation-free layer ---
// moe_layer_noalloc carves its workspace from this file-scope device array
// instead of a caller buffer.  Each GPU the library runs on holds its own
// copy (MOE_NOALLOC_SCRATCH_BYTES) until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// for the symbol): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in noalloc_ptr.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[kMaxDevices];

// The device address of the current device's scratch array.
moe_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "moe_layer_noalloc: device %d beyond the %d it keeps scratch for", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (!noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "moe_layer_noalloc: hipGetSymbolAddress(scratch)");
    if (!p || !al(p, 256)) return fail(MOE_ERR_HIP, "moe_layer_noalloc: scratch address not 256-byte aligned");
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return MOE_OK;
}

}  // namespace

namespace {

// The fused layer behind moe_layer, moe_layer_ex and moe_layer_noalloc
// (opt NULL: plain top-k, no shared term, no bias; noalloc: the workspace is
// the current device's scratch array).
moe_status layer_impl(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                      const float* bias, const void* w13, const void* w2, int32_t w_dtype,
                      const float* s13, const float* s2, int64_t T, int32_t H, int32_t I,
                      int32_t E, int32_t k, int64_t capacity, void* out, int32_t out_dtype,
                      const moe_layer_aux* aux, const moe_layer_options* opt, void* workspace,
                      size_t workspace_bytes, void* stream, bool noalloc = false) {
  const moe_layer_options no_opt{0, 0, nullptr, 1.0f, nullptr};
  const moe_layer_options& o = opt ? *opt : no_opt;
  const bool grouped = o.n_group != 0;
  const bool merge = o.shared != nullptr || o.out_bias != nullptr;
  if (!is_act(x_dtype)) return fail(MOE_ERR_UNSUPPORTED, "x dtype must be MOE_F32 or MOE_BF16");
  if (out_dtype != x_dtype) return fail(MOE_ERR_UNSUPPORTED, "out dtype must equal x dtype");
  int32_t act;
  if (w_dtype == MOE_F32 && x_dtype == MOE_F32)
    act = MOE_F32;
  else if (w_dtype == MOE_BF16 && x_dtype == MOE_BF16)
    act = MOE_BF16;
  else if (w_dtype == MOE_I8 || w_dtype == MOE_I4A8)
    act = MOE_I8;
  else if (w_dtype == MOE_I4 && x_dtype == MOE_BF16)
    act = MOE_BF16;
  else
    return fail(MOE_ERR_UNSUPPORTED,
                "layer dtypes (x %d, w %d) not implemented: f32/f32, bf16/bf16, W8A8 (any x, i8 w), "
                "W4A16 (bf16 x, i4 w) or W4A8 (any x, i4a8 w)",
                x_dtype, w_dtype);
  const int32_t ydt = w_dtype == MOE_F32 ? MOE_F32 : MOE_BF16;
  MOE_TRY(ffn_checks(act, w_dtype, ydt, T, H, I, E, k));
  // the route outputs live in the workspace: validate the rest with aligned
  // stand-ins for them (never dereferenced)
  alignas(16) static int32_t stand_in[4];
  int32_t* const si = stand_in;
  moe::RoutePlan rp;
  MOE_TRY(route_checks(x, x_dtype, wg, wg_dtype, T, H, E, k, si, (float*)si,
                       act == MOE_I8 ? (int8_t*)si : nullptr, act == MOE_I8 ? (float*)si : nullptr, &rp, !grouped));
  if (grouped) {
    const int32_t ng = o.n_group, tg = o.topk_group;
    if (ng < 1 || ng > 64 || E % ng != 0)
      return fail(MOE_ERR_INVALID_ARG, "n_group (%d) must divide E (%d) and be in [1, 64]", ng, E);
    if (tg < 1 || tg > ng)
      return fail(MOE_ERR_INVALID_ARG, "topk_group (%d) must be in [1, n_group=%d]", tg, ng);
    if ((int64_t)k > (int64_t)tg * (E / ng))
      return fail(MOE_ERR_INVALID_ARG, "k (%d) exceeds the %d experts of the kept groups", k, tg * (E / ng));
    if (rp.kind != 2)
      return fail(MOE_ERR_UNSUPPORTED,
                  "group-limited routing needs 16 < E <= 256, E %% 16 == 0, bf16 x and bf16 wg (got E=%d)", E);
  }
  if (!std::isfinite(o.shared_factor)) return fail(MOE_ERR_INVALID_ARG, "shared_factor must be finite");
  if (T == 0) return ok("none (T=0)");
  MOE_NONNULL(w13);
  MOE_NONNULL(w2);
  MOE_NONNULL(out);
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16) {
    MOE_NONNULL(s13);
    MOE_NONNULL(s2);
  }
  MOE_ALIGNED(w13, 16);
  MOE_ALIGNED(w2, 16);
  MOE_ALIGNED(out, 16);
  if (o.shared) {
    MOE_ALIGNED(o.shared, 16);
    if (o.shared != out) {
      const size_t bytes = (size_t)T * (size_t)H * (out_dtype == MOE_BF16 ? 2 : 4);
      const char *sa = (const char*)o.shared, *oa = (const char*)out;
      if (sa < oa + bytes && oa < sa + bytes)
        return fail(MOE_ERR_INVALID_ARG, "shared overlaps out without being out");
    }
  }
  if (o.out_bias) MOE_ALIGNED(o.out_bias, 16);
  const LayerCarve c = carve_layer(T, H, I, E, k, x_dtype, wg_dtype, w_dtype, grouped);
  if (noalloc) {
    if (c.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
      return fail(MOE_ERR_UNSUPPORTED,
                  "moe_layer_noalloc: this shape needs %zu bytes of scratch, above the %zu it holds "
                  "(call moe_layer with a workspace)",
                  c.total, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    MOE_TRY(noalloc_scratch(&workspace));
    workspace_bytes = MOE_NOALLOC_SCRATCH_BYTES;
  }
  MOE_TRY(check_ws(workspace, workspace_bytes, c.total));
  if (aux) {
    for (int i = 0; i < 6; ++i) {
      if (!aux->stage_events[i]) continue;
      const hipError_t q = hipEventQuery((hipEvent_t)aux->stage_events[i]);
      if (q != hipSuccess && q != hipErrorNotReady)
        return fail(MOE_ERR_INVALID_ARG, "moe_layer stage_events[%d]: %s", i, hipGetErrorString(q));
    }
  }

  uint8_t* base = (uint8_t*)workspace;
  auto pick = [&](auto* user, size_t off) {
    typedef decltype(user) P;
    return user ? user : (P)(base + off);
  };
  const moe_layer_aux none{};
  const moe_layer_aux& a = aux ? *aux : none;
  int32_t* ids = pick(a.topk_ids, c.ids);
  float* w = pick(a.topk_w, c.w);
  float* p = a.topk_p;
  int32_t* counts = pick(a.counts, c.counts);
  int32_t* offsets = pick(a.offsets, c.offsets);
  int32_t* sorted_slot = pick(a.sorted_slot, c.sorted_slot);
  int32_t* pos = pick(a.pos, c.pos);
  int32_t* num_dropped = pick(a.num_dropped, c.num_dropped);
  int8_t* xq = act == MOE_I8 ? pick(a.xq, c.xq) : nullptr;
  float* xs = act == MOE_I8 ? pick(a.xs, c.xs) : nullptr;
  int32_t* tiles = (int32_t*)(base + c.tiles);
  int32_t* num_tiles = (int32_t*)(base + c.num_tiles);
  void* y = base + c.y;
  void* scratch = base + c.scratch;
  hipStream_t s = (hipStream_t)stream;
  // the caller's timing events around the steps (already checked)
  auto mark = [&](int i) -> hipError_t {
    return a.stage_events[i] ? hipEventRecord((hipEvent_t)a.stage_events[i], s) : hipSuccess;
  };

  // the fused route + align (moe_route_align) saves a launch but puts every
  // token's top-k on one workgroup: measured ~2 us slower on the GPU at
  // decode than route_topk's four workgroups plus the align launch, so the
  // layer, which runs GPU-bound, keeps the two launches
  const bool fused = false;
  hipError_t e = mark(0);
  if (e != hipSuccess) return hip_fail(e, "moe_layer stage event");
  if (fused) {
    e = moe::launch_route_align_fused(c.rp, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, ids, w, p, xq, xs, scratch,
                                      capacity > 0 ? capacity : 0, c.fp.block_m, c.fp.max_tiles, counts, offsets,
                                      sorted_slot, pos, tiles, num_tiles, num_dropped, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer route+align launch");
    if ((e = mark(1)) != hipSuccess || (e = mark(2)) != hipSuccess) return hip_fail(e, "moe_layer stage event");
  } else {
    // a route step that publishes per-workgroup counts lets one align launch
    // take them instead of histogramming the ids again
    const bool from_route = !grouped && moe::route_publishes_hist(c.rp, T, k);
    int32_t* whist = from_route ? (int32_t*)((uint8_t*)scratch + moe::route_hist_offset(c.rp)) : nullptr;
    if (grouped)
      e = moe::launch_route_grouped(c.rp, x, wg, bias, T, H, E, k, o.n_group, o.topk_group, ids, w, p, xq, xs,
                                    scratch, s);
    else
      e = moe::launch_route(c.rp, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, ids, w, p, xq, xs, scratch, s, whist);
    if (e != hipSuccess) return hip_fail(e, "moe_layer route launch");
    if ((e = mark(1)) != hipSuccess) return hip_fail(e, "moe_layer stage event");
    if (from_route)
      e = moe::launch_align_from_route(ids, whist, moe::route_hist_groups(c.rp, T, k), moe::route_hist_tokens(c.rp, k), T, k, E,
                                       capacity > 0 ? capacity : 0, c.fp.block_m, c.fp.max_tiles, counts, offsets,
                                       sorted_slot, pos, tiles, num_tiles, num_dropped, s);
    else
      e = moe::launch_align(c.ap, ids, T, k, E, capacity > 0 ? capacity : 0, c.fp.block_m, c.fp.max_tiles, counts,
                            offsets, sorted_slot, pos, tiles, num_tiles, num_dropped, scratch, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer align launch");
    if ((e = mark(2)) != hipSuccess) return hip_fail(e, "moe_layer stage event");
  }
  e = moe::launch_ffn_up(c.fp, act == MOE_I8 ? (const void*)xq : x, xs, w13, w_dtype, s13,
                         sorted_slot, tiles, num_tiles, T, H, I, k, scratch, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer ffn up launch");
  if ((e = mark(3)) != hipSuccess) return hip_fail(e, "moe_layer stage event");
  e = moe::launch_ffn_down(c.fp, w2, w_dtype, s2, sorted_slot, tiles, num_tiles, w, T, H, I, k, y,
                           scratch, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer ffn down launch");
  if ((e = mark(4)) != hipSuccess) return hip_fail(e, "moe_layer stage event");
  if (merge)
    e = moe::launch_combine_shared(y, ydt, pos, nullptr, T, k, H, o.shared, o.shared_factor, o.out_bias, out,
                                   out_dtype, s);
  else
    e = moe::launch_combine(y, ydt, pos, nullptr, T, k, H, out, out_dtype, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer combine launch");
  if ((e = mark(5)) != hipSuccess) return hip_fail(e, "moe_layer stage event");
  const bool from_route_d = !grouped && moe::route_publishes_hist(c.rp, T, k);
  return ok(route_name(c.rp) + (grouped ? "<grouped>" : "") + " | " +
            (fused ? std::string("align(fused into route)")
             : from_route_d ? std::string("align(from route counts, one launch)")
             : c.ap.nblocks == 0 ? std::string("align(one block)")
                                 : "align(blocks=" + std::to_string(c.ap.nblocks) + ")") + " | " +
            c.fp.up_name + "+" + c.fp.down_name + "(block_m=" + std::to_string(c.fp.block_m) +
            ") | combine_kernel<pre-weighted" + (merge ? ",shared+bias>" : ">"));
}

}  // namespace

extern "C" {

moe_status moe_layer(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                     const float* bias, const void* w13, const void* w2, int32_t w_dtype,
                     const float* s13, const float* s2, int64_t T, int32_t H, int32_t I,
                     int32_t E, int32_t k, int64_t capacity, void* out, int32_t out_dtype,
                     const moe_layer_aux* aux, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return layer_impl(x, x_dtype, wg, wg_dtype, bias, w13, w2, w_dtype, s13, s2, T, H, I, E, k, capacity, out,
                    out_dtype, aux, nullptr, workspace, workspace_bytes, stream);
}

moe_status moe_layer_ex(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                        const float* bias, const void* w13, const void* w2, int32_t w_dtype,
                        const float* s13, const float* s2, int64_t T, int32_t H, int32_t I,
                        int32_t E, int32_t k, int64_t capacity, void* out, int32_t out_dtype,
                        const moe_layer_aux* aux, const moe_layer_options* options, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return layer_impl(x, x_dtype, wg, wg_dtype, bias, w13, w2, w_dtype, s13, s2, T, H, I, E, k, capacity, out,
                    out_dtype, aux, options, workspace, workspace_bytes, stream);
}

moe_status moe_layer_noalloc(const void* x, int32_t x_dtype, const void* wg, int32_t wg_dtype,
                             const float* bias, const void* w13, const void* w2, int32_t w_dtype,
                             const float* s13, const float* s2, int64_t T, int32_t H, int32_t I,
                             int32_t E, int32_t k, int64_t capacity, void* out, int32_t out_dtype,
                             const moe_layer_aux* aux, void* stream) {
  const moe_status st = layer_impl(x, x_dtype, wg, wg_dtype, bias, w13, w2, w_dtype, s13, s2, T, H, I, E, k,
                                   capacity, out, out_dtype, aux, nullptr, nullptr, 0, stream, true);
  if (st == MOE_OK && T > 0) g_dispatch += " (no-alloc scratch)";
  return st;
}

}  // extern "C"
