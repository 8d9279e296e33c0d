// Internal declarations shared by the HIP kernels and the C-ABI layer.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA bf16/int8, 160 KiB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bit pattern, round to nearest even: gfx950's
// v_cvt_pk_bf16_f32 (one instruction for two values)
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_hw r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp): the
// result is rounded to bf16 or re-quantised to int8 afterwards
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// 8 consecutive values <-> fp32 registers (16-byte aligned rows)
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

// ---------------------------------------------------- per-token int8 codes
// Code of x at scale s: round-half-even(x / s) clamped to [-128, 127], equal
// to what the correctly rounded quotient gives.  rs = 1/s, correctly rounded,
// once per row.  With |x| <= 127 s (s is a row's absmax / 127), x * rs is
// within 2^-15 of the correctly rounded quotient, so the two round to the
// same integer unless x * rs lies within 2^-14 of a half-integer (or is not
// finite): only those rare elements take the division.
__device__ __forceinline__ int quant_code(float x, float s, float rs) {
  const float y = x * rs;
  float q = rintf(y);
  if (!(fabsf(fabsf(y - q) - 0.5f) >= 0x1p-14f) || !(fabsf(y) <= 128.f)) q = rintf(x / s);
  return (int)fminf(fmaxf(q, -128.f), 127.f);
}

// ------------------------------------------------------------- wave utils
// 64-lane reductions without LDS round trips: DPP inside each row of 16 lanes
// (two butterfly steps inside quads, then rotations by 4 and 8 lanes, after
// which lanes 0, 16, 32 and 48 hold their row's result), then four readlanes.
// The result is wave-uniform and the same on every lane; the sum's
// association order is fixed, so it is deterministic.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}
// The value of lane l ^ 16 (l ^ 32): gfx950's row-swap permutes exchange
// odd and even 16-lane rows (the two 32-lane halves) of their two operands in
// the VALU, without a trip through the LDS crossbar.  Given the same register
// twice, the half that moved holds the partner lane's value.
__device__ __forceinline__ float lane_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                  false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                  false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:4, row_ror:8
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x124>(v);
  return v + dpp_f32<0x128>(v);
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x124>(v));
  return fmaxf(v, dpp_f32<0x128>(v));
}
// inclusive prefix sum over the 64 lanes (Kogge-Stone by DPP row shifts
// inside rows, then the row totals carried by row broadcasts); lanes whose
// DPP source lies outside the row keep the old value 0
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ int dpp0_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp0_i32<0x111>(v);          // row_shr:1
  v += dpp0_i32<0x112>(v);          // row_shr:2
  v += dpp0_i32<0x114>(v);          // row_shr:4
  v += dpp0_i32<0x118>(v);          // row_shr:8
  v += dpp0_i32<0x142, 0xA>(v);     // row_bcast:15 into rows 1 and 3
  v += dpp0_i32<0x143, 0xC>(v);     // row_bcast:31 into rows 2 and 3
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

// ------------------------------------------- direct-to-LDS copy pipeline
// Tiles are copied from global memory straight into LDS by
// __builtin_amdgcn_global_load_lds (16 bytes per lane, lane i landing at
// byte 16*i of the instruction's 1 KiB LDS block); each wave waits for its own
// copies with an exact vmcnt and a barrier publishes them to the workgroup.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// LDS row swizzles: chunk c (16 bytes) of row r is stored at c ^ sw(r), so
// that sixteen consecutive rows read at one chunk fall on sixteen distinct
// 16-byte slots of a 256-byte bank row, and any eight consecutive rows on
// eight distinct slots of a 128-byte one.
//  64-byte rows (4 chunks): period 32;  128-byte rows (8 chunks): period 16.
template <int ROWB>
__device__ __forceinline__ int swr(int r) {
  if constexpr (ROWB == 64) return ((r >> 1) ^ (r >> 3)) & 3;
  return ((r >> 1) ^ ((r & 1) << 2)) & 7;
}

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// wait until at most m*L of this wave's vector-memory ops are outstanding,
// for a runtime m in [0, MMAX]
template <int L, int MMAX>
__device__ __forceinline__ void wait_vm_stages(int m) {
  if constexpr (MMAX > 0) {
    if (m >= MMAX) {
      wait_vmcnt<MMAX * L>();
      return;
    }
    wait_vm_stages<L, MMAX - 1>(m);
  } else {
    wait_vmcnt<0>();
  }
}
// the same for a runtime per-stage count l in [0, LMAX] (wave-uniform)
template <int LMAX, int MMAX>
__device__ __forceinline__ void wait_vm_dyn(int l, int m) {
  if constexpr (LMAX > 0) {
    if (l == LMAX) {
      wait_vm_stages<LMAX, MMAX>(m);
      return;
    }
    wait_vm_dyn<LMAX - 1, MMAX>(l, m);
  } else {
    wait_vmcnt<0>();
  }
}
// All of this wave's LDS reads have returned, then the workgroup barrier.
// The memory clobber keeps every LDS access on its side of the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------- launchers
// route.hip
struct RoutePlan {
  int kind;      // 0 = fused FMA (E <= 16), 2 = MFMA logits + top-k (E > 16),
                 // 3 = fused MFMA logits + top-k (E <= 64, large batches)
  int bt;        // tokens per workgroup
  int ks;        // K splits (kind 2) or parts of H (kind 3)
  int nw;        // waves per workgroup (kind 0)
  size_t ws_bytes;
  int be;        // experts per workgroup (kind 2)
};
// fused_ok = false: never kind 3 (the group-limited router runs on kind 2)
RoutePlan plan_route(int64_t T, int H, int E, int k, int x_dtype, int wg_dtype, bool fused_ok = true);
// whist (may be NULL): where the route step publishes each workgroup's
// per-expert selection counts, [route_hist_groups(p, T)][E] int32, for
// launch_align_from_route (kinds 0 and 3: the route workgroups; kind 2: its
// top-k workgroups).  Kind 2 also uses ws for its partial logits, so whist
// must start at ws + route_hist_offset(p) there.
hipError_t launch_route(const RoutePlan& p, const void* x, int x_dtype, const void* wg, int wg_dtype,
                        const float* bias, int64_t T, int H, int E, int k, int32_t* ids, float* w,
                        float* prob, int8_t* xq, float* xs, void* ws, hipStream_t s, int32_t* whist = nullptr);
// whether the route step publishes per-workgroup counts for this batch (at
// least kAlignFromRouteSlots slots)
constexpr int64_t kAlignFromRouteSlots = 4096;
bool route_publishes_hist(const RoutePlan& p, int64_t T, int k);
// tokens per publishing workgroup (tg), the number of such workgroups (each
// over tokens [g tg, (g + 1) tg)), where whist starts in the route workspace,
// and the route workspace bytes including whist (0 when nothing is published)
int route_hist_tokens(const RoutePlan& p, int k);
int64_t route_hist_groups(const RoutePlan& p, int64_t T, int k);
size_t route_hist_offset(const RoutePlan& p);
size_t route_hist_bytes(const RoutePlan& p, int64_t T, int k, int E);
// route and align in one launch where one workgroup can take every token
// (route_align_fusable): the align outputs as in launch_align
bool route_align_fusable(const RoutePlan& p, int64_t T, int k);
hipError_t launch_route_align_fused(const RoutePlan& p, const void* x, int x_dtype, const void* wg, int wg_dtype,
                                    const float* bias, int64_t T, int H, int E, int k, int32_t* ids, float* w,
                                    float* prob, int8_t* xq, float* xs, void* ws, int64_t cap, int block_m,
                                    int64_t max_tiles, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                                    int32_t* pos, int32_t* tiles, int32_t* num_tiles, int32_t* num_dropped,
                                    hipStream_t s);
// group-limited variant (kind 2 plans only): n_group contiguous groups,
// the topk_group best by their two largest probabilities
hipError_t launch_route_grouped(const RoutePlan& p, const void* x, const void* wg, const float* bias,
                                int64_t T, int H, int E, int k, int n_group, int topk_group,
                                int32_t* ids, float* w, float* prob, int8_t* xq, float* xs, void* ws,
                                hipStream_t s);

// align.hip
struct AlignPlan {
  int slots_per_block;
  int nblocks;
  size_t ws_bytes;
};
AlignPlan plan_align(int64_t T, int k, int E);
hipError_t launch_align(const AlignPlan& p, const int32_t* ids, int64_t T, int k, int E, int64_t cap,
                        int block_m, int64_t max_tiles, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_slot, int32_t* pos, int32_t* tiles, int32_t* num_tiles,
                        int32_t* num_dropped, void* ws, hipStream_t s);
// The same outputs from the route step's published counts: whist[g][E] for
// the ng route workgroups of tg tokens each (g over tokens [g tg, ...)); one
// launch, no workspace.
hipError_t launch_align_from_route(const int32_t* ids, const int32_t* whist, int64_t ng, int tg, int64_t T, int k,
                                   int E, int64_t cap, int block_m, int64_t max_tiles, int32_t* counts,
                                   int32_t* offsets, int32_t* sorted_slot, int32_t* pos, int32_t* tiles,
                                   int32_t* num_tiles, int32_t* num_dropped, hipStream_t s);

// combine.hip
hipError_t launch_combine(const void* y, int y_dtype, const int32_t* pos, const float* w, int64_t T,
                          int k, int H, void* out, int out_dtype, hipStream_t s);
// the same plus factor * shared[t] (out dtype, may be null or equal to out)
// and bias[h] (fp32, may be null), added to the fp32 sum before the write
hipError_t launch_combine_shared(const void* y, int y_dtype, const int32_t* pos, const float* w,
                                 int64_t T, int k, int H, const void* shared, float factor,
                                 const float* bias, void* out, int out_dtype, hipStream_t s);

// ffn_*.hip
struct FfnPlan {
  int block_m;        // row-tile height the align step must use
  int64_t max_tiles;  // host-side upper bound on the number of row tiles
  size_t ws_bytes;    // h (+ row maxima, codes and scales for W8A8)
  int up_var, down_var;
  char up_name[64];
  char down_name[64];
};
FfnPlan plan_ffn(int64_t T, int H, int I, int E, int k, int w_dtype);
// The FFN workspace carries h (and, for W8A8, row maxima, codes and scales)
// from the up launch to the down launch.
hipError_t launch_ffn_up(const FfnPlan& p, const void* x, const float* xs, const void* w13,
                         int w_dtype, const float* s13, const int32_t* sorted_slot,
                         const int32_t* tiles, const int32_t* num_tiles, int64_t T, int H, int I,
                         int k, void* ws, hipStream_t s);
hipError_t launch_ffn_down(const FfnPlan& p, const void* w2, int w_dtype, const float* s2,
                           const int32_t* sorted_slot, const int32_t* tiles,
                           const int32_t* num_tiles, const float* topk_w, int64_t T, int H, int I,
                           int k, void* y, void* ws, hipStream_t s);

int64_t align_max_tiles(int64_t T, int k, int E, int block_m);

// int4 codes [n] (one per int8, in [-8, 7]) -> packed [n / 2], n % 16 == 0
hipError_t launch_pack_i4(const int8_t* codes, int64_t n, uint8_t* packed, hipStream_t s);

}  // namespace moe
