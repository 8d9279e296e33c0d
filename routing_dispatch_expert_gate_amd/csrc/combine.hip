// Combine (moe_sum): out[t] = sum over token t's kept slots of w * Y[pos].
//
// The MoE FlashAttention page (framerc.cn, step 5 of the MoE layer and its
// second fusion) merges the expert outputs weighted by the route weights,
// accumulating on chip; the LightOP page, section 3.2 (MoE Sum), reads and
// writes with 128-bit vectors and spreads one token over several blocks.
//
// One thread owns 8 consecutive output values of one token: it loads the k
// slot positions (and weights), issues all k independent row loads (16 bytes
// for bf16 Y), accumulates in fp32 registers in slot order, and writes once.
// k is rounded up to a compile-time KT (2, 4 or 8; the extra slots are
// masked) so the loads and sums unroll exactly.  Dropped slots (pos < 0) add
// nothing, so a fully dropped token gets 0.  When H is a multiple of 512 a
// wave's 64 threads share one token, so the token index is made
// wave-uniform and its positions and weights come through scalar loads, off
// the vector memory path the rows use.  (Measured, T = 4096, H = 4096, bf16:
// k = 8 57 -> 50 us with the scalar loads; k = 2 19.3 -> 16.3 us with 8
// values per thread instead of 16.)
//
// The EXTRA variant (LightOP page, section 3.2: MoE Sum fuses the shared
// expert's factor and a bias add) adds factor * S[t] and b to the fp32 sum
// before the single write: S and b are read once, in the same 16-byte chunks
// as the output, so the fused form costs T*H*sizeof(S) + H*4 bytes more and
// saves a separate elementwise pass over out.  Each thread reads its chunk of
// S before writing the same chunk of out, so out may be S itself.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename YT, typename OT, bool WEIGHTED, int KT, bool EXTRA, bool UNIF>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                     const int32_t* __restrict__ pos,
                                                     const float* __restrict__ w, int64_t T, int k,
                                                     int H, OT* out, const OT* shared, float factor,
                                                     const float* __restrict__ bias) {
  constexpr int VPT = 8;
  constexpr int NC = VPT / 8;   // 8-value chunks per thread
  const int cpr = H / VPT;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= T * cpr) return;
  int64_t t = g / cpr;
  // UNIF: cpr is a multiple of 64, so the wave's threads share t
  if constexpr (UNIF) t = __builtin_amdgcn_readfirstlane((int)t);
  const int c = (int)(g - t * cpr);
  int p[KT];
  float wt[KT];
#pragma unroll
  for (int j = 0; j < KT; ++j) {
    p[j] = j < k ? pos[t * k + j] : -1;
    wt[j] = (WEIGHTED && j < k) ? w[t * k + j] : 1.f;
  }
  float v[KT][NC][8];
#pragma unroll
  for (int j = 0; j < KT; ++j)
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      if (p[j] >= 0) {
        load8(y + (int64_t)p[j] * H + c * VPT + q * 8, v[j][q]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][q][i] = 0.f;
      }
    }
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KT; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = WEIGHTED ? fmaf(wt[j], v[j][q][i], acc[i]) : acc[i] + v[j][q][i];
    if constexpr (EXTRA) {
      // routed sum, then + factor * S, then + b (each rounded in fp32)
      if (shared) {
        float sv[8];
        load8(shared + t * H + c * VPT + q * 8, sv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(factor, sv[i], acc[i]);
      }
      if (bias) {
        float bv[8];
        load8(bias + c * VPT + q * 8, bv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += bv[i];
      }
    }
    store8(out + t * H + c * VPT + q * 8, acc);
  }
}

struct Extra {
  const void* shared;  // [T, H] in the output dtype, or null
  float factor;
  const float* bias;   // [H], or null
};

template <typename YT, typename OT, int KT, bool EXTRA, bool UNIF>
void launch_u(const void* y, const int32_t* pos, const float* w, int64_t T, int k, int H, void* out,
              const Extra& x, hipStream_t s) {
  const int64_t work = T * (H / 8);
  const dim3 grid((unsigned)((work + 255) / 256));
  if (w)
    combine_kernel<YT, OT, true, KT, EXTRA, UNIF><<<grid, 256, 0, s>>>(
        (const YT*)y, pos, w, T, k, H, (OT*)out, (const OT*)x.shared, x.factor, x.bias);
  else
    combine_kernel<YT, OT, false, KT, EXTRA, UNIF><<<grid, 256, 0, s>>>(
        (const YT*)y, pos, w, T, k, H, (OT*)out, (const OT*)x.shared, x.factor, x.bias);
}

template <typename YT, typename OT, int KT, bool EXTRA>
hipError_t launch_k(const void* y, const int32_t* pos, const float* w, int64_t T, int k, int H,
                    void* out, const Extra& x, hipStream_t s) {
  if (H % 512 == 0)
    launch_u<YT, OT, KT, EXTRA, true>(y, pos, w, T, k, H, out, x, s);
  else
    launch_u<YT, OT, KT, EXTRA, false>(y, pos, w, T, k, H, out, x, s);
  return hipGetLastError();
}

template <typename YT, typename OT, bool EXTRA>
hipError_t launch_t(const void* y, const int32_t* pos, const float* w, int64_t T, int k, int H,
                    void* out, const Extra& x, hipStream_t s) {
  if (k <= 2) return launch_k<YT, OT, 2, EXTRA>(y, pos, w, T, k, H, out, x, s);
  if (k <= 4) return launch_k<YT, OT, 4, EXTRA>(y, pos, w, T, k, H, out, x, s);
  return launch_k<YT, OT, 8, EXTRA>(y, pos, w, T, k, H, out, x, s);
}

template <bool EXTRA>
hipError_t launch_dt(const void* y, int y_dtype, const int32_t* pos, const float* w, int64_t T,
                     int k, int H, void* out, int out_dtype, const Extra& x, hipStream_t s) {
  const bool yb = y_dtype == 1, ob = out_dtype == 1;
  if (yb && ob) return launch_t<uint16_t, uint16_t, EXTRA>(y, pos, w, T, k, H, out, x, s);
  if (yb && !ob) return launch_t<uint16_t, float, EXTRA>(y, pos, w, T, k, H, out, x, s);
  if (!yb && ob) return launch_t<float, uint16_t, EXTRA>(y, pos, w, T, k, H, out, x, s);
  return launch_t<float, float, EXTRA>(y, pos, w, T, k, H, out, x, s);
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dtype, const int32_t* pos, const float* w,
                          int64_t T, int k, int H, void* out, int out_dtype, hipStream_t s) {
  return launch_dt<false>(y, y_dtype, pos, w, T, k, H, out, out_dtype, Extra{nullptr, 0.f, nullptr}, s);
}

hipError_t launch_combine_shared(const void* y, int y_dtype, const int32_t* pos, const float* w,
                                 int64_t T, int k, int H, const void* shared, float factor,
                                 const float* bias, void* out, int out_dtype, hipStream_t s) {
  return launch_dt<true>(y, y_dtype, pos, w, T, k, H, out, out_dtype, Extra{shared, factor, bias}, s);
}

}  // namespace moe
