// Combine (moe_sum): out[t] = sum over token t's kept slots of w * Y[pos].
//
// The MoE FlashAttention page (framerc.cn, step 5 of the MoE layer and its
// second fusion) merges the expert outputs weighted by the route weights,
// accumulating on chip; the LightOP page, section 3.2 (MoE Sum), reads and
// writes with 128-bit vectors and spreads one token over several blocks.
//
// One thread owns 8 consecutive output values of one token: it loads the k
// slot positions (and weights), issues up to k independent 16-byte row loads,
// accumulates in fp32 registers in slot order, and writes once.  A 4096-wide
// token is spread over two 256-thread blocks.  Dropped slots (pos < 0) add
// nothing, so a fully dropped token gets 0.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename YT, typename OT, bool WEIGHTED>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                     const int32_t* __restrict__ pos,
                                                     const float* __restrict__ w, int64_t T, int k,
                                                     int H, OT* __restrict__ out) {
  const int cpr = H >> 3;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= T * cpr) return;
  const int64_t t = g / cpr;
  const int c = (int)(g - t * cpr);
  int p[kMaxK];
  float wt[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    p[j] = j < k ? pos[t * k + j] : -1;
    wt[j] = (WEIGHTED && j < k) ? w[t * k + j] : 1.f;
  }
  float v[kMaxK][8];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (p[j] >= 0) {
      load8(y + (int64_t)p[j] * H + c * 8, v[j]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
    }
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = WEIGHTED ? fmaf(wt[j], v[j][i], acc[i]) : acc[i] + v[j][i];
  store8(out + t * H + c * 8, acc);
}

template <typename YT, typename OT>
hipError_t launch_t(const void* y, const int32_t* pos, const float* w, int64_t T, int k, int H,
                    void* out, hipStream_t s) {
  const int64_t work = T * (H / 8);
  const dim3 grid((unsigned)((work + 255) / 256));
  if (w)
    combine_kernel<YT, OT, true><<<grid, 256, 0, s>>>((const YT*)y, pos, w, T, k, H, (OT*)out);
  else
    combine_kernel<YT, OT, false><<<grid, 256, 0, s>>>((const YT*)y, pos, w, T, k, H, (OT*)out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dtype, const int32_t* pos, const float* w,
                          int64_t T, int k, int H, void* out, int out_dtype, hipStream_t s) {
  const bool yb = y_dtype == 1, ob = out_dtype == 1;
  if (yb && ob) return launch_t<uint16_t, uint16_t>(y, pos, w, T, k, H, out, s);
  if (yb && !ob) return launch_t<uint16_t, float>(y, pos, w, T, k, H, out, s);
  if (!yb && ob) return launch_t<float, uint16_t>(y, pos, w, T, k, H, out, s);
  return launch_t<float, float>(y, pos, w, T, k, H, out, s);
}

}  // namespace moe
