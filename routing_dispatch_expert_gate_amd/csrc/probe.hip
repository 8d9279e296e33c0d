// Diagnostic outside the MoE path: the MFMA rate this device sustains, for
// stating a measured peak beside the published one.  Built into its own
// library (libmoe_probe.so), not into libmoe.so, and declared in probe.h.
// Each wave keeps a 128 x 128 block of accumulators (16 fragments of MFMA 32x32x16 bf16) and runs the MFMAs from
// registers only: no memory traffic, no LDS, no barriers.  The operands are
// small integers, so every sum is exact; the result is written so the loop
// is not removed.
#include "moe_internal.h"
#include "probe.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void mfma_rate_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  u32x4 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // bf16 1.0 (0x3F80) or 0 in each half, by lane
    const uint32_t v = (lane + i) & 1 ? 0x3F803F80u : 0u;
    a[i] = u32x4{v, v, v, v};
    b[i] = u32x4{v, 0u, v, 0u};
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                            __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

}  // namespace moe

extern "C" int moe_probe_mfma_rate(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out) return -1;
  moe::mfma_rate_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(out, iters);
  return (int)hipGetLastError();
}
