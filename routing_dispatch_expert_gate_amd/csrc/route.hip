// Router: gate logits, softmax, top-k, renormalisation, optional per-token
// int8 quantisation of x.
//
// What is computed follows the MoE Router page (2048ai.net, section on the
// router as a small network): logits = x Wg^T, softmax over the experts, the
// k largest probabilities, divided by their sum.  The kernel techniques follow
// the LightOP page, section 3.1 (gate, softmax and top-k fused in one kernel,
// shuffle broadcast of results, designated lanes writing coalesced output,
// exponentials only where needed, unrolled argmax with erase of the winner).
// The quantisation is the per-token int8 rule of the LightOP page, section 4.1.
//
// Three variants, picked on the host by shape (never silently):
//   kind 0  E <= 16: fp32 FMA.  Each wave keeps its slice of Wg (8 values of
//           H per lane, all experts) in registers
//           and re-uses it for 16 tokens; per-token partial logits are reduced
//           across the 64 lanes with a multi-value butterfly (E values in
//           log2(64) steps, halving the vector each step), then across waves
//           through LDS.  Logits never leave the chip.
//   kind 1  16 < E <= 64, bf16: MFMA 16x16x32 bf16 over a 64-expert slice,
//           x tiles staged in LDS, logits kept in LDS, top-k in the same kernel.
//   kind 2  64 < E <= 256, bf16: the same MFMA tile computes a [BT x 64]
//           logits block per workgroup (experts split over workgroups so each
//           CU streams a quarter of Wg instead of all of it, and K optionally
//           split for decode-sized T), partial logits go to the workspace, and
//           a second kernel sums the K splits in a fixed order and runs the
//           wave top-k.  Deterministic: no floating-point atomics.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// --------------------------------------------------------------- top-k ----
// One wave selects the top-k of one token.  Lane l owns the logits of experts
// l + 64*j (j < 4, -inf beyond E).  Lanes 0..k-1 write selection i = lane.
__device__ void wave_topk_store(float v[4], int E, int k, int64_t t, int32_t* __restrict__ ids,
                                float* __restrict__ w, float* __restrict__ prob) {
  const int lane = threadIdx.x & 63;
  float m = wave_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  float s = 0.f;
  if (prob) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < E) s += expf(v[j] - m);
    s = wave_sum(s);
  }
  int my_id = 0;
  float my_l = -INFINITY;
  for (int i = 0; i < k; ++i) {
    float bv = v[0];
    int bi = lane;
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (v[j] > bv) {
        bv = v[j];
        bi = lane + 64 * j;
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == i) {
      my_id = bi;
      my_l = bv;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (bi == lane + 64 * j) v[j] = -INFINITY;
  }
  const float ex = lane < k ? expf(my_l - m) : 0.f;
  const float se = wave_sum(ex);
  if (lane < k) {
    ids[t * k + lane] = my_id;
    w[t * k + lane] = ex / se;
    if (prob) prob[t * k + lane] = ex / s;
  }
}

// ------------------------------------------------------- per-token quant --
// codes of 8 values with scale s: round-half-even(x / s) clamped to [-128, 127]
__device__ __forceinline__ uint2 quant8(const float (&v)[8], float s) {
  uint32_t b[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = rintf(v[i] / s);
    q = fminf(fmaxf(q, -128.f), 127.f);
    b[i >> 2] |= (uint32_t)((int)q & 0xFF) << (8 * (i & 3));
  }
  return make_uint2(b[0], b[1]);
}

__device__ __forceinline__ float row_scale(float absmax) {
  return absmax == 0.f ? 1.f : absmax / 127.f;
}

// One wave quantises one row of H values.
template <typename XT>
__device__ void wave_quant_row(const XT* __restrict__ xrow, int H, int8_t* __restrict__ qrow,
                               float* __restrict__ s_out) {
  const int lane = threadIdx.x & 63;
  float am = 0.f;
  for (int h = lane * 8; h < H; h += 512) {
    float v[8];
    load8(xrow + h, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
  }
  const float s = row_scale(wave_max(am));
  for (int h = lane * 8; h < H; h += 512) {
    float v[8];
    load8(xrow + h, v);
    *reinterpret_cast<uint2*>(qrow + h) = quant8(v, s);
  }
  if (lane == 0) *s_out = s;
}

// ------------------------------------------------------------ kind 0 -----
// Multi-value butterfly: lane l ends with the 64-lane sum of value
// index l / (64 / EP) in a[0].
template <int EP>
__device__ __forceinline__ void multi_reduce(float (&a)[EP], int lane) {
  int o = 32;
#pragma unroll
  for (int n = EP; n > 1; n >>= 1, o >>= 1) {
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float send = up ? a[i] : a[i + n / 2];
      const float keep = up ? a[i + n / 2] : a[i];
      a[i] = keep + __shfl_xor(send, o, kWave);
    }
  }
  for (; o > 0; o >>= 1) a[0] += __shfl_xor(a[0], o, kWave);
}

constexpr int kFmaTB = 16;   // tokens per workgroup

template <int EP, int NCH, typename XT, typename WT, bool QUANT>
__global__ __launch_bounds__(EP <= 8 ? 1024 : 512) void route_fma_kernel(
    const XT* __restrict__ x, const WT* __restrict__ wg, const float* __restrict__ bias, int64_t T,
    int H, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    float* __restrict__ prob, int8_t* __restrict__ xq, float* __restrict__ xs) {
  __shared__ float part[16][kFmaTB][EP];
  __shared__ float amax_s[16][kFmaTB];
  const int nw = blockDim.x >> 6;
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;

  // this lane's slice of Wg: NCH chunks of 8 consecutive h, for every expert
  float wr[NCH][EP][8];
  int h0[NCH];
  bool hv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    h0[c] = ((wv * NCH + c) * 64 + lane) * 8;
    hv[c] = h0[c] < H;
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (hv[c] && e < E) load8(wg + (size_t)e * H + h0[c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) wr[c][e][i] = v[i];
    }
  }

  const int64_t t0 = (int64_t)blockIdx.x * kFmaTB;
  const int ntok = (int)((T - t0) < kFmaTB ? (T - t0) : kFmaTB);
  for (int tt = 0; tt < ntok; ++tt) {
    const XT* xrow = x + (t0 + tt) * H;
    float acc[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = 0.f;
    float am = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (!hv[c]) continue;
      float v[8];
      load8(xrow + h0[c], v);
#pragma unroll
      for (int e = 0; e < EP; ++e)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[e] = fmaf(v[i], wr[c][e][i], acc[e]);
      if (QUANT)
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
    }
    multi_reduce<EP>(acc, lane);
    if ((lane & (64 / EP - 1)) == 0) part[wv][tt][lane / (64 / EP)] = acc[0];
    if (QUANT) {
      am = wave_max(am);
      if (lane == 0) amax_s[wv][tt] = am;
    }
  }
  __syncthreads();

  for (int tt = wv; tt < ntok; tt += nw) {
    float v[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (lane < E) {
      float s = 0.f;
      for (int q = 0; q < nw; ++q) s += part[q][tt][lane];
      if (bias) s += bias[lane];
      v[0] = s;
    }
    wave_topk_store(v, E, k, t0 + tt, ids, w, prob);
  }

  if (QUANT) {
    for (int tt = 0; tt < ntok; ++tt) {
      float am = 0.f;
      for (int q = 0; q < nw; ++q) am = fmaxf(am, amax_s[q][tt]);
      const float s = row_scale(am);
      const int64_t t = t0 + tt;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (!hv[c]) continue;
        float v[8];
        load8(x + t * H + h0[c], v);
        *reinterpret_cast<uint2*>(xq + t * H + h0[c]) = quant8(v, s);
      }
      if (threadIdx.x == 0) xs[t] = s;
    }
  }
}

// ------------------------------------------------------- kinds 1 and 2 ----
// MFMA 16x16x32 bf16: lane l supplies A[m = l%16][k = 8*(l/16) .. +8] and
// B[k = 8*(l/16) .. +8][n = l%16]; it receives D[m = 4*(l/16) + i][n = l%16].
// Rows of the LDS x tile are 64 bf16 (8 chunks of 16 B); chunk c of row r is
// stored at chunk c ^ (r & 7) so the 16-lane column reads are conflict-free.
template <int BT, bool FUSED, bool QUANT>
__global__ __launch_bounds__(256) void route_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, const float* __restrict__ bias,
    int64_t T, int H, int E, int k, int kchunk, float* __restrict__ part,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ prob,
    int8_t* __restrict__ xq, float* __restrict__ xs) {
  constexpr int MF = BT / 16;
  constexpr int APASS = (BT * 8 + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BT * 64];
  __shared__ float Ls[FUSED ? BT : 1][FUSED ? 65 : 1];
  __shared__ float rowmax_s[BT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int eb = blockIdx.y * 64 + wv * 16 + (lane & 15);
  const bool e_ok = eb < E;
  const uint16_t* brow = wg + (size_t)(e_ok ? eb : 0) * H + (lane >> 4) * 8;
  const int kbeg = blockIdx.z * kchunk;
  const int nk = kchunk / 64;

  const uint16_t* arow[APASS];
  int alds[APASS];
  bool aval[APASS];
#pragma unroll
  for (int p = 0; p < APASS; ++p) {
    const int idx = tid + 256 * p;
    const int r = idx >> 3, c = idx & 7;
    aval[p] = idx < BT * 8 && t0 + r < T;
    arow[p] = x + (aval[p] ? (t0 + r) * H : 0) + c * 8;
    alds[p] = r * 64 + ((c ^ (r & 7)) * 8);
  }

  f32x4 acc[MF];
#pragma unroll
  for (int i = 0; i < MF; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float am[APASS];
  uint4 areg[APASS];
#pragma unroll
  for (int p = 0; p < APASS; ++p) am[p] = 0.f;

  auto load_a = [&](int kk) {
#pragma unroll
    for (int p = 0; p < APASS; ++p) {
      areg[p] = aval[p] ? *reinterpret_cast<const uint4*>(arow[p] + kk) : make_uint4(0, 0, 0, 0);
      if (QUANT) {
        const uint32_t u[4] = {areg[p].x, areg[p].y, areg[p].z, areg[p].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          am[p] = fmaxf(am[p], fabsf(__uint_as_float(u[i] << 16)));
          am[p] = fmaxf(am[p], fabsf(__uint_as_float(u[i] & 0xFFFF0000u)));
        }
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int p = 0; p < APASS; ++p)
      if (tid + 256 * p < BT * 8) *reinterpret_cast<uint4*>(&As[buf][alds[p]]) = areg[p];
  };
  const bf16x8 bzero = {};
  auto load_b = [&](int kk, bf16x8& b0, bf16x8& b1) {
    b0 = e_ok ? *reinterpret_cast<const bf16x8*>(brow + kk) : bzero;
    b1 = e_ok ? *reinterpret_cast<const bf16x8*>(brow + kk + 32) : bzero;
  };

  bf16x8 b0, b1;
  load_a(kbeg);
  load_b(kbeg, b0, b1);
  store_a(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bf16x8 cb0 = b0, cb1 = b1;
    if (kt + 1 < nk) {
      load_a(kbeg + (kt + 1) * 64);
      load_b(kbeg + (kt + 1) * 64, b0, b1);
    }
#pragma unroll
    for (int mi = 0; mi < MF; ++mi) {
      const int r = mi * 16 + (lane & 15);
      const int c0 = lane >> 4;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&As[cur][r * 64 + ((c0 ^ (r & 7)) * 8)]);
      const bf16x8 a1 =
          *reinterpret_cast<const bf16x8*>(&As[cur][r * 64 + (((c0 + 4) ^ (r & 7)) * 8)]);
      acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, cb0, acc[mi], 0, 0, 0);
      acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, cb1, acc[mi], 0, 0, 0);
    }
    if (kt + 1 < nk) store_a(cur ^ 1);
    __syncthreads();
  }

  if (!FUSED) {
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + mi * 16 + 4 * (lane >> 4) + i;
        if (t < T && e_ok) part[((size_t)blockIdx.z * T + t) * E + eb] = acc[mi][i];
      }
    return;
  }

  // fused: logits of this block's tokens stay in LDS
#pragma unroll
  for (int mi = 0; mi < MF; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      Ls[mi * 16 + 4 * (lane >> 4) + i][wv * 16 + (lane & 15)] = acc[mi][i];
  if (QUANT) {
#pragma unroll
    for (int p = 0; p < APASS; ++p) {
      float v = am[p];
      v = fmaxf(v, __shfl_xor(v, 1, kWave));
      v = fmaxf(v, __shfl_xor(v, 2, kWave));
      v = fmaxf(v, __shfl_xor(v, 4, kWave));
      const int idx = tid + 256 * p;
      if ((idx & 7) == 0 && idx < BT * 8) rowmax_s[idx >> 3] = v;
    }
  }
  __syncthreads();
  for (int tt = wv; tt < BT; tt += 4) {
    if (t0 + tt >= T) break;
    float v[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (lane < E) v[0] = Ls[tt][lane] + (bias ? bias[lane] : 0.f);
    wave_topk_store(v, E, k, t0 + tt, ids, w, prob);
  }
  if (QUANT) {
    const int cpr = H / 8;   // 8-value chunks per row
    for (int q = tid; q < BT * cpr; q += 256) {
      const int rr = q / cpr, c = q - rr * cpr;
      const int64_t t = t0 + rr;
      if (t >= T) break;
      float v[8];
      load8(x + t * H + c * 8, v);
      *reinterpret_cast<uint2*>(xq + t * H + c * 8) = quant8(v, row_scale(rowmax_s[rr]));
    }
    if (tid < BT && t0 + tid < T) xs[t0 + tid] = row_scale(rowmax_s[tid]);
  }
}

template <bool QUANT>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ part, int ks, const float* __restrict__ bias, int64_t T, int E, int k,
    int H, const uint16_t* __restrict__ x, int32_t* __restrict__ ids, float* __restrict__ w,
    float* __restrict__ prob, int8_t* __restrict__ xq, float* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      float s = 0.f;
      for (int z = 0; z < ks; ++z) s += part[((size_t)z * T + t) * E + e];
      v[j] = s + (bias ? bias[e] : 0.f);
    } else {
      v[j] = -INFINITY;
    }
  }
  wave_topk_store(v, E, k, t, ids, w, prob);
  if (QUANT) wave_quant_row(x + t * H, H, xq + t * H, xs + t);
}

template <int EP, int NCH, typename XT, typename WT>
hipError_t launch_fma(const RoutePlan& p, const void* x, const void* wg, const float* bias,
                      int64_t T, int H, int E, int k, int32_t* ids, float* w, float* prob,
                      int8_t* xq, float* xs, hipStream_t s) {
  const dim3 grid((unsigned)((T + kFmaTB - 1) / kFmaTB));
  const dim3 block(64 * p.nw);
  if (xq)
    route_fma_kernel<EP, NCH, XT, WT, true><<<grid, block, 0, s>>>(
        (const XT*)x, (const WT*)wg, bias, T, H, E, k, ids, w, prob, xq, xs);
  else
    route_fma_kernel<EP, NCH, XT, WT, false><<<grid, block, 0, s>>>(
        (const XT*)x, (const WT*)wg, bias, T, H, E, k, ids, w, prob, xq, xs);
  return hipGetLastError();
}

template <int EP, int NCH>
hipError_t launch_fma_dt(const RoutePlan& p, const void* x, int xd, const void* wg, int wd,
                         const float* bias, int64_t T, int H, int E, int k, int32_t* ids, float* w,
                         float* prob, int8_t* xq, float* xs, hipStream_t s) {
  if (xd == kF32 && wd == kF32)
    return launch_fma<EP, NCH, float, float>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, s);
  if (xd == kF32 && wd == kBF16)
    return launch_fma<EP, NCH, float, uint16_t>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, s);
  if (xd == kBF16 && wd == kF32)
    return launch_fma<EP, NCH, uint16_t, float>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, s);
  return launch_fma<EP, NCH, uint16_t, uint16_t>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, s);
}

template <int BT>
hipError_t launch_mfma(const RoutePlan& p, const void* x, const void* wg, const float* bias,
                       int64_t T, int H, int E, int k, int32_t* ids, float* w, float* prob,
                       int8_t* xq, float* xs, void* ws, hipStream_t s) {
  const unsigned bx = (unsigned)((T + BT - 1) / BT);
  const uint16_t* xb = (const uint16_t*)x;
  const uint16_t* wb = (const uint16_t*)wg;
  if (p.kind == 1) {
    const dim3 grid(bx, 1, 1);
    if (xq)
      route_mfma_kernel<BT, true, true><<<grid, 256, 0, s>>>(xb, wb, bias, T, H, E, k, H, nullptr,
                                                             ids, w, prob, xq, xs);
    else
      route_mfma_kernel<BT, true, false><<<grid, 256, 0, s>>>(xb, wb, bias, T, H, E, k, H, nullptr,
                                                              ids, w, prob, xq, xs);
    return hipGetLastError();
  }
  float* part = (float*)ws;
  const dim3 grid(bx, (unsigned)((E + 63) / 64), (unsigned)p.ks);
  route_mfma_kernel<BT, false, false><<<grid, 256, 0, s>>>(xb, wb, bias, T, H, E, k, H / p.ks, part,
                                                           ids, w, prob, xq, xs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 g2((unsigned)((T + 3) / 4));
  if (xq)
    route_topk_kernel<true><<<g2, 256, 0, s>>>(part, p.ks, bias, T, E, k, H, xb, ids, w, prob, xq, xs);
  else
    route_topk_kernel<false><<<g2, 256, 0, s>>>(part, p.ks, bias, T, E, k, H, xb, ids, w, prob, xq, xs);
  return hipGetLastError();
}

}  // namespace

RoutePlan plan_route(int64_t T, int H, int E, int k, int x_dtype, int wg_dtype) {
  (void)k;
  RoutePlan p{-1, 0, 1, 0, 0};
  if (E <= 16) {
    // one 8-value chunk of H per lane: H / 512 waves, Wg slice of 8*E registers
    const int nw = (H + 511) / 512;
    if (nw > (E <= 8 ? 16 : 8)) return p;
    p.kind = 0;
    p.bt = kFmaTB;
    p.nw = nw;
    return p;
  }
  if (x_dtype != kBF16 || wg_dtype != kBF16 || E % 16 != 0 || E > kMaxE) return p;
  p.bt = T >= 4096 ? 64 : (T >= 1024 ? 32 : 16);
  const int64_t tblocks = (T + p.bt - 1) / p.bt;
  if (E <= 64 && tblocks >= 64) {
    p.kind = 1;
    return p;
  }
  p.kind = 2;
  const int64_t blocks = tblocks * ((E + 63) / 64);
  int ks = 1;
  while (blocks * ks < 256 && H % (ks * 2 * 64) == 0 && H / (ks * 2) >= 256) ks *= 2;
  p.ks = ks;
  p.ws_bytes = (size_t)ks * (size_t)T * (size_t)E * sizeof(float);
  return p;
}

hipError_t launch_route(const RoutePlan& p, const void* x, int x_dtype, const void* wg,
                        int wg_dtype, const float* bias, int64_t T, int H, int E, int k,
                        int32_t* ids, float* w, float* prob, int8_t* xq, float* xs, void* ws,
                        hipStream_t s) {
  if (p.kind == 0) {
    if (E <= 8)
      return launch_fma_dt<8, 1>(p, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, ids, w, prob, xq,
                                 xs, s);
    return launch_fma_dt<16, 1>(p, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, ids, w, prob, xq,
                                xs, s);
  }
  switch (p.bt) {
    case 64:
      return launch_mfma<64>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, ws, s);
    case 32:
      return launch_mfma<32>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, ws, s);
    default:
      return launch_mfma<16>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, ws, s);
  }
}

}  // namespace moe
