// Expert FFN: per-expert SwiGLU over the expert-sorted rows, as a pair of
// grouped GEMMs driven by the align step's row-tile list.
//
// What is computed: the MoE FlashAttention page (framerc.cn) runs each
// expert's FFN on its own tokens (step 4) and its fused MoE call takes the
// expert weights stacked in one tensor with activation "silu"; the LightOP
// page, sections 4.1 and 4.3, gives the W16A16 / W8A8 MoE variants and the
// W8A8 rule (per-token int8 activations, per-channel int8 weights, int32
// accumulation, output scaled by both scales).  For sorted row r of expert e
// (token t): h = silu(W1 x_t) * (W3 x_t);  Y[r] = w_r * (W2 h).
//
// gfx950 design:
//  * One workgroup computes a BM x BN output tile of one row tile (one
//    expert, <= BM rows) from the tile list; the grid is the host-known upper
//    bound on tiles times the N blocks, and workgroups past the device-side
//    tile count exit at once (no host synchronisation).
//  * K advances 128 bytes at a time (64 bf16 or 128 int8).  Tiles of A and B
//    go global -> registers -> LDS, double buffered: the next k-step's global
//    loads are in flight while the MFMAs consume the current LDS stage.  Each
//    128-byte LDS row is split in eight 16-byte chunks stored at chunk
//    c ^ (row & 7), so the 32-row column reads of the MFMA operands spread
//    over all banks.
//  * MFMA 32x32x16 bf16 (fp32 accumulate) or 32x32x32 int8 (int32
//    accumulate).  In both a lane supplies 16 contiguous bytes of K for row
//    (lane % 32) at k-chunk (lane / 32); the byte layout of the mainloop is
//    therefore identical for the two types.
//  * The up GEMM gathers x rows through sorted_slot (dispatch without a
//    permuted copy of x), loads the W1 and W3 rows of the same h columns in
//    one B tile, and applies SwiGLU in registers: only h is written.
//  * The down GEMM multiplies each output row by its route weight before the
//    single bf16 rounding, so the combine only sums.
//  * W8A8: the up epilogue dequantises with the token and channel scales,
//    writes h in fp32 and folds each row's max |h| in with an integer atomic
//    max (non-negative floats order like their bit patterns); a row pass then
//    quantises h with the per-token rule, and the down GEMM runs int8 MFMA.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kI8 = 2;

__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

template <bool I8>
struct Mma;
template <>
struct Mma<false> {
  typedef f32x16 Acc;
  static __device__ __forceinline__ Acc run(const uint4& a, const uint4& b, const Acc& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mma<true> {
  typedef i32x16 Acc;
  static __device__ __forceinline__ Acc run(const uint4& a, const uint4& b, const Acc& c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                 __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
  }
};

// acc[FM][NF] += A_tile * B_tile^T over nk steps of 128 bytes of K.
// aload(p, kt) returns this thread's p-th A chunk of step kt; bptr[p] points
// at this thread's p-th B chunk of step 0.  Chunk q = tid + p*NT is row q/8,
// 16-byte column q%8.  wrow: first A row of this wave; brow_of(nf): first B
// row of the wave's nf-th 32-column fragment.
template <bool I8, int BM, int BNB, int NT, int FM, int NF, typename ALoad, typename BRow>
__device__ __forceinline__ void gemm_mainloop(uint8_t* __restrict__ smem, ALoad&& aload,
                                              const uint8_t* const* bptr, int nk, int wrow,
                                              BRow&& brow_of, typename Mma<I8>::Acc (&acc)[FM][NF]) {
  constexpr int APASS = BM * 8 / NT;
  constexpr int BPASS = BNB * 8 / NT;
  constexpr int STAGE = (BM + BNB) * 128;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  uint4 ar[APASS], br[BPASS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int p = 0; p < APASS; ++p) ar[p] = aload(p, kt);
#pragma unroll
    for (int p = 0; p < BPASS; ++p) br[p] = *reinterpret_cast<const uint4*>(bptr[p] + (size_t)kt * 128);
  };
  auto sstore = [&](int st) {
    uint8_t* base = smem + st * STAGE;
#pragma unroll
    for (int p = 0; p < APASS; ++p) {
      const int q = tid + p * NT;
      *reinterpret_cast<uint4*>(base + swz(q >> 3, q & 7)) = ar[p];
    }
#pragma unroll
    for (int p = 0; p < BPASS; ++p) {
      const int q = tid + p * NT;
      *reinterpret_cast<uint4*>(base + BM * 128 + swz(q >> 3, q & 7)) = br[p];
    }
  };
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* As = smem + cur * STAGE;
    const uint8_t* Bs = As + BM * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 2 * s + (lane >> 5);
      uint4 a[FM], b[NF];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        a[fm] = *reinterpret_cast<const uint4*>(As + swz(wrow + fm * 32 + (lane & 31), c));
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
        b[nf] = *reinterpret_cast<const uint4*>(Bs + swz(brow_of(nf) + (lane & 31), c));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) acc[fm][nf] = Mma<I8>::run(a[fm], b[nf], acc[fm][nf]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }
}

// MFMA 32x32 accumulator element v of lane l sits at row 8*(v/4) + 4*(l/32) + v%4,
// column l%32 of the fragment.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// ------------------------------------------------------------- up GEMM ---
template <bool I8, int BM, int BNH, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void ffn_up_kernel(
    const uint8_t* __restrict__ act, const float* __restrict__ xs, const uint8_t* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int H, int I, int k,
    int n_blocks, void* __restrict__ hout, uint32_t* __restrict__ rowmax) {
  constexpr int NT = WM * WN * 64;
  constexpr int BNB = 2 * BNH;
  constexpr int WROWS = BM / WM, FM = WROWS / 32;
  constexpr int WCOLS = BNH / WN, FN = WCOLS / 32, NF = 2 * FN;
  constexpr int APASS = BM * 8 / NT, BPASS = BNB * 8 / NT;
  constexpr int EB = I8 ? 1 : 2;
  static_assert(APASS * NT == BM * 8 && BPASS * NT == BNB * 8, "tile / thread mismatch");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BNB) * 128];

  const int tile = blockIdx.x / n_blocks;
  const int nb = blockIdx.x - tile * n_blocks;
  if (tile >= *num_tiles) return;
  const int4 td = reinterpret_cast<const int4*>(tiles)[tile];
  const int e = td.x, r0 = td.y, rows = td.z;
  const int n0 = nb * BNH;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / WN, wn = wv - (wv / WN) * WN;
  const int64_t row_bytes = (int64_t)H * EB;

  const uint8_t* aptr[APASS];
  bool aval[APASS];
#pragma unroll
  for (int p = 0; p < APASS; ++p) {
    const int q = tid + p * NT, r = q >> 3, c = q & 7;
    aval[p] = r < rows;
    const int tok = aval[p] ? sorted_slot[r0 + r] / k : 0;
    aptr[p] = act + (int64_t)tok * row_bytes + c * 16;
  }
  const uint8_t* bptr[BPASS];
#pragma unroll
  for (int p = 0; p < BPASS; ++p) {
    const int q = tid + p * NT, r = q >> 3, c = q & 7;
    const int wrow = r < BNH ? n0 + r : I + n0 + (r - BNH);
    bptr[p] = w13 + ((int64_t)e * 2 * I + wrow) * row_bytes + c * 16;
  }
  typename Mma<I8>::Acc acc[FM][NF];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) acc[fm][nf] = typename Mma<I8>::Acc{};

  auto aload = [&](int p, int kt) -> uint4 {
    return aval[p] ? *reinterpret_cast<const uint4*>(aptr[p] + (size_t)kt * 128) : make_uint4(0, 0, 0, 0);
  };
  auto brow_of = [&](int nf) -> int {
    return nf < FN ? wn * WCOLS + nf * 32 : BNH + wn * WCOLS + (nf - FN) * 32;
  };
  gemm_mainloop<I8, BM, BNB, NT, FM, NF>(smem, aload, bptr, (int)(row_bytes / 128), wm * WROWS,
                                         brow_of, acc);

  if (!I8) {
    uint16_t* h = reinterpret_cast<uint16_t*>(hout);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WROWS + fm * 32 + acc_row(v, lane);
        if (row >= rows) continue;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int col = n0 + wn * WCOLS + f * 32 + (lane & 31);
          const float g = (float)acc[fm][f][v], u = (float)acc[fm][FN + f][v];
          h[(int64_t)(r0 + row) * I + col] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
        }
      }
  } else {
    float* h = reinterpret_cast<float*>(hout);
    float sg[FN], su[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int col = n0 + wn * WCOLS + f * 32 + (lane & 31);
      sg[f] = s13[(int64_t)e * 2 * I + col];
      su[f] = s13[(int64_t)e * 2 * I + I + col];
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WROWS + fm * 32 + acc_row(v, lane);
        const bool valid = row < rows;
        const float xsr = valid ? xs[sorted_slot[r0 + row] / k] : 0.f;
        float m = 0.f;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int col = n0 + wn * WCOLS + f * 32 + (lane & 31);
          const float g = (float)acc[fm][f][v] * xsr * sg[f];
          const float u = (float)acc[fm][FN + f][v] * xsr * su[f];
          const float hv = silu_f32(g) * u;
          if (valid) h[(int64_t)(r0 + row) * I + col] = hv;
          m = fmaxf(m, fabsf(hv));
        }
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
        if (valid && (lane & 31) == 0) atomicMax(rowmax + r0 + row, __float_as_uint(m));
      }
  }
}

// ----------------------------------------------------------- down GEMM ---
template <bool I8, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void ffn_down_kernel(
    const uint8_t* __restrict__ hin, const float* __restrict__ hs, const uint8_t* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    const float* __restrict__ topk_w, int H, int I, int n_blocks, uint16_t* __restrict__ y) {
  constexpr int NT = WM * WN * 64;
  constexpr int WROWS = BM / WM, FM = WROWS / 32;
  constexpr int WCOLS = BN / WN, NF = WCOLS / 32;
  constexpr int APASS = BM * 8 / NT, BPASS = BN * 8 / NT;
  constexpr int EB = I8 ? 1 : 2;
  static_assert(APASS * NT == BM * 8 && BPASS * NT == BN * 8, "tile / thread mismatch");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * 128];

  const int tile = blockIdx.x / n_blocks;
  const int nb = blockIdx.x - tile * n_blocks;
  if (tile >= *num_tiles) return;
  const int4 td = reinterpret_cast<const int4*>(tiles)[tile];
  const int e = td.x, r0 = td.y, rows = td.z;
  const int n0 = nb * BN;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / WN, wn = wv - (wv / WN) * WN;
  const int64_t row_bytes = (int64_t)I * EB;

  const uint8_t* aptr[APASS];
  bool aval[APASS];
#pragma unroll
  for (int p = 0; p < APASS; ++p) {
    const int q = tid + p * NT, r = q >> 3, c = q & 7;
    aval[p] = r < rows;
    aptr[p] = hin + (int64_t)(aval[p] ? r0 + r : 0) * row_bytes + c * 16;
  }
  const uint8_t* bptr[BPASS];
#pragma unroll
  for (int p = 0; p < BPASS; ++p) {
    const int q = tid + p * NT, r = q >> 3, c = q & 7;
    bptr[p] = w2 + ((int64_t)e * H + n0 + r) * row_bytes + c * 16;
  }
  typename Mma<I8>::Acc acc[FM][NF];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) acc[fm][nf] = typename Mma<I8>::Acc{};
  auto aload = [&](int p, int kt) -> uint4 {
    return aval[p] ? *reinterpret_cast<const uint4*>(aptr[p] + (size_t)kt * 128) : make_uint4(0, 0, 0, 0);
  };
  auto brow_of = [&](int nf) -> int { return wn * WCOLS + nf * 32; };
  gemm_mainloop<I8, BM, BN, NT, FM, NF>(smem, aload, bptr, (int)(row_bytes / 128), wm * WROWS,
                                        brow_of, acc);

  float sc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
    sc[f] = I8 ? s2[(int64_t)e * H + n0 + wn * WCOLS + f * 32 + (lane & 31)] : 1.f;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wm * WROWS + fm * 32 + acc_row(v, lane);
      if (row >= rows) continue;
      float wr = topk_w ? topk_w[sorted_slot[r0 + row]] : 1.f;
      if (I8) wr *= hs[r0 + row];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int col = n0 + wn * WCOLS + f * 32 + (lane & 31);
        y[(int64_t)(r0 + row) * H + col] = (uint16_t)f32_to_bf16_bits((float)acc[fm][f][v] * sc[f] * wr);
      }
    }
}

// ----------------------------------------------------- W8A8 h quantise ---
// One wave per sorted row of a tile: s = max|h| / 127 (1 if 0),
// q = round-half-even(h / s) clamped to [-128, 127]; fp32 IEEE arithmetic.
__global__ __launch_bounds__(256) void quant_h_kernel(const float* __restrict__ h,
                                                      const uint32_t* __restrict__ rowmax,
                                                      const int32_t* __restrict__ tiles,
                                                      const int32_t* __restrict__ num_tiles, int I,
                                                      int8_t* __restrict__ hq, float* __restrict__ hs) {
  const int tile = blockIdx.x;
  if (tile >= *num_tiles) return;
  const int4 td = reinterpret_cast<const int4*>(tiles)[tile];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x >> 6; i < td.z; i += 4) {
    const int64_t r = td.y + i;
    const float am = __uint_as_float(rowmax[r]);
    const float s = am == 0.f ? 1.f : am / 127.f;
    for (int c = lane * 8; c < I; c += 512) {
      float v[8];
      load8(h + r * I + c, v);
      uint32_t b[2] = {0u, 0u};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float z = rintf(v[q] / s);
        z = fminf(fmaxf(z, -128.f), 127.f);
        b[q >> 2] |= (uint32_t)((int)z & 0xFF) << (8 * (q & 3));
      }
      *reinterpret_cast<uint2*>(hq + r * I + c) = make_uint2(b[0], b[1]);
    }
    if (lane == 0) hs[r] = s;
  }
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ------------------------------------------------------------ fp32 path --
// Plain LDS-tiled FMA GEMMs (32 x 32 output tile, 256 threads, 4 rows each).
template <bool UP>
__global__ __launch_bounds__(256) void ffn_f32_kernel(
    const float* __restrict__ a, const float* __restrict__ wts, const int32_t* __restrict__ sorted_slot,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    const float* __restrict__ topk_w, int H, int I, int k, int n_blocks, float* __restrict__ out) {
  __shared__ float As[32][33], Bg[32][33], Bu[UP ? 32 : 1][33];
  const int tile = blockIdx.x / n_blocks;
  const int nb = blockIdx.x - tile * n_blocks;
  if (tile >= *num_tiles) return;
  const int4 td = reinterpret_cast<const int4*>(tiles)[tile];
  const int e = td.x, r0 = td.y, rows = td.z;
  const int n0 = nb * 32;
  const int tid = threadIdx.x, tx = tid & 31, ty = tid >> 5;
  const int K = UP ? H : I;
  const int lr = tid >> 3, lc = (tid & 7) * 4;
  const bool lval = lr < rows;
  const float* arow = UP ? a + (int64_t)(lval ? sorted_slot[r0 + lr] / k : 0) * K
                         : a + (int64_t)(lval ? r0 + lr : 0) * K;
  const float* grow = UP ? wts + ((int64_t)e * 2 * I + n0 + lr) * K : wts + ((int64_t)e * H + n0 + lr) * K;
  const float* urow = UP ? wts + ((int64_t)e * 2 * I + I + n0 + lr) * K : grow;
  float ag[4] = {0, 0, 0, 0}, au[4] = {0, 0, 0, 0};
  for (int k0 = 0; k0 < K; k0 += 32) {
    const float4 av = lval ? *reinterpret_cast<const float4*>(arow + k0 + lc) : make_float4(0, 0, 0, 0);
    const float4 gv = *reinterpret_cast<const float4*>(grow + k0 + lc);
    As[lr][lc] = av.x; As[lr][lc + 1] = av.y; As[lr][lc + 2] = av.z; As[lr][lc + 3] = av.w;
    Bg[lr][lc] = gv.x; Bg[lr][lc + 1] = gv.y; Bg[lr][lc + 2] = gv.z; Bg[lr][lc + 3] = gv.w;
    if (UP) {
      const float4 uv = *reinterpret_cast<const float4*>(urow + k0 + lc);
      Bu[lr][lc] = uv.x; Bu[lr][lc + 1] = uv.y; Bu[lr][lc + 2] = uv.z; Bu[lr][lc + 3] = uv.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      const float b = Bg[tx][kk];
      const float bu = UP ? Bu[tx][kk] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float av2 = As[ty * 4 + i][kk];
        ag[i] = fmaf(av2, b, ag[i]);
        if (UP) au[i] = fmaf(av2, bu, au[i]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= rows) continue;
    if (UP) {
      out[(int64_t)(r0 + row) * I + n0 + tx] = silu_f32(ag[i]) * au[i];
    } else {
      const float wr = topk_w ? topk_w[sorted_slot[r0 + row]] : 1.f;
      out[(int64_t)(r0 + row) * H + n0 + tx] = ag[i] * wr;
    }
  }
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct FfnBufs {
  void* h;
  uint32_t* rowmax;
  int8_t* hq;
  float* hs;
};

FfnBufs carve_ffn(void* ws, int64_t n, int I, int w_dtype) {
  uint8_t* wsb = (uint8_t*)ws;
  FfnBufs b{wsb, nullptr, nullptr, nullptr};
  if (w_dtype == kI8) {
    size_t off = align256((size_t)n * I * 4);
    b.rowmax = (uint32_t*)(wsb + off);
    off += align256((size_t)n * 4);
    b.hq = (int8_t*)(wsb + off);
    off += align256((size_t)n * I);
    b.hs = (float*)(wsb + off);
  }
  return b;
}

template <bool I8>
hipError_t launch_up(const FfnPlan& p, const void* act, const float* xs, const void* w13,
                     const float* s13, const int32_t* sorted_slot, const int32_t* tiles,
                     const int32_t* num_tiles, int64_t T, int H, int I, int k, const FfnBufs& b,
                     hipStream_t s) {
  const int64_t n = T * k;
  if (I8) zero_u32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(b.rowmax, n);
  const unsigned mt = (unsigned)p.max_tiles;
  if (I % 128 == 0) {
    const int nbk = I / 128;
    ffn_up_kernel<I8, 128, 128, 2, 2><<<mt * nbk, 256, 0, s>>>(
        (const uint8_t*)act, xs, (const uint8_t*)w13, s13, sorted_slot, tiles, num_tiles, H, I, k,
        nbk, b.h, b.rowmax);
  } else {
    const int nbk = I / 64;
    ffn_up_kernel<I8, 128, 64, 2, 2><<<mt * nbk, 256, 0, s>>>(
        (const uint8_t*)act, xs, (const uint8_t*)w13, s13, sorted_slot, tiles, num_tiles, H, I, k,
        nbk, b.h, b.rowmax);
  }
  return hipGetLastError();
}

template <bool I8>
hipError_t launch_down(const FfnPlan& p, const void* w2, const float* s2, const int32_t* sorted_slot,
                       const int32_t* tiles, const int32_t* num_tiles, const float* topk_w, int H,
                       int I, void* y, const FfnBufs& b, hipStream_t s) {
  const unsigned mt = (unsigned)p.max_tiles;
  const uint8_t* hin = (const uint8_t*)b.h;
  if (I8) {
    quant_h_kernel<<<mt, 256, 0, s>>>((const float*)b.h, b.rowmax, tiles, num_tiles, I, b.hq, b.hs);
    hin = (const uint8_t*)b.hq;
  }
  if (H % 128 == 0) {
    const int nbk = H / 128;
    ffn_down_kernel<I8, 128, 128, 2, 2><<<mt * nbk, 256, 0, s>>>(
        hin, b.hs, (const uint8_t*)w2, s2, sorted_slot, tiles, num_tiles, topk_w, H, I, nbk, (uint16_t*)y);
  } else {
    const int nbk = H / 64;
    ffn_down_kernel<I8, 128, 64, 2, 2><<<mt * nbk, 256, 0, s>>>(
        hin, b.hs, (const uint8_t*)w2, s2, sorted_slot, tiles, num_tiles, topk_w, H, I, nbk, (uint16_t*)y);
  }
  return hipGetLastError();
}

}  // namespace

FfnPlan plan_ffn(int64_t T, int H, int I, int E, int k, int w_dtype) {
  FfnPlan p{};
  const int64_t n = T * k;
  if (w_dtype == kF32) {
    p.block_m = 32;
    p.ws_bytes = align256((size_t)n * I * 4);
    p.up_name = "ffn_f32_kernel<up>";
    p.down_name = "ffn_f32_kernel<down>";
  } else if (w_dtype == kBF16) {
    p.block_m = 128;
    p.ws_bytes = align256((size_t)n * I * 2);
    p.up_name = I % 128 == 0 ? "ffn_up_kernel<bf16,128,128,2,2>" : "ffn_up_kernel<bf16,128,64,2,2>";
    p.down_name = H % 128 == 0 ? "ffn_down_kernel<bf16,128,128,2,2>" : "ffn_down_kernel<bf16,128,64,2,2>";
  } else {
    p.block_m = 128;
    p.ws_bytes = align256((size_t)n * I * 4) + align256((size_t)n * 4) + align256((size_t)n * I) +
                 align256((size_t)n * 4);
    p.up_name = I % 128 == 0 ? "ffn_up_kernel<i8,128,128,2,2>" : "ffn_up_kernel<i8,128,64,2,2>";
    p.down_name = H % 128 == 0 ? "ffn_down_kernel<i8,128,128,2,2>" : "ffn_down_kernel<i8,128,64,2,2>";
  }
  p.max_tiles = align_max_tiles(T, k, E, p.block_m);
  return p;
}

hipError_t launch_ffn_up(const FfnPlan& p, const void* x, const float* xs, const void* w13,
                         int w_dtype, const float* s13, const int32_t* sorted_slot,
                         const int32_t* tiles, const int32_t* num_tiles, int64_t T, int H, int I,
                         int k, void* ws, hipStream_t s) {
  const FfnBufs b = carve_ffn(ws, T * k, I, w_dtype);
  if (w_dtype == kF32) {
    const unsigned mt = (unsigned)p.max_tiles;
    ffn_f32_kernel<true><<<mt * (I / 32), 256, 0, s>>>((const float*)x, (const float*)w13, sorted_slot,
                                                        tiles, num_tiles, nullptr, H, I, k, I / 32,
                                                        (float*)b.h);
    return hipGetLastError();
  }
  if (w_dtype == kBF16)
    return launch_up<false>(p, x, xs, w13, s13, sorted_slot, tiles, num_tiles, T, H, I, k, b, s);
  return launch_up<true>(p, x, xs, w13, s13, sorted_slot, tiles, num_tiles, T, H, I, k, b, s);
}

hipError_t launch_ffn_down(const FfnPlan& p, const void* w2, int w_dtype, const float* s2,
                           const int32_t* sorted_slot, const int32_t* tiles,
                           const int32_t* num_tiles, const float* topk_w, int64_t T, int H, int I,
                           int k, void* y, void* ws, hipStream_t s) {
  const FfnBufs b = carve_ffn(ws, T * k, I, w_dtype);
  if (w_dtype == kF32) {
    const unsigned mt = (unsigned)p.max_tiles;
    ffn_f32_kernel<false><<<mt * (H / 32), 256, 0, s>>>((const float*)b.h, (const float*)w2,
                                                         sorted_slot, tiles, num_tiles, topk_w, H, I,
                                                         k, H / 32, (float*)y);
    return hipGetLastError();
  }
  if (w_dtype == kBF16)
    return launch_down<false>(p, w2, s2, sorted_slot, tiles, num_tiles, topk_w, H, I, y, b, s);
  return launch_down<true>(p, w2, s2, sorted_slot, tiles, num_tiles, topk_w, H, I, y, b, s);
}

}  // namespace moe
