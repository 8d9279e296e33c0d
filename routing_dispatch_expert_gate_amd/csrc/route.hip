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
// Two variants, picked on the host by shape (never silently):
//   kind 0  E <= 16: fp32 FMA.  Each wave keeps its slice of Wg (8 values of
//           H per lane, all experts) in registers and re-uses it for the
//           workgroup's 1, 4 or 16 tokens (by batch size), whose x chunks are
//           loaded in batches before their FMAs; the partial logits of a
//           group of rows are summed across the 64 lanes in one butterfly of
//           DPP and row-swap permutes, then across waves through LDS.  Logits
//           never leave the chip.
//   kind 2  E > 16, bf16: MFMA 32x32x16 bf16 over 64-token x 64-expert tiles,
//           K streamed through a deep direct-to-LDS pipeline (split while the
//           grid is small), partial logits to the workspace; a second kernel,
//           one wave per token, sums the splits in a fixed order, runs the
//           top-k and writes the per-token int8 codes.  Deterministic: no
//           floating-point atomics.
//           The same pair, with the top-k kernel's group-limited
//           selection, serves the group-limited router.
#include <math.h>

#include "block_align.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// --------------------------------------------------------------- top-k ----
// One wave selects the top-k of one token.  Lane l owns the logits of experts
// l + 64*j (j < 4, -inf beyond E).  Lanes 0..k-1 write selection i = lane.
// Selection by k argmax rounds over v (excluded experts hold -inf); m is the
// token's largest logit and s its softmax denominator (used only for prob).
__device__ void wave_topk_select_store(float v[4], int k, float m, float s, int64_t t,
                                       int32_t* __restrict__ ids, float* __restrict__ w,
                                       float* __restrict__ prob, int* hist = nullptr) {
  const int lane = threadIdx.x & 63;
  int my_id = 0;
  float my_l = -INFINITY;
  for (int i = 0; i < k; ++i) {
    // the largest remaining logit (DPP and readlanes: wave-uniform), then the
    // lowest expert id holding it: experts are lane + 64 j, so the first j
    // whose ballot is not empty, and its lowest lane
    const float bv = wave_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    int bi = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t hit = __ballot(v[j] == bv);
      if (bi < 0 && hit != 0ull) bi = 64 * j + __ffsll((unsigned long long)hit) - 1;
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
    if (hist) atomicAdd(&hist[my_id], 1);   // counts only: their order is irrelevant
  }
}

// The same selection for E <= 64, one logit per lane (lane = expert, -inf
// past E): k argmax rounds, the first of which gives the token's maximum.
__device__ void wave_topk64_store(float v, int E, int k, int64_t t, int32_t* __restrict__ ids,
                                  float* __restrict__ w, float* __restrict__ prob, int* hist = nullptr) {
  const int lane = threadIdx.x & 63;
  const float m = wave_max(v);
  const float s = prob ? wave_sum(lane < E ? expf(v - m) : 0.f) : 0.f;
  int my_id = 0;
  float my_l = -INFINITY;
  for (int i = 0; i < k; ++i) {
    const float bv = i == 0 ? m : wave_max(v);
    const int bi = __ffsll((unsigned long long)__ballot(v == bv)) - 1;   // lowest expert holding it
    if (lane == i) {
      my_id = bi;
      my_l = bv;
    }
    if (lane == bi) v = -INFINITY;
  }
  const float ex = lane < k ? expf(my_l - m) : 0.f;
  const float se = wave_sum(ex);
  if (lane < k) {
    ids[t * k + lane] = my_id;
    w[t * k + lane] = ex / se;
    if (prob) prob[t * k + lane] = ex / s;
    if (hist) atomicAdd(&hist[my_id], 1);   // counts only: their order is irrelevant
  }
}

__device__ __forceinline__ float wave_logit_max(const float v[4]) {
  return wave_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
}
__device__ __forceinline__ float wave_softmax_denominator(const float v[4], int E, float m) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (lane + 64 * j < E) s += expf(v[j] - m);
  return wave_sum(s);
}

__device__ void wave_topk_store(float v[4], int E, int k, int64_t t, int32_t* __restrict__ ids,
                                float* __restrict__ w, float* __restrict__ prob, int* hist = nullptr) {
  const float m = wave_logit_max(v);
  const float s = prob ? wave_softmax_denominator(v, E, m) : 0.f;
  wave_topk_select_store(v, k, m, s, t, ids, w, prob, hist);
}

// Group-limited top-k of one token (LightOP page, section 3.1, Moe Fuse Gate:
// pick the groups first, keeping each group's Top1/Top2).  The E experts form
// G contiguous groups of E/G; a group's score is the sum of the
// exponentials of its two largest logits (its probabilities' sum times the
// token's common softmax denominator, so the order is that of the
// probabilities); the TG best groups (equal scores: lower group first) keep
// their experts, every other expert is set to -inf, and the usual argmax
// rounds select k, weighted as in the plain router with the full softmax.
// L: this wave's 256-float LDS row; gs: its 64-float LDS row.  G <= 64.
__device__ void wave_grouped_topk_store(float v[4], float* L, float* gs, int E, int k, int G, int TG,
                                        int64_t t, int32_t* __restrict__ ids, float* __restrict__ w,
                                        float* __restrict__ prob) {
  const int lane = threadIdx.x & 63;
  const float m = wave_logit_max(v);
  const float s = prob ? wave_softmax_denominator(v, E, m) : 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) L[lane + 64 * j] = v[j];
  __builtin_amdgcn_wave_barrier();
  const int gsz = E / G;
  float score = -INFINITY;
  if (lane < G) {
    // the group's two largest logits (a tie counts twice)
    float a1 = -INFINITY, a2 = -INFINITY;
    for (int i = 0; i < gsz; ++i) {
      const float u = L[lane * gsz + i];
      if (u > a1) {
        a2 = a1;
        a1 = u;
      } else if (u > a2) {
        a2 = u;
      }
    }
    score = expf(a1 - m) + (gsz > 1 ? expf(a2 - m) : 0.f);
    gs[lane] = score;
  }
  __builtin_amdgcn_wave_barrier();
  int rank = 0;
  if (lane < G)
    for (int g = 0; g < G; ++g) {
      const float o = gs[g];
      rank += (o > score || (o == score && g < lane)) ? 1 : 0;
    }
  const uint64_t keep = __ballot(lane < G && rank < TG);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E && !((keep >> (e / gsz)) & 1ull)) v[j] = -INFINITY;
  }
  wave_topk_select_store(v, k, m, s, t, ids, w, prob);
}

// Top-k of one token by rank, for E <= 64: the token's E logits are in an LDS
// row (16-byte aligned, padded with -inf to a multiple of 4, read by every
// lane at once); lane l < E ranks expert
// l by counting the experts ahead of it in (logit descending, id ascending)
// order, and the k lanes of rank < k write selection rank.  The same order
// and arithmetic as wave_topk_store, without its serial argmax rounds.
__device__ void wave_topk_rank_store(const float* L, int E, int k, int64_t t, int32_t* __restrict__ ids,
                                     float* __restrict__ w, float* __restrict__ prob, int* hist = nullptr) {
  const int lane = threadIdx.x & 63;
  const float v = lane < E ? L[lane] : -INFINITY;
  int rank = 0;
  for (int j = 0; j < E; j += 4) {
    const float4 q = *reinterpret_cast<const float4*>(L + j);   // padded past E
    rank += (q.x > v || (q.x == v && j < lane)) ? 1 : 0;
    rank += (q.y > v || (q.y == v && j + 1 < lane)) ? 1 : 0;
    rank += (q.z > v || (q.z == v && j + 2 < lane)) ? 1 : 0;
    rank += (q.w > v || (q.w == v && j + 3 < lane)) ? 1 : 0;
  }
  const bool in = lane < E;
  const uint64_t top = __ballot(in && rank == 0);
  // the largest logit, from the lane of rank 0
  const float mf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), __ffsll((unsigned long long)top) - 1));
  const bool sel = in && rank < k;
  const float ex = sel ? expf(v - mf) : 0.f;
  const float se = wave_sum(ex);
  float s = 0.f;
  if (prob) s = wave_sum(in ? expf(v - mf) : 0.f);
  if (sel) {
    ids[t * k + rank] = lane;
    w[t * k + rank] = ex / se;
    if (prob) prob[t * k + rank] = ex / s;
    if (hist) atomicAdd(&hist[lane], 1);   // counts only: their order is irrelevant
  }
}

// ------------------------------------------------------- per-token quant --
// Codes of 4 or 8 values with scale s (rs = 1/s), as quant_code, for a row
// whose reciprocal scale is finite (rok; s is the row's max |x| / 127, so
// every |x * rs| <= 127 (1 + 2^-23) and rounds into [-127, 127]): x * rs
// rounds to the integer of the correctly rounded quotient unless it lies
// within 2^-14 of a half-integer; a group holding such a value (or a row
// without rok) takes the division for the whole group, clamped as the rule
// writes it (about one group in a thousand), so the common path has no
// branch, clamp or division per value.
__device__ __forceinline__ uint32_t pack_codes4(const float (&q)[4]) {
  const int32_t a = (int32_t)q[0], b = (int32_t)q[1], c = (int32_t)q[2], d = (int32_t)q[3];
  // v_perm_b32: selector bytes 0-3 pick the second operand's bytes, 4-7 the
  // first's, 0x0c gives zero
  return __builtin_amdgcn_perm(b, a, 0x0c0c0400u) | __builtin_amdgcn_perm(d, c, 0x04000c0cu);
}
template <int N>
__device__ __forceinline__ void quant_group(const float (&v)[N], float s, float rs, bool rok, float (&q)[N]) {
  bool risky = !rok;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float y = v[i] * rs;
    q[i] = rintf(y);
    // bitwise, not short-circuit: no branch per value
    risky = risky | !(fabsf(fabsf(y - q[i]) - 0.5f) >= 0x1p-14f);
  }
  if (risky) {
#pragma unroll
    for (int i = 0; i < N; ++i) q[i] = fminf(fmaxf(rintf(v[i] / s), -128.f), 127.f);
  }
}
__device__ __forceinline__ uint32_t quant4(const float (&v)[4], float s, float rs, bool rok) {
  float q[4];
  quant_group<4>(v, s, rs, rok, q);
  return pack_codes4(q);
}
__device__ __forceinline__ uint2 quant8(const float (&v)[8], float s, float rs, bool rok) {
  float q[8];
  quant_group<8>(v, s, rs, rok, q);
  const float lo[4] = {q[0], q[1], q[2], q[3]}, hi[4] = {q[4], q[5], q[6], q[7]};
  return make_uint2(pack_codes4(lo), pack_codes4(hi));
}
// whether a row's reciprocal scale is finite (a denormal scale's is not)
__device__ __forceinline__ bool rs_ok(float rs) { return rs <= 3.4028234e38f; }

__device__ __forceinline__ float row_scale(float absmax) {
  return absmax == 0.f ? 1.f : absmax / 127.f;
}

// ------------------------------------------------------------ kind 0 -----
// DPP move of a float from another lane (0 where the source lane is outside
// the row): quad_perm xor 1 = 0xB1, xor 2 = 0x4E; row_shr:n = 0x110 + n.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Wave sums of N values per lane (N = tokens x experts of a load batch), by
// a butterfly over the six lane bits, in the order 3, 2, 1, 0, 4, 5: the
// partner of each step differs from the lane in that bit only (DPP
// row_mirror, row_half_mirror, quad_perm xor 2 and xor 1, then the row-swap
// permutes for 16 and 32), and while more than one value is left the lane
// keeps the half its bit selects and adds the partner's copy of that half.
// Lane l ends with max(N / 64, 1) totals a[0..], of the flat indices
// bfly_base<N>(l) + i.  No step goes through the LDS crossbar and the N
// chains are independent, so they pipeline.
template <int S>
__device__ __forceinline__ float bfly_partner(float v) {
  if constexpr (S == 0) return dpp_f<0x140>(v);
  else if constexpr (S == 1) return dpp_f<0x141>(v);
  else if constexpr (S == 2) return dpp_f<0x4E>(v);
  else if constexpr (S == 3) return dpp_f<0xB1>(v);
  else if constexpr (S == 4) return lane_xor16(v);
  else return lane_xor32(v);
}
__device__ __forceinline__ constexpr int bfly_bit(int s) { return s < 4 ? 3 - s : s; }

template <int N, int S = 0>
__device__ __forceinline__ void wave_sum_all(float (&a)[N], int lane) {
  if constexpr (S < 6) {
    constexpr int n = (N >> S) > 1 ? (N >> S) : 1;   // values left before this step
    if constexpr (n >= 2) {
      constexpr int h = n / 2;
      const bool up = ((lane >> bfly_bit(S)) & 1) != 0;
#pragma unroll
      for (int i = 0; i < h; ++i) {
        const float send = up ? a[i] : a[i + h];
        const float keep = up ? a[i + h] : a[i];
        a[i] = keep + bfly_partner<S>(send);
      }
    } else {
      a[0] += bfly_partner<S>(a[0]);
    }
    wave_sum_all<N, S + 1>(a, lane);
  }
}
// first flat index of lane l's totals, and whether l is the one lane of its
// duplicates (N < 64 leaves 64 / N lanes with the same totals) that stores
template <int N>
__device__ __forceinline__ int bfly_base(int lane) {
  int b = 0;
#pragma unroll
  for (int s = 0; s < 6; ++s)
    if ((N >> s) >= 2) b += ((lane >> bfly_bit(s)) & 1) * (N >> (s + 1));
  return b;
}
template <int N>
__device__ __forceinline__ bool bfly_writer(int lane) {
  bool w = true;
#pragma unroll
  for (int s = 0; s < 6; ++s)
    if ((N >> s) < 2) w = w && ((lane >> bfly_bit(s)) & 1) == 0;
  return w;
}

// tokens per workgroup: 16 where the grid still fills the chip (and for the
// fused route + align, whose one workgroup takes every token); fewer for
// smaller batches, since a workgroup's E*H FMAs per token run on one CU
constexpr int kFmaTB = 16;
inline int fma_tokens_per_wg(int64_t T) { return T >= 16 * 256 ? 16 : T >= 4 * 256 ? 4 : 1; }

// The raw bytes of 8 consecutive x values, loaded in one go and widened later
// (so a batch of rows can be in flight before the first use).
template <typename XT>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  u32x4 a;
  __device__ __forceinline__ void load(const uint16_t* p) { a = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void zero() { a = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void get(float (&v)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Raw8<float> {
  u32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const u32x4*>(p)[0];
    b = reinterpret_cast<const u32x4*>(p)[1];
  }
  __device__ __forceinline__ void zero() { a = b = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void get(float (&v)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  }
};

// WIDE: more than 8 waves (H > 4096, E <= 8 only), 1024 threads and hence at
// most 128 VGPRs: fewer rows in flight.
// A workgroup's token rows are loaded in batches of PF rows, each batch before
// its first FMA; the partial logits of G rows at a time are summed over the
// wave by wave_sum_all.
template <int EP, bool WIDE, typename XT, typename WT, bool QUANT, bool ALIGN, int TB, int NVMAX = 64>
__global__ __launch_bounds__(WIDE ? 1024 : 512) void route_fma_kernel(
    const XT* __restrict__ x, const WT* __restrict__ wg, const float* __restrict__ bias, int64_t T,
    int H, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    float* __restrict__ prob, int8_t* __restrict__ xq, float* __restrict__ xs, const AlignArgs al,
    int32_t* __restrict__ whist) {
  // rows per load batch (all sixteen at once costs occupancy: measured
  // slower at large T)
  constexpr int PF0 = (sizeof(XT) == 4 ? 4 : 8) / (WIDE ? 2 : 1), PF = PF0 < TB ? PF0 : TB;
  static_assert(TB % PF == 0, "batches");
  static_assert(!ALIGN || TB == kFmaTB, "the fused align takes one workgroup of kFmaTB tokens");
  // rows per wave reduction: at most NVMAX sums at once (64 measured best at
  // one workgroup per CU, 32 with several resident)
  constexpr int G = PF * EP <= NVMAX ? PF : NVMAX / EP, NV = G * EP;
  static_assert(PF % G == 0, "reduction groups");
  __shared__ float part[16][TB][EP];
  __shared__ float amax_s[16][TB];
  __shared__ __attribute__((aligned(16))) float lg[TB][16];
  __shared__ int hist[16];   // this workgroup's selections per expert (whist)
  const int nw = blockDim.x >> 6;
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;

  // this lane's slice of Wg: 8 consecutive h, for every expert
  float wr[EP][8];
  const int h0 = (wv * 64 + lane) * 8;
  const bool hv = h0 < H;
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (hv && e < E) load8(wg + (size_t)e * H + h0, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) wr[e][i] = v[i];
  }

  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int ntok = (int)((T - t0) < TB ? (T - t0) : TB);
  for (int tb = 0; tb < ntok; tb += PF) {
    Raw8<XT> r[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      if (hv && tb + u < ntok)
        r[u].load(x + (t0 + tb + u) * H + h0);
      else
        r[u].zero();
    }
    // G rows at a time: their G x EP partial dot products (rows past ntok
    // are zeros), summed over the wave together
#pragma unroll
    for (int g0 = 0; g0 < PF; g0 += G) {
      float acc[NV];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        float v[8];
        r[g0 + u].get(v);
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaf(v[i], wr[e][i], a);
          acc[u * EP + e] = a;
        }
        if (QUANT) {
          float am = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
          am = wave_max(am);
          if (lane == 0 && tb + g0 + u < ntok) amax_s[wv][tb + g0 + u] = am;
        }
      }
      wave_sum_all<NV>(acc, lane);
      if (bfly_writer<NV>(lane)) {
        const int base = bfly_base<NV>(lane);
#pragma unroll
        for (int i = 0; i < (NV >= 64 ? NV / 64 : 1); ++i) {
          const int j = base + i, u = j / EP;
          if (tb + g0 + u < ntok) part[wv][tb + g0 + u][j - u * EP] = acc[i];
        }
      }
    }
  }
  __syncthreads();

  // logits (plus bias) of the block's tokens, rows padded with -inf
  if (threadIdx.x < 16) hist[threadIdx.x] = 0;
  for (int i = threadIdx.x; i < TB * 16; i += blockDim.x) {
    const int tt = i >> 4, e = i & 15;
    float s = -INFINITY;
    if (tt < ntok && e < E) {
      s = 0.f;
      for (int q = 0; q < nw; ++q) s += part[q][tt][e];
      if (bias) s += bias[e];
    }
    lg[tt][e] = s;
  }
  __syncthreads();
  for (int tt = wv; tt < ntok; tt += nw)
    wave_topk_rank_store(&lg[tt][0], E, k, t0 + tt, ids, w, prob, whist ? hist : nullptr);
  if (whist) {
    // publish the workgroup's per-expert selection counts for the align step
    __syncthreads();
    if (threadIdx.x < E) whist[(int64_t)blockIdx.x * E + threadIdx.x] = hist[threadIdx.x];
  }

  if (QUANT) {
    for (int tb = 0; tb < ntok; tb += PF) {
      Raw8<XT> r[PF];
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        if (hv && tb + u < ntok)
          r[u].load(x + (t0 + tb + u) * H + h0);
        else
          r[u].zero();
      }
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int tt = tb + u;
        if (tt >= ntok) break;
        float am = 0.f;
        for (int q = 0; q < nw; ++q) am = fmaxf(am, amax_s[q][tt]);
        const float s = row_scale(am);
        if (hv) {
          float v[8];
          r[u].get(v);
          *reinterpret_cast<uint2*>(xq + (t0 + tt) * H + h0) = quant8(v, s, 1.f / s, rs_ok(1.f / s));
        }
        if (threadIdx.x == 0) xs[t0 + tt] = s;
      }
    }
  }
  if constexpr (ALIGN) {
    // a single workgroup routed every token: align its T*k slots here
    __syncthreads();
    block_align<16>([&](int64_t sl) { return ids[sl]; }, T * k, E, al.ebits, al.cap, al.bm, al.max_tiles,
                    al.counts, al.offsets, al.sorted_slot, al.pos, al.tiles, al.num_tiles, al.num_dropped);
  }
}

// ------------------------------------------------------------ kind 2 -----
// Gate logits on MFMA: one workgroup computes an RT-token x RE-expert tile
// of x Wg^T over a K range (all of H unless split).  K is streamed 64 bf16
// (128 bytes) per stage from global memory straight into LDS, as many stages
// deep as 128 KiB holds; waves form a 2 x 2 grid, each owning (RT/2) x (RE/2)
// outputs as 32 x 32 MFMA 32x32x16 fragments.  Token rows past T and expert
// rows past E copy a valid row; their results are never used.  The tile is
// written to the workspace; with quantisation the first expert block also
// folds each token row's absmax over its K range from the A stages as they
// pass through LDS.  route_topk_kernel then sums the K splits, runs the top-k
// and writes the codes, one wave per token.
// Tiles: 64 x 64, K split while the grid is small; at large batches with E
// a multiple of 128, 128 x 128 split in K back up to a full grid: each
// workgroup then reads half the bytes per output of a 64 x 64 tile, which is
// what bounds the step (each CU's copy rate), for more partial logits.
constexpr int kRT = 64;                        // tokens per tile (small batches)
constexpr int kTopkHistTokens = 16;            // tokens per top-k workgroup that publishes counts
// top-k workgroups per published count row: about 1024 slots, one align block
inline int topk_hist_group(int k) {
  const int g = 1024 / (kTopkHistTokens * k);
  return g < 1 ? 1 : g;
}
constexpr int kRE = 64;                        // experts per tile (small batches)
constexpr int kRRow = 128;                     // bytes of K per stage row
constexpr int kRLds = 128 * 1024;              // bytes of stages
constexpr int kRouteGemmWaves128 = 8;          // waves of a 128 x 128 tile (4, 8 or 16; 8 measured best)

// workspace: partial logits [ks][T][E] fp32, then per-split row absmax [ks][T]
size_t route_part_bytes(int64_t T, int E, int ks) {
  return ((size_t)ks * (size_t)T * (size_t)E * sizeof(float) + 255) & ~(size_t)255;
}

template <bool QUANT, int RT, int RE, int WM = 2, int WN = 2>
__global__ __launch_bounds__(WM* WN * 64) void route_gemm_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ wg, int64_t T,
                                                                int H, int E, int kchunk,
                                                                float* __restrict__ part,
                                                                float* __restrict__ amax_part,
                                                                int32_t* __restrict__ zero, int nzero) {
  constexpr int NW = WM * WN, NT = NW * 64;
  // the top-k step's count rows, cleared here for its atomic adds
  if (zero) {
    const int64_t nthr = (int64_t)gridDim.x * gridDim.y * gridDim.z * NT;
    const int64_t me = (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * NT + threadIdx.x;
    for (int64_t i = me; i < nzero; i += nthr) zero[i] = 0;
  }
  constexpr int STAGE = (RT + RE) * kRRow;
  constexpr int RS = kRLds / STAGE;              // stages
  constexpr int RL = STAGE / 1024 / NW;          // 1 KiB copies per wave per stage
  constexpr int FR = RT / WM / 32, FE = RE / WN / 32;   // fragments per wave
  static_assert(RL * NW * 1024 == STAGE && RS >= 3, "stages");
  static_assert(FR >= 1 && FE >= 1, "wave tile");
  __shared__ __attribute__((aligned(16))) uint8_t smem[RS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / WN, wn = wv - (wv / WN) * WN;
  const int64_t t0 = (int64_t)blockIdx.x * RT;
  const int e0 = blockIdx.y * RE;
  const int64_t rowbytes = (int64_t)H * 2;
  const int nk = kchunk / kRRow;

  // this wave's copies: 1 KiB block q = wv*RL + j holds stage rows 8q..8q+7
  // (rows [0, RT) tokens, then RE experts); lane i copies row 8q + i/8, LDS
  // chunk i%8, which holds logical chunk (i%8) ^ sw(row)
  const uint8_t* src[RL];
#pragma unroll
  for (int j = 0; j < RL; ++j) {
    const int q = wv * RL + j;
    const int srow = q * 8 + (lane >> 3);
    const bool tok = srow < RT;
    const int trow = tok ? srow : srow - RT;
    const int c = (lane & 7) ^ swr<kRRow>(trow);
    int64_t grow;
    const uint8_t* base;
    if (tok) {
      grow = t0 + trow < T ? t0 + trow : T - 1;
      base = reinterpret_cast<const uint8_t*>(x);
    } else {
      grow = e0 + trow < E ? e0 + trow : 0;
      base = reinterpret_cast<const uint8_t*>(wg);
    }
    src[j] = base + grow * rowbytes + (int64_t)blockIdx.z * kchunk + c * 16;
  }
  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % RS) * STAGE;
#pragma unroll
    for (int j = 0; j < RL; ++j)
      __builtin_amdgcn_global_load_lds((glb_void*)(src[j] + kt * kRRow),
                                       (lds_void*)(st + (wv * RL + j) * 1024), 16, 0, 0);
  };
  int lo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r = lane & 31;
    lo[s] = r * kRRow + (((2 * s + (lane >> 5)) ^ swr<kRRow>(r)) << 4);
  }
  // quantisation: TPR threads fold |x| of each stage token row, CPT 16-byte
  // chunks each
  constexpr int TPR = NT / RT, CPT = 8 / TPR;
  static_assert(TPR >= 2 && TPR <= 8 && CPT * TPR == 8, "absmax fold threads per row");
  const int qrow = tid / TPR;
  int qoff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) qoff[i] = qrow * kRRow + (((CPT * (tid % TPR) + i) ^ swr<kRRow>(qrow)) << 4);
  uint32_t amax = 0;   // bf16 magnitude bits

  f32x16 acc[FR][FE];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FE; ++j) acc[i][j] = f32x16{};
#pragma unroll
  for (int p = 0; p < RS - 1; ++p)
    if (p < nk) issue(p);
  for (int kt = 0; kt < nk; ++kt) {
    const int after = nk - 1 - kt < RS - 2 ? nk - 1 - kt : RS - 2;
    wait_vm_stages<RL, RS - 2>(after);
    lds_barrier();
    if (kt + RS - 1 < nk) issue(kt + RS - 1);
    const uint8_t* As = smem + (kt % RS) * STAGE;
    const uint8_t* Bs = As + RT * kRRow;
    u32x4 af[4][FR], bf[4][FE];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int i = 0; i < FR; ++i)
        af[s][i] = *reinterpret_cast<const u32x4*>(As + (wm * (RT / WM) + 32 * i) * kRRow + lo[s]);
#pragma unroll
      for (int j = 0; j < FE; ++j)
        bf[s][j] = *reinterpret_cast<const u32x4*>(Bs + (wn * (RE / WN) + 32 * j) * kRRow + lo[s]);
    }
    if constexpr (QUANT) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(As + qoff[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          amax = max(amax, v[j] & 0x7FFFu);
          amax = max(amax, (v[j] >> 16) & 0x7FFFu);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FE; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[s][i]),
                                                              __builtin_bit_cast(bf16x8, bf[s][j]), acc[i][j], 0, 0,
                                                              0);
  }

#pragma unroll
  for (int j = 0; j < FE; ++j) {
    const int e = e0 + wn * (RE / WN) + 32 * j + (lane & 31);
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t t = t0 + wm * (RT / WM) + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (t < T && e < E) part[((int64_t)blockIdx.z * T + t) * E + e] = acc[i][j][v];
      }
  }
  if constexpr (QUANT) {
    // the TPR threads of a row are adjacent lanes
    amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0xB1, 0xF, 0xF, false));   // lane ^ 1
    if constexpr (TPR >= 4)
      amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x4E, 0xF, 0xF, false));   // lane ^ 2
    if constexpr (TPR == 8)   // quads now uniform: row_half_mirror pairs the two quads of each 8 lanes
      amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x141, 0xF, 0xF, false));
    if (blockIdx.y == 0 && tid % TPR == 0 && t0 + qrow < T)
      amax_part[(int64_t)blockIdx.z * T + t0 + qrow] = __uint_as_float(amax << 16);
  }
}

// One wave: the top-k (and, with quantisation, the int8 codes) of token t.
// Sums the K splits of its logits in a fixed order (ZC splits' loads in
// flight), adds the bias, selects the top-k (by rank from an LDS row when
// E <= 64, else by argmax rounds) and, with quantisation, writes the token's
// codes with the absmax the logits kernel folded (XPF x chunks of the row
// fetched before the selection).  lrow: this wave's 64-float LDS row;
// grow/gscore: its 256- and 64-float rows for the group-limited selection.
template <bool QUANT, bool GROUPED, int XPF, int ZC>
__device__ __forceinline__ void topk_token(int64_t t, const float* __restrict__ part, const float* __restrict__ amax_part, int ks,
                           const float* __restrict__ bias, int64_t T, int E, int k, int H,
                           const uint16_t* __restrict__ x, int32_t* __restrict__ ids, float* __restrict__ w,
                           float* __restrict__ prob, int8_t* __restrict__ xq, float* __restrict__ xs,
                           int n_group, int topk_group, float* lrow, float* grow, float* gscore,
                           int* hist = nullptr) {
  const int lane = threadIdx.x & 63;
  // W8A8, XPF > 0 (small batches, latency-bound): the token's x row (its
  // first XPF*512 values) and its per-split absmax are fetched before the
  // selection, which they do not depend on, so their memory latency overlaps
  // the partial-logit loads.  Large batches keep the registers for occupancy.
  // Every load of this prefetch is issued before the first use of any of
  // them (loads complete in order, so an early use would wait for all).
  constexpr int QPF = QUANT ? XPF : 0;
  constexpr int AMP = QPF >= 8 ? 16 : 1;   // per-split absmax values fetched early
  uint4 xr[QPF > 0 ? QPF : 1];
  float amr[AMP];
  float am = 0.f;
  auto load_amax = [&](int z_begin) {
    for (int z0 = z_begin; z0 < ks; z0 += 8) {
      float a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = z0 + u < ks ? amax_part[(size_t)(z0 + u) * T + t] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) am = fmaxf(am, a[u]);
    }
  };
  if constexpr (QPF > 0) {
    const uint16_t* xrow = x + t * H;
#pragma unroll
    for (int u = 0; u < QPF; ++u)
      if (lane * 8 + u * 512 < H) xr[u] = *reinterpret_cast<const uint4*>(xrow + lane * 8 + u * 512);
#pragma unroll
    for (int u = 0; u < AMP; ++u) amr[u] = u < ks ? amax_part[(size_t)u * T + t] : 0.f;
  }
  // the bias, fetched with the partial logits
  float bv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    bv[j] = (bias && e < E) ? bias[e] : 0.f;
  }
  // the K-split partial logits, ZC splits per batch of loads (one batch, so
  // one memory latency, for up to ZC splits), summed in split order
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < ks; z0 += ZC) {
    float q[4][ZC];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < ZC; ++u) {
        const int e = lane + 64 * j;
        q[j][u] = (e < E && z0 + u < ks) ? part[((size_t)(z0 + u) * T + t) * E + e] : 0.f;
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u0 = 0; u0 < ZC; u0 += 8)
        v[j] += ((q[j][u0] + q[j][u0 + 1]) + (q[j][u0 + 2] + q[j][u0 + 3])) +
                ((q[j][u0 + 4] + q[j][u0 + 5]) + (q[j][u0 + 6] + q[j][u0 + 7]));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? v[j] + bv[j] : -INFINITY;
  }
  if constexpr (GROUPED) {
    wave_grouped_topk_store(v, grow, gscore, E, k, n_group, topk_group, t, ids, w, prob);
  } else if (E <= 64) {
    lrow[lane] = v[0];
    __builtin_amdgcn_wave_barrier();
    wave_topk_rank_store(lrow, E, k, t, ids, w, prob, hist);
  } else {
    wave_topk_store(v, E, k, t, ids, w, prob, hist);
  }
  if constexpr (QUANT) {
    if constexpr (QPF == 0) {
      load_amax(0);
    } else {
#pragma unroll
      for (int u = 0; u < AMP; ++u) am = fmaxf(am, amr[u]);
      load_amax(AMP);   // splits past the first 16, if any
    }
    const float s = row_scale(am);
    const float rs = 1.f / s;
    const bool rok = rs_ok(rs);
    const uint16_t* xrow = x + t * H;
    int8_t* qrow = xq + t * H;
#pragma unroll
    for (int u = 0; u < QPF; ++u) {
      const int h = lane * 8 + u * 512;
      if (h < H) {
        const uint32_t q4[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
        float c[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c[2 * i] = __uint_as_float(q4[i] << 16);
          c[2 * i + 1] = __uint_as_float(q4[i] & 0xFFFF0000u);
        }
        *reinterpret_cast<uint2*>(qrow + h) = quant8(c, s, rs, rok);
      }
    }
    // the rest of a longer row: 4 chunks of 8 values per lane in flight
    for (int h0 = lane * 8 + QPF * 512; h0 < H; h0 += 4 * 512) {
      float c[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (h0 + u * 512 < H) load8(xrow + h0 + u * 512, c[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (h0 + u * 512 < H) *reinterpret_cast<uint2*>(qrow + h0 + u * 512) = quant8(c[u], s, rs, rok);
    }
    if (lane == 0) xs[t] = s;
  }
}

// LAT: a batch small enough that the kernel is one dependent chain per token
// (at most 256 workgroups): fetch all split partials at once; otherwise keep
// registers for occupancy.
// One wave per token, NWV tokens per workgroup.  With whist (NWV = 16 only),
// the workgroup counts its selections per expert in LDS and adds the nonzero
// counts to row blockIdx / hg of whist (integer atomics: the sums are exact
// in any order), so each row holds the counts of hg consecutive workgroups,
// about 1024 slots, the align step's block ([FA-MoE] fusion one: the gate's
// tail does the histogram).  The logits kernel cleared the rows.
// LAT with codes (NWV = 4): the codes do not depend on the selection, only on
// the row's max |x|, which the logits kernel folded, so workgroups past the
// first ntk (the top-k ones) write them, kQuantSpan values of one token row
// each, in parallel with the selection instead of after it in each token's
// wave (decode, T = 16, E = 256, H = 4096: route step 14.8 -> 11.6 us).
constexpr int kQuantSpan = 2048;   // values per code workgroup (256 threads x 8)

template <bool QUANT, bool GROUPED, bool LAT, int NWV>
__global__ __launch_bounds__(NWV * 64) void route_topk_kernel(
    const float* __restrict__ part, const float* __restrict__ amax_part, int ks,
    const float* __restrict__ bias, int64_t T, int E, int k, int H, const uint16_t* __restrict__ x,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ prob, int8_t* __restrict__ xq,
    float* __restrict__ xs, int n_group, int topk_group, int32_t* __restrict__ whist, int hg) {
  static_assert(!GROUPED || NWV == 4, "the group-limited top-k publishes no counts");
  constexpr bool HIST = NWV > 4;
  constexpr bool SPLITQ = QUANT && LAT && NWV == 4;
  __shared__ __attribute__((aligned(16))) float lrow[NWV][64];
  __shared__ __attribute__((aligned(16))) float grow[GROUPED ? NWV : 1][256];
  __shared__ float gscore[GROUPED ? NWV : 1][64];
  __shared__ int hist[HIST ? kMaxE : 1];
  const int wv = threadIdx.x >> 6;
  if constexpr (SPLITQ) {
    const int64_t ntk = (T + NWV - 1) / NWV;
    if ((int64_t)blockIdx.x >= ntk) {
      // code workgroup: token row tq, values [c kQuantSpan, (c + 1) kQuantSpan)
      const int cpr = (H + kQuantSpan - 1) / kQuantSpan;
      const int64_t cb = (int64_t)blockIdx.x - ntk;
      const int64_t tq = cb / cpr;
      const int c = (int)(cb - tq * cpr);
      if (tq >= T) return;
      float am = 0.f;
      for (int z = 0; z < ks; ++z) am = fmaxf(am, amax_part[(size_t)z * T + tq]);
      const float sc = row_scale(am);
      const float rs = 1.f / sc;
      const int h0 = c * kQuantSpan + 8 * (int)threadIdx.x;
      if (h0 < H) {
        float v[8];
        load8(x + tq * H + h0, v);
        *reinterpret_cast<uint2*>(xq + tq * H + h0) = quant8(v, sc, rs, rs_ok(rs));
      }
      if (c == 0 && threadIdx.x == 0) xs[tq] = sc;
      return;
    }
  }
  const int64_t t = (int64_t)blockIdx.x * NWV + wv;
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < E; i += NWV * 64) hist[i] = 0;
    __syncthreads();
  } else {
    if (t >= T) return;
  }
  if (t < T)
    topk_token<QUANT && !SPLITQ, GROUPED, LAT ? 8 : 0, LAT ? 16 : 8>(
        t, part, amax_part, ks, bias, T, E, k, H, x, ids, w, prob, xq, xs, n_group, topk_group, lrow[wv],
        grow[GROUPED ? wv : 0], gscore[GROUPED ? wv : 0], HIST ? hist : nullptr);
  if constexpr (HIST) {
    __syncthreads();
    int32_t* row = whist + (int64_t)(blockIdx.x / hg) * E;
    for (int i = threadIdx.x; i < E; i += NWV * 64)
      if (hist[i] != 0) atomicAdd(&row[i], hist[i]);
  }
}

// ------------------------------------------------------------ kind 3 -----
// E <= 64, bf16: gate, softmax and top-k (and, with quantisation, the int8
// codes) in one kernel, with the logits on chip and x read from memory once.
// A workgroup of NW waves (16, or 8 so that two share a CU) takes
// BM = 16 NW / KQ tokens and every expert over all of H.  Wave (tb, q) owns
// tokens [16 tb, 16 tb + 16) of the block and the q-th of KQ contiguous parts
// of H.  It loads its whole x slice straight
// into registers, all loads issued at once, laid out as the A operand of MFMA
// 16x16x32 bf16 (row = lane % 16, eight K values at 8 (lane / 16) of each
// 32-value substep); the same registers give the int8 codes, made a few
// substeps per stage inside the K loop once the row's max |x| has been
// exchanged through LDS at the first stage.  Wg streams through LDS: a stage
// holds RB / 2 K values of every part for all 64 expert rows (rows past E
// copy row 0), S stages deep, copied straight into LDS by every wave.  Each
// wave accumulates its 16 tokens x 64 experts (four 16 x 16 fragments) over
// its part; the KQ parts are then summed through LDS in part order, the
// bias added, and the top-k taken by argmax rounds, one wave per token.  No
// atomics: deterministic.
constexpr int kFE = 64;   // experts per fused tile

// f(IntC<I>) for I = B, B+1, ..., E-1: a loop whose index is a compile-time
// constant in every iteration (register arrays indexed by it stay registers)
template <int V>
struct IC {
  static constexpr int value = V;
};
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    static_for<B + 1, E>(f);
  }
}

// the part count for H (x slice of at most 512 values per wave, whole
// 32-value substeps, whole stages), or 0 if the fused kernel does not apply
inline int fused_parts(int H) {
  for (int kq = 2; kq <= 8; kq *= 2) {
    const int part = H / kq;
    if (H % kq == 0 && (part == 64 || part == 128 || part == 256 || part == 512)) return kq;
  }
  return 0;
}

template <bool QUANT, int KQ, int NSUB, int NW, int LDSB>
__global__ __launch_bounds__(NW * 64) void route_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, const float* __restrict__ bias, int64_t T,
    int H, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ prob,
    int8_t* __restrict__ xq, float* __restrict__ xs, int32_t* __restrict__ whist) {
  constexpr int BM = 16 * NW / KQ;                 // tokens per workgroup
  constexpr int RB = KQ >= 8 ? 64 : 128;           // stage row bytes
  constexpr int SPS = RB / 64;                     // substeps per stage
  constexpr int NST = NSUB / SPS;                  // stages per K loop
  constexpr int BROWS = kFE * KQ;                  // stage rows: (part, expert)
  constexpr int STAGE = BROWS * RB;
  constexpr int SMAX = LDSB / STAGE;
  // short loops issue every stage before the first wait
  constexpr int S = NST + 1 < SMAX ? (NST + 1 < 2 ? 2 : NST + 1) : SMAX;
  constexpr int L = STAGE / 1024 / NW;             // 1 KiB copies per wave per stage
  constexpr int CPR = RB / 16, RPB = 1024 / RB;
  static_assert(L >= 1 && L * NW * 1024 == STAGE, "copies split evenly over the waves");
  static_assert(NST * SPS == NSUB && S >= 2, "stages");
  // One LDS allocation (with a second LDS object the compiler can no longer
  // tell the stage reads from the in-flight copies and drains every copy
  // before each stage): the stages, which the partial logits [KQ][BM][64]
  // fp32 (whose first plane becomes the logits) reuse after the K loop, then
  // the per-part row maxima of |x| [KQ][BM].
  constexpr int PL_BYTES = BM * kFE * 4 * KQ;
  constexpr int AMX_OFF = S * STAGE > PL_BYTES ? S * STAGE : PL_BYTES;
  constexpr int HIST_OFF = AMX_OFF + (QUANT ? KQ * BM * 4 : 0);
  constexpr int SMEM = HIST_OFF + kFE * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  float* const amx = reinterpret_cast<float*>(smem + AMX_OFF);
  // this workgroup's selections per expert (whist), zeroed before any copy
  // into LDS is in flight
  int* const hist = reinterpret_cast<int*>(smem + HIST_OFF);
  if (threadIdx.x < kFE) hist[threadIdx.x] = 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tb = wv / KQ, q = wv - tb * KQ;
  const int64_t t0 = (int64_t)blockIdx.x * BM;
  const int part = H / KQ;
  const int lr = lane & 15, lk = lane >> 4;

  // x slice: token row t0 + 16 tb + lr, values [q part + 32 s + 8 lk, +8)
  const int64_t trow = t0 + tb * 16 + lr;
  const uint16_t* xrow = x + (trow < T ? trow : T - 1) * (int64_t)H + q * part + 8 * lk;
  u32x4 a[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) a[s] = *reinterpret_cast<const u32x4*>(xrow + 32 * s);

  // Wg copies: this wave's 1 KiB blocks wv * L + j of each stage; lane i
  // copies stage row RPB * blk + i / CPR (row = part * 64 + expert) into LDS
  // chunk i % CPR, which holds logical chunk (i % CPR) ^ sw(row)
  // (byte offsets into Wg, which is at most 256 x 4096 bf16 = 2 MiB)
  uint32_t src[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const int row = (wv * L + j) * RPB + lane / CPR;
    const int qq = row / kFE, e = row - qq * kFE;
    const int c = (lane % CPR) ^ swr<RB>(row);
    src[j] = (uint32_t)((e < E ? e : 0) * H * 2 + qq * part * 2 + c * 16);
  }
  const uint8_t* const wgb = reinterpret_cast<const uint8_t*>(wg);
  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % S) * STAGE;
#pragma unroll
    for (int j = 0; j < L; ++j)
      __builtin_amdgcn_global_load_lds((glb_void*)(wgb + src[j] + kt * RB), (lds_void*)(st + (wv * L + j) * 1024),
                                       16, 0, 0);
  };
  // B fragment of expert block eb at logical chunk c of this wave's part
  int boff[4][SPS];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int ss = 0; ss < SPS; ++ss) {
      const int row = q * kFE + eb * 16 + lr;
      boff[eb][ss] = row * RB + (((4 * ss + lk) ^ swr<RB>(row)) << 4);
    }

  // int8 codes (QUANT): the lane's row max |x| over this wave's part is
  // published at the first stage (the x loads are done by then) and read at
  // the second; the codes of the row's values in the lane's registers are
  // then made and stored a few substeps per stage, overlapping the K loop
  // (after it when the loop has one stage)
  const bool row_ok = trow < T;
  float qs = 1.f, qrs = 1.f;
  bool qrok = true;
  constexpr int QPS = NST > 1 ? (NSUB + NST - 2) / (NST - 1) : NSUB;   // substeps coded per stage
  auto publish_absmax = [&]() {
    uint32_t m = 0;
#pragma unroll
    for (int ss = 0; ss < NSUB; ++ss)
#pragma unroll
      for (int j = 0; j < 4; ++j) m = max(m, max(a[ss][j] & 0x7FFFu, (a[ss][j] >> 16) & 0x7FFFu));
    float mf = __uint_as_float(m << 16);
    mf = fmaxf(mf, lane_xor16(mf));
    mf = fmaxf(mf, lane_xor32(mf));
    if (lk == 0) amx[q * BM + tb * 16 + lr] = mf;
  };
  auto take_scale = [&]() {
    float am = 0.f;
#pragma unroll
    for (int qq = 0; qq < KQ; ++qq) am = fmaxf(am, amx[qq * BM + tb * 16 + lr]);
    qs = row_scale(am);
    qrs = 1.f / qs;
    qrok = rs_ok(qrs);
    if (row_ok && q == 0 && lk == 0) xs[trow] = qs;
  };
  int8_t* const qrow = QUANT ? xq + trow * (int64_t)H + q * part + 8 * lk : nullptr;
  auto store_codes = [&](auto s0c, auto s1c) {
    constexpr int S0 = decltype(s0c)::value;
    constexpr int S1 = decltype(s1c)::value < NSUB ? decltype(s1c)::value : NSUB;
    if (!row_ok) return;
    static_for<S0, S1>([&](auto ssc) {
      constexpr int ss = decltype(ssc)::value;
      uint32_t wd[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float c[4] = {__uint_as_float(a[ss][2 * h] << 16), __uint_as_float(a[ss][2 * h] & 0xFFFF0000u),
                            __uint_as_float(a[ss][2 * h + 1] << 16),
                            __uint_as_float(a[ss][2 * h + 1] & 0xFFFF0000u)};
        wd[h] = quant4(c, qs, qrs, qrok);
      }
      *reinterpret_cast<uint2*>(qrow + 32 * ss) = make_uint2(wd[0], wd[1]);
    });
  };

  f32x4 acc[4];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb) acc[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < NST) issue(p);
  static_for<0, NST>([&](auto ktc) {
    constexpr int kt = decltype(ktc)::value;
    constexpr int after = NST - 1 - kt < S - 2 ? NST - 1 - kt : S - 2;
    wait_vmcnt<L * after>();   // the x loads, issued first, are done too
    if constexpr (QUANT && kt == 0) publish_absmax();
    lds_barrier();
    if constexpr (kt + S - 1 < NST) issue(kt + S - 1);
    if constexpr (QUANT && kt == 1) take_scale();
    if constexpr (QUANT && kt >= 1) store_codes(IC<(kt - 1) * QPS>{}, IC<kt * QPS>{});
    const uint8_t* st = smem + (kt % S) * STAGE;
#pragma unroll
    for (int ss = 0; ss < SPS; ++ss) {
      u32x4 b[4];
#pragma unroll
      for (int eb = 0; eb < 4; ++eb) b[eb] = *reinterpret_cast<const u32x4*>(st + boff[eb][ss]);
#pragma unroll
      for (int eb = 0; eb < 4; ++eb)
        acc[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[kt * SPS + ss]),
                                                          __builtin_bit_cast(bf16x8, b[eb]), acc[eb], 0, 0, 0);
    }
  });
  lds_barrier();   // every wave is done with the stages
  if constexpr (QUANT) {
    if constexpr (NST == 1) {
      take_scale();
      store_codes(IC<0>{}, IC<NSUB>{});
    }
  }

  // partial logits [part][token][expert] in the freed stage memory: lane
  // holds expert 16 eb + lr, tokens 16 tb + 4 lk + i
  float* pl = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int i = 0; i < 4; ++i) pl[(q * BM + tb * 16 + 4 * lk + i) * kFE + eb * 16 + lr] = acc[eb][i];
  __syncthreads();
  // logits = the parts summed in order, plus the bias, in place over the
  // first part's plane (each thread reads and writes its own entries)
  for (int i = tid; i < BM * kFE; i += NW * 64) {
    const int e = i % kFE;
    float v = 0.f;
#pragma unroll
    for (int qq = 0; qq < KQ; ++qq) v += pl[qq * BM * kFE + i];
    pl[i] = e < E ? v + (bias ? bias[e] : 0.f) : -INFINITY;
  }
  __syncthreads();
  const int ntok = (int)(T - t0 < BM ? T - t0 : BM);
  for (int t = wv; t < ntok; t += NW)
    wave_topk64_store(pl[t * kFE + lane], E, k, t0 + t, ids, w, prob, whist ? hist : nullptr);
  if (whist) {
    // publish the workgroup's per-expert selection counts for the align step
    __syncthreads();
    if (threadIdx.x < E) whist[(int64_t)blockIdx.x * E + threadIdx.x] = hist[threadIdx.x];
  }
}

// Route and align fused for small batches (T <= kFusedTopkT): one workgroup
// of sixteen waves takes the tokens' top-k in turn, then the same workgroup
// aligns the T*k slots (block_align.h), reading back the ids its own waves
// wrote (visible after the barrier).  One launch instead of two.
constexpr int kFusedTopkT = 64;

template <bool QUANT, bool GROUPED>
__global__ __launch_bounds__(1024) void route_topk_align_kernel(
    const float* __restrict__ part, const float* __restrict__ amax_part, int ks,
    const float* __restrict__ bias, int64_t T, int E, int k, int H, const uint16_t* __restrict__ x,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ prob, int8_t* __restrict__ xq,
    float* __restrict__ xs, int n_group, int topk_group, const AlignArgs al) {
  __shared__ __attribute__((aligned(16))) float lrow[16][64];
  __shared__ __attribute__((aligned(16))) float grow[GROUPED ? 16 : 1][256];
  __shared__ float gscore[GROUPED ? 16 : 1][64];
  const int wv = threadIdx.x >> 6;
  for (int64_t t = wv; t < T; t += 16)
    // (1024 threads: at most 128 VGPRs, so fewer x chunks held)
    topk_token<QUANT, GROUPED, 2, 8>(t, part, amax_part, ks, bias, T, E, k, H, x, ids, w, prob, xq, xs, n_group,
                                  topk_group, lrow[wv], grow[GROUPED ? wv : 0], gscore[GROUPED ? wv : 0]);
  __syncthreads();
  block_align<16>([&](int64_t s) { return ids[s]; }, T * k, E, al.ebits, al.cap, al.bm, al.max_tiles, al.counts,
                  al.offsets, al.sorted_slot, al.pos, al.tiles, al.num_tiles, al.num_dropped);
}

template <int EP, bool WIDE, typename XT, typename WT>
hipError_t launch_fma(const RoutePlan& p, const void* x, const void* wg, const float* bias,
                      int64_t T, int H, int E, int k, int32_t* ids, float* w, float* prob,
                      int8_t* xq, float* xs, const AlignArgs* al, int32_t* whist, hipStream_t s) {
  const int tb = al ? kFmaTB : p.bt;
  const dim3 grid((unsigned)((T + tb - 1) / tb));
  const dim3 block(64 * p.nw);
  const AlignArgs none{};
#define MOE_FMA(Q, A, TB, NVM)                                                                         \
  route_fma_kernel<EP, WIDE, XT, WT, Q, A, TB, NVM><<<grid, block, 0, s>>>((const XT*)x, (const WT*)wg, bias, \
                                                                           T, H, E, k, ids, w, prob, xq, xs,   \
                                                                           al ? *al : none, whist)
  if (al) {
    if (xq)
      MOE_FMA(true, true, kFmaTB, 64);
    else
      MOE_FMA(false, true, kFmaTB, 64);
  } else if (tb == 16 && T >= 4 * 16 * 256) {
    if (xq)
      MOE_FMA(true, false, 16, 32);
    else
      MOE_FMA(false, false, 16, 32);
  } else if (tb == 16) {
    if (xq)
      MOE_FMA(true, false, 16, 64);
    else
      MOE_FMA(false, false, 16, 64);
  } else if (tb == 4) {
    if (xq)
      MOE_FMA(true, false, 4, 64);
    else
      MOE_FMA(false, false, 4, 64);
  } else {
    if (xq)
      MOE_FMA(true, false, 1, 64);
    else
      MOE_FMA(false, false, 1, 64);
  }
#undef MOE_FMA
  return hipGetLastError();
}

template <int EP, bool WIDE>
hipError_t launch_fma_dt(const RoutePlan& p, const void* x, int xd, const void* wg, int wd,
                         const float* bias, int64_t T, int H, int E, int k, int32_t* ids, float* w,
                         float* prob, int8_t* xq, float* xs, const AlignArgs* al, int32_t* whist, hipStream_t s) {
  if (xd == kF32 && wd == kF32)
    return launch_fma<EP, WIDE, float, float>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, al, whist, s);
  if (xd == kF32 && wd == kBF16)
    return launch_fma<EP, WIDE, float, uint16_t>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, al, whist, s);
  if (xd == kBF16 && wd == kF32)
    return launch_fma<EP, WIDE, uint16_t, float>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, al, whist, s);
  return launch_fma<EP, WIDE, uint16_t, uint16_t>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, al, whist, s);
}

template <bool GROUPED>
hipError_t launch_mfma(const RoutePlan& p, const void* x, const void* wg, const float* bias,
                       int64_t T, int H, int E, int k, int32_t* ids, float* w, float* prob,
                       int8_t* xq, float* xs, void* ws, int n_group, int topk_group, const AlignArgs* al,
                       hipStream_t s, int32_t* whist = nullptr) {
  const uint16_t* xb = (const uint16_t*)x;
  const uint16_t* wb = (const uint16_t*)wg;
  float* part = (float*)ws;
  float* amax_part = (float*)((uint8_t*)ws + route_part_bytes(T, E, p.ks));
  const dim3 grid((unsigned)((T + p.bt - 1) / p.bt), (unsigned)((E + p.be - 1) / p.be), (unsigned)p.ks);
  // with whist: the top-k workgroups add their counts into rows of
  // topk_hist_group(k) workgroups each, which the logits kernel clears
  const int hg = topk_hist_group(k);
  const int nzero = whist ? (int)(((T + kTopkHistTokens - 1) / kTopkHistTokens + hg - 1) / hg) * E : 0;
#define MOE_RG(RT, RE, WM, WN)                                                                                 \
  if (xq)                                                                                                      \
    route_gemm_kernel<true, RT, RE, WM, WN><<<grid, WM * WN * 64, 0, s>>>(xb, wb, T, H, E, 2 * H / p.ks, part,  \
                                                                           amax_part, whist, nzero);            \
  else                                                                                                         \
    route_gemm_kernel<false, RT, RE, WM, WN><<<grid, WM * WN * 64, 0, s>>>(xb, wb, T, H, E, 2 * H / p.ks, part, \
                                                                            amax_part, whist, nzero);
  if (p.bt == 128 && p.nw == 16) {
    MOE_RG(128, 128, 4, 4)
  } else if (p.bt == 128 && p.nw == 8) {
    MOE_RG(128, 128, 2, 4)
  } else if (p.bt == 128) {
    MOE_RG(128, 128, 2, 2)
  } else {
    MOE_RG(64, 64, 2, 2)
  }
#undef MOE_RG
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (al) {
    if (xq)
      route_topk_align_kernel<true, GROUPED><<<1, 1024, 0, s>>>(part, amax_part, p.ks, bias, T, E, k, H, xb, ids, w,
                                                                prob, xq, xs, n_group, topk_group, *al);
    else
      route_topk_align_kernel<false, GROUPED><<<1, 1024, 0, s>>>(part, amax_part, p.ks, bias, T, E, k, H, xb, ids,
                                                                 w, prob, xq, xs, n_group, topk_group, *al);
    return hipGetLastError();
  }
  const bool lat = T <= 4 * 256;
  if constexpr (!GROUPED) {
    if (whist) {
      const dim3 g16((unsigned)((T + kTopkHistTokens - 1) / kTopkHistTokens));
#define MOE_TOPKH(Q, LAT)                                                                                       \
  route_topk_kernel<Q, false, LAT, kTopkHistTokens><<<g16, kTopkHistTokens * 64, 0, s>>>(                       \
      part, amax_part, p.ks, bias, T, E, k, H, xb, ids, w, prob, xq, xs, n_group, topk_group, whist, hg)
      // (with codes the latency form needs more than the 128 VGPRs a wave of
      // a 16-wave workgroup can hold, so it takes the other)
      if (xq)
        MOE_TOPKH(true, false);
      else if (lat)
        MOE_TOPKH(false, true);
      else
        MOE_TOPKH(false, false);
#undef MOE_TOPKH
      return hipGetLastError();
    }
  }
  // (the latency form with codes adds its code workgroups after the top-k ones)
  const dim3 g2((unsigned)((T + 3) / 4));
  const dim3 g2q((unsigned)((T + 3) / 4 + T * ((H + kQuantSpan - 1) / kQuantSpan)));
#define MOE_TOPK(Q, LAT)                                                                              \
  route_topk_kernel<Q, GROUPED, LAT, 4><<<(Q) && (LAT) ? g2q : g2, 256, 0, s>>>(                     \
      part, amax_part, p.ks, bias, T, E, k, H, xb, ids, w, prob, xq, xs, n_group, topk_group, nullptr, 1)
  if (xq && lat)
    MOE_TOPK(true, true);
  else if (xq)
    MOE_TOPK(true, false);
  else if (lat)
    MOE_TOPK(false, true);
  else
    MOE_TOPK(false, false);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace

RoutePlan plan_route(int64_t T, int H, int E, int k, int x_dtype, int wg_dtype, bool fused_ok) {
  (void)k;
  RoutePlan p{-1, 0, 1, 0, 0};
  if (E <= 16) {
    // one 8-value chunk of H per lane: H / 512 waves, Wg slice of 8*E registers
    const int nw = (H + 511) / 512;
    if (nw > (E <= 8 ? 16 : 8)) return p;
    p.kind = 0;
    p.bt = fma_tokens_per_wg(T);
    p.nw = nw;
    return p;
  }
  if (x_dtype != kBF16 || wg_dtype != kBF16 || E % 16 != 0 || E > kMaxE) return p;
  // E <= 64: the fused kernel (logits on chip, x read once) when its grid
  // has at least 64 workgroups; smaller batches split K over more of them
  const int kq = E <= kFE ? fused_parts(H) : 0;
  if (fused_ok && kq > 0 && (T + 256 / kq - 1) / (256 / kq) >= 64) {
    p.kind = 3;
    // 8 waves (two workgroups per CU, so one's x stream overlaps the
    // other's top-k) for parts of H up to a quarter; measured, T = 16384,
    // H = 2048, E = 64: 26.0 -> 25.0 us, with codes 43.1 -> 40.0 us; T = 4096,
    // H = 2048, E = 32: 19.7 -> 14.1 us; at eight parts (H = 4096) 16 waves
    // stay (28.8 against 31.1 us)
    p.nw = kq <= 4 ? 8 : 16;
    p.bt = 16 * p.nw / kq;
    p.be = kFE;
    p.ks = kq;
    return p;
  }
  p.bt = kRT;
  p.be = kRE;
  p.kind = 2;
  int64_t blocks = ((T + kRT - 1) / kRT) * ((E + kRE - 1) / kRE);
  if (blocks >= 256 && E % 128 == 0) {
    // large batch: 128 x 128 tiles, split in K back up to a full grid (at
    // E = 64 the 128 x 64 tile measured no faster than 64 x 64)
    p.bt = 128;
    p.be = 128;
    blocks = ((T + 127) / 128) * (E / 128);
  }
  p.nw = kRouteGemmWaves128;
  // split K while the grid is small: each split keeps >= 2 stages of 64 values
  int ks = 1;
  // (at most 16 splits: the top-k of a small batch loads 16 at once;
  // T=16, E=256: 32 splits 11.2 us, 16 splits 9.6 us, 8 splits 10.6 us)
  while (blocks * ks < 256 && H % (128 * ks) == 0 && H >= 256 * ks && ks < 16) ks *= 2;
  p.ks = ks;
  p.ws_bytes = route_part_bytes(T, E, ks) + (size_t)ks * (size_t)T * sizeof(float);
  return p;
}

namespace {
template <int KQ, int NSUB>
hipError_t launch_fused_n(const RoutePlan& p, const void* x, const void* wg, const float* bias, int64_t T, int H,
                          int E, int k, int32_t* ids, float* w, float* prob, int8_t* xq, float* xs, int32_t* whist,
                          hipStream_t s) {
  const dim3 grid((unsigned)((T + p.bt - 1) / p.bt));
  const uint16_t *xb = (const uint16_t*)x, *wb = (const uint16_t*)wg;
  if (p.nw == 8) {
    // two workgroups per CU: at most 64 KiB of stages each
    if (xq)
      route_fused_kernel<true, KQ, NSUB, 8, 64 * 1024><<<grid, 512, 0, s>>>(xb, wb, bias, T, H, E, k, ids, w, prob,
                                                                           xq, xs, whist);
    else
      route_fused_kernel<false, KQ, NSUB, 8, 64 * 1024><<<grid, 512, 0, s>>>(xb, wb, bias, T, H, E, k, ids, w, prob,
                                                                            xq, xs, whist);
  } else {
    if (xq)
      route_fused_kernel<true, KQ, NSUB, 16, 128 * 1024><<<grid, 1024, 0, s>>>(xb, wb, bias, T, H, E, k, ids, w,
                                                                              prob, xq, xs, whist);
    else
      route_fused_kernel<false, KQ, NSUB, 16, 128 * 1024><<<grid, 1024, 0, s>>>(xb, wb, bias, T, H, E, k, ids, w,
                                                                               prob, xq, xs, whist);
  }
  return hipGetLastError();
}

hipError_t launch_fused(const RoutePlan& p, const void* x, const void* wg, const float* bias, int64_t T, int H,
                        int E, int k, int32_t* ids, float* w, float* prob, int8_t* xq, float* xs, int32_t* whist,
                        hipStream_t s) {
  const int nsub = H / p.ks / 32;
#define MOE_FUSED(KQ, NS) return launch_fused_n<KQ, NS>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, whist, s)
  if (p.ks == 2) {
    if (nsub == 2) MOE_FUSED(2, 2);
    if (nsub == 4) MOE_FUSED(2, 4);
    if (nsub == 8) MOE_FUSED(2, 8);
    if (nsub == 16) MOE_FUSED(2, 16);
  }
  if (p.ks == 4 && nsub == 16) MOE_FUSED(4, 16);
  if (p.ks == 8 && nsub == 16) MOE_FUSED(8, 16);
#undef MOE_FUSED
  return hipErrorInvalidValue;
}

hipError_t route_any(const RoutePlan& p, const void* x, int x_dtype, const void* wg, int wg_dtype,
                     const float* bias, int64_t T, int H, int E, int k, int32_t* ids, float* w, float* prob,
                     int8_t* xq, float* xs, void* ws, const AlignArgs* al, hipStream_t s, int32_t* whist = nullptr) {
  if (p.kind == 3) return launch_fused(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, whist, s);
  if (p.kind == 0) {
#define MOE_FMA_DT(EP, WIDE) \
  return launch_fma_dt<EP, WIDE>(p, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, ids, w, prob, xq, xs, al, whist, s)
    if (E <= 8 && p.nw > 8) MOE_FMA_DT(8, true);
    if (E <= 8) MOE_FMA_DT(8, false);
    MOE_FMA_DT(16, false);
#undef MOE_FMA_DT
  }
  return launch_mfma<false>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, ws, 1, 1, al, s, whist);
}
}  // namespace

hipError_t launch_route(const RoutePlan& p, const void* x, int x_dtype, const void* wg,
                        int wg_dtype, const float* bias, int64_t T, int H, int E, int k,
                        int32_t* ids, float* w, float* prob, int8_t* xq, float* xs, void* ws,
                        hipStream_t s, int32_t* whist) {
  return route_any(p, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, ids, w, prob, xq, xs, ws, nullptr, s,
                   route_publishes_hist(p, T, k) ? whist : nullptr);
}

// (small batches keep the one-workgroup align, whose single wave is faster
// than a workgroup summing the counts: 4.0 vs 5.3 us at 128 slots)
bool route_publishes_hist(const RoutePlan& p, int64_t T, int k) {
  return (p.kind == 0 || p.kind == 2 || p.kind == 3) && T * k >= kAlignFromRouteSlots;
}

int route_hist_tokens(const RoutePlan& p, int k) {
  return p.kind == 2 ? kTopkHistTokens * topk_hist_group(k) : p.bt;
}

int64_t route_hist_groups(const RoutePlan& p, int64_t T, int k) {
  if (!route_publishes_hist(p, T, k) || T <= 0) return 0;
  const int tg = route_hist_tokens(p, k);
  return (T + tg - 1) / tg;
}

size_t route_hist_offset(const RoutePlan& p) { return (p.ws_bytes + 255) & ~(size_t)255; }

size_t route_hist_bytes(const RoutePlan& p, int64_t T, int k, int E) {
  const int64_t ng = route_hist_groups(p, T, k);
  return ng > 0 ? route_hist_offset(p) + (size_t)ng * (size_t)E * 4 : 0;
}

bool route_align_fusable(const RoutePlan& p, int64_t T, int k) {
  // kind 0: one workgroup routes every token; kind 2: one workgroup takes
  // every token's top-k.  Either then aligns the T*k slots itself.
  if (p.kind == 0) return T <= kFmaTB && T * k <= (int64_t)p.nw * 64 * kBlockIds;
  return p.kind == 2 && T <= kFusedTopkT;
}

hipError_t launch_route_align_fused(const RoutePlan& p, const void* x, int x_dtype, const void* wg, int wg_dtype,
                                    const float* bias, int64_t T, int H, int E, int k, int32_t* ids, float* w,
                                    float* prob, int8_t* xq, float* xs, void* ws, int64_t cap, int block_m,
                                    int64_t max_tiles, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                                    int32_t* pos, int32_t* tiles, int32_t* num_tiles, int32_t* num_dropped,
                                    hipStream_t s) {
  if (!route_align_fusable(p, T, k)) return hipErrorInvalidValue;
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  const AlignArgs al{cap, block_m, ebits, max_tiles, counts, offsets, sorted_slot, pos, tiles, num_tiles,
                     num_dropped};
  return route_any(p, x, x_dtype, wg, wg_dtype, bias, T, H, E, k, ids, w, prob, xq, xs, ws, &al, s);
}

hipError_t launch_route_grouped(const RoutePlan& p, const void* x, const void* wg, const float* bias,
                                int64_t T, int H, int E, int k, int n_group, int topk_group,
                                int32_t* ids, float* w, float* prob, int8_t* xq, float* xs, void* ws,
                                hipStream_t s) {
  if (p.kind != 2) return hipErrorInvalidValue;
  return launch_mfma<true>(p, x, wg, bias, T, H, E, k, ids, w, prob, xq, xs, ws, n_group, topk_group, nullptr,
                           s);
}

}  // namespace moe
