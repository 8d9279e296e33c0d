// Align / dispatch: group the T*k (token, choice) slots by expert.
//
// Definition (MoE Router page, 2048ai.net: the token-dispatch section counts
// assignments per destination; the overlap section caps each expert at C and
// sends the excess to the residual path): rank(s) = number of earlier slots
// routed to the same expert; slot s is kept iff rank(s) < C; the kept slots of
// expert e occupy sorted rows offsets[e] .. offsets[e+1)-1 in slot order.
//
// Technique (LightOP page, section 3.2, MoE Align: parallel prefix sum,
// hierarchical atomics, fused map/mask/fill), three launches and no host sync:
//   1. align_hist: each block histograms a contiguous slot range in LDS
//      (LDS atomics only; the counts do not depend on their order).
//   2. align_scan: one block sums the block histograms into per-expert
//      counts, applies the capacity, scans the kept counts into offsets, and
//      writes the GEMM row-tile list.
//   3. align_scatter: each block sums the histograms of the blocks before it
//      (its per-expert base), re-reads its range; four waves take contiguous
//      quarters, count per wave (LDS atomics), scan over waves, and then rank
//      their slots 64 at a time in slot order: the lanes holding the same
//      expert are found with one ballot per bit of the expert id and ranked
//      by popcount of the lower lanes.  Ranks therefore come from an ordered
//      scan, never from the order atomics return in, so every output is
//      deterministic.
// Up to kOneBlockSlots slots the three steps run in one workgroup of up to
// sixteen waves instead (align_one_block_kernel, block_align.h; one wave per
// 512 slots): each wave loads a contiguous share of the ids into registers
// at once, counts them in its own LDS histogram, wave 0 scans, and each wave
// ranks its share from the same registers.  One launch instead of three: at
// these sizes the launches cost more than the work.
#include "block_align.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kAlignThreads = 256;

__global__ __launch_bounds__(kAlignThreads) void align_hist_kernel(const int32_t* __restrict__ ids,
                                                                 int64_t n, int E, int spb,
                                                                 int32_t* __restrict__ bhist) {
  __shared__ int32_t h[kMaxE];
  for (int e = threadIdx.x; e < E; e += kAlignThreads) h[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * spb;
  const int64_t s1 = s0 + spb < n ? s0 + spb : n;
  // eight loads in flight per thread, then their LDS atomics
  for (int64_t c = s0; c < s1; c += 8 * kAlignThreads) {
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t s = c + u * kAlignThreads + threadIdx.x;
      ev[u] = s < s1 ? ids[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if ((unsigned)ev[u] < (unsigned)E) atomicAdd(&h[ev[u]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kAlignThreads) bhist[(size_t)blockIdx.x * E + e] = h[e];
}

// Exclusive scan of one value per thread over the 256-thread block.
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int o = 1; o < kAlignThreads; o <<= 1) {
    const int add = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const int incl = tmp[tid];
  *total = tmp[kAlignThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kAlignThreads) void align_scan_kernel(
    const int32_t* __restrict__ bhist, int nb, int E, int64_t n, int64_t cap, int bm, int64_t max_tiles,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
    int32_t* __restrict__ num_tiles, int32_t* __restrict__ num_dropped) {
  __shared__ int tmp[kAlignThreads];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    // independent loads: the sum is in a fixed order, the loads need not be
    int part[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int b = 0;
    for (; b + 8 <= nb; b += 8)
#pragma unroll
      for (int u = 0; u < 8; ++u) part[u] += bhist[(size_t)(b + u) * E + e];
    for (; b < nb; ++b) part[0] += bhist[(size_t)b * E + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) total += part[u];
    counts[e] = total;
  }
  const int kept = e < E ? (cap > 0 && total > cap ? (int)cap : total) : 0;
  const int ntile = (kept + bm - 1) / bm;
  int n_kept = 0, n_tiles = 0;
  const int off = block_exclusive_scan(kept, tmp, &n_kept);
  const int tbase = block_exclusive_scan(ntile, tmp, &n_tiles);
  if (e < E) offsets[e] = off;
  if (e == 0) {
    offsets[E] = n_kept;
    *num_dropped = (int32_t)(n - n_kept);
    *num_tiles = n_tiles;
  }
  for (int i = 0; i < ntile; ++i) {
    const int rows = kept - i * bm < bm ? kept - i * bm : bm;
    *reinterpret_cast<int4*>(tiles + 4 * (size_t)(tbase + i)) = make_int4(e, off + i * bm, rows, 0);
  }
  for (int64_t q = n_tiles + e; q < max_tiles; q += kAlignThreads)
    *reinterpret_cast<int4*>(tiles + 4 * q) = make_int4(-1, 0, 0, 0);
}

// The ranking pass of one block over slots [s0, s1) (256 threads): four
// waves take contiguous quarters, count them per wave (LDS atomics), turn
// the counts into per-wave bases after the block's own base(e) (the slots of
// expert e before s0), and then rank their slots 64 at a time in slot order:
// the lanes holding the same expert are found with one ballot per bit of the
// expert id and ranked by popcount of the lower lanes.  off(e) is expert e's
// first sorted row, N the kept total; the block also fills its share of the
// unused tail [N, n) of sorted_slot.  wh: 4 * kMaxE ints of LDS, zeroed.
// This wave's quarter of a block's slots [s0, s1), and its ids: eight loads
// in flight per lane, kept for the ranking pass when the quarter fits (the
// usual 1024-slot blocks: four per lane).  Issued before a block's other
// loads, so their latencies overlap.
constexpr int kKeepIds = 8;
struct WaveIds {
  int64_t w0, w1;
  bool kept_regs;
  int idv[kKeepIds];
};
__device__ __forceinline__ WaveIds load_wave_ids(const int32_t* __restrict__ ids, int64_t s0, int64_t s1) {
  WaveIds q;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t sub = (((s1 - s0) + 3) / 4 + 63) / 64 * 64;
  q.w0 = s0 + wv * sub < s1 ? s0 + wv * sub : s1;
  q.w1 = q.w0 + sub < s1 ? q.w0 + sub : s1;
  q.kept_regs = q.w1 - q.w0 <= 64 * kKeepIds;
#pragma unroll
  for (int u = 0; u < kKeepIds; ++u) {
    const int64_t s = q.w0 + 64 * u + lane;
    q.idv[u] = s < q.w1 ? ids[s] : -1;
  }
  return q;
}

template <typename Base, typename Off>
__device__ void scatter_block(const int32_t* __restrict__ ids, int64_t n, int E, int ebits, int64_t s0, int64_t s1,
                              WaveIds& q, Base base, Off off, int64_t N, int64_t cap,
                              int32_t* __restrict__ sorted_slot, int32_t* __restrict__ pos, int32_t* wh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int64_t w0 = q.w0, w1 = q.w1;
  int32_t* my = wh + wv * kMaxE;
  constexpr int KEEP = kKeepIds;
  int* const idv = q.idv;
  const bool kept_regs = q.kept_regs;
  for (int64_t c = w0; c < w1; c += 64 * KEEP) {
    if (c != w0) {   // a quarter longer than the registers hold: later chunks
#pragma unroll
      for (int u = 0; u < KEEP; ++u) {
        const int64_t s = c + 64 * u + lane;
        idv[u] = s < w1 ? ids[s] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < KEEP; ++u)
      if ((unsigned)idv[u] < (unsigned)E) atomicAdd(&my[idv[u]], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) {
    int run = base(e);
    for (int q = 0; q < 4; ++q) {
      const int v = wh[q * kMaxE + e];
      wh[q * kMaxE + e] = run;
      run += v;
    }
  }
  __syncthreads();

  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t b0 = w0; b0 < w1; b0 += 64) {
    const int64_t s = b0 + lane;
    const bool in_range = s < w1;
    int e = -1;
    if (kept_regs) {
      const int u = (int)((b0 - w0) >> 6);   // uniform, < KEEP
#pragma unroll
      for (int v = 0; v < KEEP; ++v)
        if (v == u) e = idv[v];
    } else if (in_range) {
      e = ids[s];
    }
    const bool valid = in_range && (unsigned)e < (unsigned)E;   // out-of-range ids are dropped
    // lanes holding the same expert: agree on every bit of the id
    uint64_t same = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    int rank = 0;
    if (valid) rank = my[e] + __popcll(same & lt);   // every lane reads before any leader adds
    if (valid && (same & lt) == 0) my[e] += __popcll(same);
    if (in_range) {
      const bool kept = valid && (cap <= 0 || rank < cap);
      const int p = kept ? off(e) + rank : -1;
      pos[s] = p;
      if (kept) sorted_slot[p] = (int32_t)s;
    }
  }

  // sentinel fill of the unused tail [N, n) of sorted_slot, split over blocks
  const int64_t f1 = N + s1 < n ? N + s1 : n;
  for (int64_t i = N + s0 + tid; i < f1; i += kAlignThreads) sorted_slot[i] = -1;
}

__global__ __launch_bounds__(kAlignThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int ebits, int spb, const int32_t* __restrict__ bhist,
    const int32_t* __restrict__ offsets, int64_t cap, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ pos) {
  __shared__ int32_t wh[4 * kMaxE];
  for (int i = threadIdx.x; i < 4 * kMaxE; i += kAlignThreads) wh[i] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * spb;
  const int64_t s1 = s0 + spb < n ? s0 + spb : n;
  WaveIds q = load_wave_ids(ids, s0, s1);
  // this block's base for expert e: slots of e in all earlier blocks
  // (independent loads: the sum is exact in any order)
  auto base = [&](int e) {
    int part[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int nbefore = blockIdx.x;
    int b = 0;
    for (; b + 8 <= nbefore; b += 8)
#pragma unroll
      for (int u = 0; u < 8; ++u) part[u] += bhist[(size_t)(b + u) * E + e];
    for (; b < nbefore; ++b) part[0] += bhist[(size_t)b * E + e];
    int run = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) run += part[u];
    return run;
  };
  scatter_block(ids, n, E, ebits, s0, s1, q, base, [&](int e) { return offsets[e]; }, (int64_t)offsets[E], cap,
                sorted_slot, pos, wh);
}

// The whole align step in one launch from the route step's published counts
// (whist[g][E]: the selections of route workgroup g, which covers tokens
// [g tg, (g + 1) tg), slots [g spg, (g + 1) spg) with spg = tg k).  Block b
// takes the slots of route workgroups [b G, (b + 1) G).  Every block sums the
// counts of the route workgroups before its own (its per-expert base) and of
// all of them (the per-expert totals), applies the capacity and scans the
// kept counts into offsets; block 0 also writes counts, offsets, the tile
// list and num_dropped.  Integer sums are exact in any order, so every
// output is deterministic, and equal to the three-launch path's.
// (E <= kMaxE = the block's 256 threads)
__global__ __launch_bounds__(kAlignThreads) void align_route_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int ebits, const int32_t* __restrict__ whist, int64_t ng,
    int G, int spg, int64_t cap, int bm, int64_t max_tiles, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot, int32_t* __restrict__ pos,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles, int32_t* __restrict__ num_dropped) {
  static_assert(kMaxE <= kAlignThreads, "one thread per expert");
  __shared__ int32_t wh[4 * kMaxE];
  __shared__ int32_t pb[kAlignThreads], pt[kAlignThreads];   // per-thread partial base / total
  __shared__ int32_t bb[kMaxE], off_s[kMaxE], wsum[8];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < 4 * kMaxE; i += kAlignThreads) wh[i] = 0;
  const int64_t g0 = (int64_t)blockIdx.x * G;
  const int64_t s0 = g0 * spg;
  const int64_t s1 = s0 + (int64_t)G * spg < n ? s0 + (int64_t)G * spg : n;
  WaveIds q = load_wave_ids(ids, s0, s1);   // in flight while the counts are summed
  // thread (r, e), r < R = 256 / E: route workgroups g = r, r + R, ...,
  // eight independent loads per step
  const int R = kAlignThreads / E;
  int sb = 0, st = 0;
  if (tid < R * E) {
    const int e = tid % E, r = tid / E;
    int64_t g = r;
    for (; g + 7 * R < ng; g += 8 * R) {
      int a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = whist[(g + u * R) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        st += a[u];
        sb += g + u * R < g0 ? a[u] : 0;
      }
    }
    for (; g < ng; g += R) {
      const int a = whist[g * E + e];
      st += a;
      sb += g < g0 ? a : 0;
    }
  }
  pb[tid] = sb;
  pt[tid] = st;
  __syncthreads();
  // thread e < E: its expert's base and total over the R partial sums, the
  // capacity, and the scans over experts of kept rows and row tiles (DPP
  // wave scans, then the four wave totals through LDS)
  int total = 0, b = 0;
  if (tid < E)
    for (int r = 0; r < R; ++r) {
      b += pb[r * E + tid];
      total += pt[r * E + tid];
    }
  const int kept = tid < E ? (cap > 0 && total > cap ? (int)cap : total) : 0;
  const int ntile = (kept + bm - 1) / bm;
  const int ik = wave_incl_scan(kept), it = wave_incl_scan(ntile);
  if (lane == 63) {
    wsum[wv] = ik;
    wsum[4 + wv] = it;
  }
  __syncthreads();
  int pk = 0, ptl = 0, n_kept = 0, n_tiles = 0;
#pragma unroll
  for (int w = 0; w < kAlignThreads / 64; ++w) {
    pk += w < wv ? wsum[w] : 0;
    ptl += w < wv ? wsum[4 + w] : 0;
    n_kept += wsum[w];
    n_tiles += wsum[4 + w];
  }
  const int off = pk + ik - kept, tbase = ptl + it - ntile;
  if (tid < E) {
    bb[tid] = b;
    off_s[tid] = off;
  }
  if (blockIdx.x == 0) {
    if (tid < E) {
      counts[tid] = total;
      offsets[tid] = off;
    }
    if (tid == 0) {
      offsets[E] = n_kept;
      *num_dropped = (int32_t)(n - n_kept);
      *num_tiles = n_tiles;
    }
    for (int i = 0; i < ntile; ++i) {
      const int rows = kept - i * bm < bm ? kept - i * bm : bm;
      *reinterpret_cast<int4*>(tiles + 4 * (size_t)(tbase + i)) = make_int4(tid, off + i * bm, rows, 0);
    }
    for (int64_t i = n_tiles + tid; i < max_tiles; i += kAlignThreads)
      *reinterpret_cast<int4*>(tiles + 4 * i) = make_int4(-1, 0, 0, 0);
  }
  __syncthreads();
  scatter_block(ids, n, E, ebits, s0, s1, q, [&](int e) { return bb[e]; }, [&](int e) { return off_s[e]; },
                (int64_t)n_kept, cap, sorted_slot, pos, wh);
}

// ------------------------------------------------- one-workgroup variant --
constexpr int kOneThreads = 1024;
constexpr int kOneWaves = kOneThreads / 64;
constexpr int64_t kOneBlockSlots = (int64_t)kOneThreads * kBlockIds;

__global__ __launch_bounds__(kOneThreads) void align_one_block_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int ebits, int64_t cap, int bm, int64_t max_tiles,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ pos, int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ num_dropped) {
  block_align<kOneWaves>([&](int64_t s) { return ids[s]; }, n, E, ebits, cap, bm, max_tiles, counts, offsets,
                         sorted_slot, pos, tiles, num_tiles, num_dropped);
}

}  // namespace

int64_t align_max_tiles(int64_t T, int k, int E, int block_m) {
  const int64_t n = T * k;
  return (n + block_m - 1) / block_m + (E < n ? E : n);
}

AlignPlan plan_align(int64_t T, int k, int E) {
  AlignPlan p;
  const int64_t n = T * k;
  if (n <= kOneBlockSlots) {
    p.slots_per_block = (int)(n > 0 ? n : 1);
    p.nblocks = 0;   // one workgroup, no histogram workspace
    p.ws_bytes = 0;
    return p;
  }
  // at most 1024 blocks: each scatter block sums the histograms before it
  p.slots_per_block = 1024;
  if (n > (int64_t)1024 * 1024) p.slots_per_block = (int)(((n + 1023) / 1024 + 255) / 256 * 256);
  p.nblocks = (int)((n + p.slots_per_block - 1) / p.slots_per_block);
  if (p.nblocks < 1) p.nblocks = 1;
  p.ws_bytes = (size_t)p.nblocks * (size_t)E * sizeof(int32_t);
  return p;
}

hipError_t launch_align(const AlignPlan& p, const int32_t* ids, int64_t T, int k, int E, int64_t cap,
                        int block_m, int64_t max_tiles, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_slot, int32_t* pos, int32_t* tiles, int32_t* num_tiles,
                        int32_t* num_dropped, void* ws, hipStream_t s) {
  const int64_t n = T * k;
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  if (p.nblocks == 0) {
    // one wave per 512 slots (8 per lane), 1 to 16 waves: wave 0's scan
    // over the per-wave counts is serial in the wave count, so a small batch
    // (decode: 128 slots) runs in one wave
    const int64_t nw = (n + 511) / 512 < 1 ? 1 : ((n + 511) / 512 > kOneWaves ? kOneWaves : (n + 511) / 512);
    align_one_block_kernel<<<1, (unsigned)(64 * nw), 0, s>>>(ids, n, E, ebits, cap, block_m, max_tiles, counts,
                                                             offsets, sorted_slot, pos, tiles, num_tiles,
                                                             num_dropped);
    return hipGetLastError();
  }
  int32_t* bhist = (int32_t*)ws;
  align_hist_kernel<<<p.nblocks, kAlignThreads, 0, s>>>(ids, n, E, p.slots_per_block, bhist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  align_scan_kernel<<<1, kAlignThreads, 0, s>>>(bhist, p.nblocks, E, n, cap, block_m, max_tiles,
                                                counts, offsets, tiles, num_tiles, num_dropped);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  align_scatter_kernel<<<p.nblocks, kAlignThreads, 0, s>>>(ids, n, E, ebits, p.slots_per_block, bhist,
                                                          offsets, cap, sorted_slot, pos);
  return hipGetLastError();
}

hipError_t launch_align_from_route(const int32_t* ids, const int32_t* whist, int64_t ng, int tg, int64_t T, int k,
                                   int E, int64_t cap, int block_m, int64_t max_tiles, int32_t* counts,
                                   int32_t* offsets, int32_t* sorted_slot, int32_t* pos, int32_t* tiles,
                                   int32_t* num_tiles, int32_t* num_dropped, hipStream_t s) {
  const int64_t n = T * k;
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  // about 256 slots per block, whole route workgroups each (more, shorter
  // blocks: measured 6.6 -> 5.0 us at 8192 slots, E = 8, against 1024)
  const int spg = tg * k;
  int G = 256 / spg;
  if (G < 1) G = 1;
  const int64_t nb = (ng + G - 1) / G;
  align_route_kernel<<<(unsigned)nb, kAlignThreads, 0, s>>>(ids, n, E, ebits, whist, ng, G, spg, cap, block_m,
                                                            max_tiles, counts, offsets, sorted_slot, pos, tiles,
                                                            num_tiles, num_dropped);
  return hipGetLastError();
}

}  // namespace moe
