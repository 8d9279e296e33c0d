// One workgroup aligns n slots: histogram, capacity, offsets, tile list,
// stable ranks (MoE Router page, 2048ai.net: token dispatch counts the
// assignments per destination, the overlap section caps each expert at C;
// LightOP page, section 3.2, MoE Align: prefix sum and fused map/mask/fill).
//
// Definition: rank(s) = number of earlier slots routed to the same expert;
// slot s is kept iff cap <= 0 or rank(s) < cap; the kept slots of expert e
// occupy sorted rows offsets[e] .. offsets[e+1]-1 in slot order.
//
// Each of the workgroup's NW waves takes a contiguous range of the slots, at
// most 64 * kBlockIds of them, and loads its ids into registers at once (one
// memory latency); it counts them in its own LDS histogram; wave 0 turns the
// per-wave counts into per-wave bases (slot order), caps them, scans kept
// rows and row tiles over the experts 64 at a time with wave shuffles, and
// writes counts, offsets and tiles; each wave then ranks its slots 64 at a
// time (lanes with the same expert found by one ballot per id bit, ranked by
// the popcount of the lower lanes).  No atomics decide a position, so every
// output is deterministic.  Requires n <= NW * 64 * kBlockIds.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kBlockIds = 16;   // ids per lane

// outputs and parameters of an align step, for kernels that fuse it
struct AlignArgs {
  int64_t cap;         // <= 0: no capacity
  int bm;              // row-tile height
  int ebits;           // bits of an expert id: ceil(log2 E)
  int64_t max_tiles;   // entries of `tiles`
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slot;
  int32_t* pos;
  int32_t* tiles;
  int32_t* num_tiles;
  int32_t* num_dropped;
};

// load_id(s) returns the expert id of slot s (any integer; ids outside
// [0, E) are dropped).  All threads of the workgroup must call this.
template <int MAXW, typename LoadId>
__device__ void block_align(LoadId load_id, int64_t n, int E, int ebits, int64_t cap, int bm, int64_t max_tiles,
                            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                            int32_t* __restrict__ sorted_slot, int32_t* __restrict__ pos,
                            int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles,
                            int32_t* __restrict__ num_dropped) {
  __shared__ int32_t ba_wh[MAXW * kMaxE];   // per-wave counts, then per-wave bases
  __shared__ int32_t ba_off[kMaxE];
  __shared__ int32_t ba_tot[2];
  const int nt = blockDim.x, nw = nt >> 6;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < nw * kMaxE; i += nt) ba_wh[i] = 0;
  __syncthreads();
  const int64_t sub = ((n + nw - 1) / nw + 63) / 64 * 64;
  const int64_t w0 = (int64_t)wv * sub < n ? (int64_t)wv * sub : n;
  const int64_t w1 = w0 + sub < n ? w0 + sub : n;
  int32_t* my = ba_wh + wv * kMaxE;
  int idv[kBlockIds];
#pragma unroll
  for (int j = 0; j < kBlockIds; ++j) {
    const int64_t s = w0 + 64 * j + lane;
    idv[j] = s < w1 ? load_id(s) : -1;
  }
#pragma unroll
  for (int j = 0; j < kBlockIds; ++j)
    if ((unsigned)idv[j] < (unsigned)E) atomicAdd(&my[idv[j]], 1);   // counts only
  __syncthreads();
  if (wv == 0) {
    int run_k = 0, run_t = 0;
    for (int c = 0; c < E; c += 64) {
      const int e = c + lane;
      int kept = 0, ntile = 0;
      if (e < E) {
        int total = 0;
        for (int q = 0; q < nw; ++q) {
          const int v = ba_wh[q * kMaxE + e];
          ba_wh[q * kMaxE + e] = total;
          total += v;
        }
        counts[e] = total;
        kept = cap > 0 && total > cap ? (int)cap : total;
        ntile = (kept + bm - 1) / bm;
      }
      const int ik = wave_incl_scan(kept), it = wave_incl_scan(ntile);   // inclusive, over the 64 lanes
      const int offv = run_k + ik - kept, tbase = run_t + it - ntile;
      if (e < E) {
        offsets[e] = offv;
        ba_off[e] = offv;
        for (int i = 0; i < ntile; ++i) {
          const int r = kept - i * bm < bm ? kept - i * bm : bm;
          *reinterpret_cast<int4*>(tiles + 4 * (size_t)(tbase + i)) = make_int4(e, offv + i * bm, r, 0);
        }
      }
      run_k += __builtin_amdgcn_readlane(ik, 63);
      run_t += __builtin_amdgcn_readlane(it, 63);
    }
    if (lane == 0) {
      offsets[E] = run_k;
      *num_dropped = (int32_t)(n - run_k);
      *num_tiles = run_t;
      ba_tot[0] = run_k;
      ba_tot[1] = run_t;
    }
  }
  __syncthreads();
  const int n_kept = ba_tot[0], n_tiles = ba_tot[1];
  for (int64_t q = n_tiles + tid; q < max_tiles; q += nt)
    *reinterpret_cast<int4*>(tiles + 4 * q) = make_int4(-1, 0, 0, 0);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < kBlockIds; ++j) {
    if (w0 + 64 * j >= w1) break;   // uniform
    const int64_t s = w0 + 64 * j + lane;
    const bool in_range = s < w1;
    const int ex = idv[j];
    const bool valid = in_range && (unsigned)ex < (unsigned)E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (ex >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    int rank = 0;
    if (valid) rank = my[ex] + __popcll(same & lt);   // every lane reads before any leader adds
    if (valid && (same & lt) == 0) my[ex] += __popcll(same);
    if (in_range) {
      const bool keep = valid && (cap <= 0 || rank < cap);
      const int p = keep ? ba_off[ex] + rank : -1;
      pos[s] = p;
      if (keep) sorted_slot[p] = (int32_t)s;
    }
  }
  for (int64_t i = n_kept + tid; i < n; i += nt) sorted_slot[i] = -1;
}

}  // namespace moe
