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
//    expert, <= BM rows) from the tile list.  The grid is the host-known
//    upper bound on tiles times the N blocks; the workgroups with work are
//    renumbered over the device-side tile count so that they spread evenly
//    over the eight XCDs, consecutive ones (the N blocks of a raster group,
//    then the next row tile) sharing an XCD's L2.
//  * K advances ROWB bytes per stage (64 or 128: 32/64 bf16, 64/128 int8).
//    Stages are copied from global memory straight into LDS with 16-byte
//    direct-to-LDS loads, S stages deep, so no registers stage the tiles;
//    rows are stored with an XOR swizzle of their 16-byte chunks so the
//    MFMA operand reads spread over all LDS banks.
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
//    writes h in bf16 (the activation dtype of the layer) and stores each
//    workgroup's max |h| per row over its columns (one plain store per row
//    and N block, no atomics); a row pass then takes the maximum over the N
//    blocks, quantises the stored h with the per-token rule, and the down
//    GEMM runs int8 MFMA.
//  * W4A16 (LightOP page, section 4.3, INT4 weights with 16-bit
//    activations): weights are int4 codes, two per byte along K (low nibble
//    first), with one fp32 scale per output channel.  B tiles are copied to
//    LDS packed (a quarter of the bf16 bytes); each lane reads its codes for
//    all four K substeps of a stage as one swizzled 16-byte chunk (the MFMA's
//    K slots are reordered alike for A and B), widens each substep's eight
//    codes exactly to bf16 in registers, and the MFMAs are the bf16 ones;
//    the epilogue applies the channel scales (before SwiGLU in the up GEMM).
//  * W4A8 (same section, INT4 weights with INT8 activations): the W8A8 path
//    with the same packed int4 B tiles (half the int8 bytes); each lane reads
//    two swizzled 16-byte chunks per stage and widens each substep's sixteen
//    codes to int8 (nibbles masked into bytes, sign-extended by a multiply
//    that cannot carry, and put back in K order with two byte permutes).
#include <math.h>
#include <stdio.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kI8 = 2;
constexpr int kI4 = 3;
constexpr int kI4A8 = 4;


template <bool I8>
struct Mma;
template <>
struct Mma<false> {
  typedef f32x16 Acc;
  static __device__ __forceinline__ Acc run(const u32x4& a, const u32x4& b, const Acc& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mma<true> {
  typedef i32x16 Acc;
  static __device__ __forceinline__ Acc run(const u32x4& a, const u32x4& b, const Acc& c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                 __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
  }
};

// MFMA 32x32 accumulator element v of lane l sits at row 8*(v/4) + 4*(l/32) + v%4,
// column l%32 of the fragment.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// Eight int4 codes (two per byte, low nibble first, two's complement) to
// eight bf16 values in K order: each code is sign-extended, converted to fp32
// and narrowed, all exactly (|code| <= 8).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 widen_i4(uint32_t w) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = (float)((int32_t)(w << (28 - 8 * j)) >> 28);
    const float hi = (float)((int32_t)(w << (24 - 8 * j)) >> 28);
    const bf16x2 p = {(__bf16)lo, (__bf16)hi};
    r[j] = __builtin_bit_cast(uint32_t, p);
  }
  return r;
}

// Packed int4 B rows in LDS (32 bytes per stage row for bf16 activations, 64
// for int8) hold 2 or 4 16-byte chunks; chunk c of row r is stored at
// c ^ swz4(r), so that the sixteen rows a 16-lane pass reads at one logical
// chunk fall on sixteen distinct 16-byte slots of a 256-byte bank row.
template <bool I8>
__device__ __forceinline__ int swz4(int r) {
  if constexpr (I8) return (r >> 2) & 3;
  return (r >> 3) & 1;
}

// Sixteen int4 codes (8 bytes, as above) to sixteen int8 values in K order.
__device__ __forceinline__ uint32_t sext_nibble_bytes(uint32_t u) {
  // bytes hold 4-bit two's complement values; 8 * 0x1E = 0xF0 stays in its byte
  return u | ((u & 0x08080808u) * 0x1Eu);
}
__device__ __forceinline__ u32x4 widen_i4_i8(uint32_t p0, uint32_t p1) {
  u32x4 r;
  const uint32_t p[2] = {p0, p1};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = sext_nibble_bytes(p[h] & 0x0F0F0F0Fu);          // codes 0, 2, 4, 6
    const uint32_t hi = sext_nibble_bytes((p[h] >> 4) & 0x0F0F0F0Fu);   // codes 1, 3, 5, 7
    // v_perm_b32 selects bytes of {hi, lo}: 0-3 are lo's, 4-7 hi's
    r[2 * h] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    r[2 * h + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
  return r;
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup P runs on
// XCD P % 8).  Renumber them so that consecutive logical ids run on the same
// XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int P, int G) {
  const int q = G >> 3, r = G & 7, x = P & 7, j = P >> 3;
  return x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

template <int N>
struct IntC {
  static constexpr int value = N;
};
// Calls f(IntC<v>) for the runtime value v in [0, MAX] (v is wave-uniform).
template <int MAX, typename F>
__device__ __forceinline__ void dispatch_valid(int v, F&& f) {
  if constexpr (MAX >= 0) {
    if (v == MAX) {
      f(IntC<MAX>{});
      return;
    }
    if constexpr (MAX > 0) dispatch_valid<MAX - 1>(v, f);
  }
}

struct GemmArgs {
  const uint8_t* act;          // up: x or xq [T, H] (rows gathered); down: h or hq [rows, I]
  const uint8_t* w;            // up: w13 [E, 2I, H]; down: w2 [E, H, I]
  const int32_t* sorted_slot;
  const int32_t* tiles;
  const int32_t* num_tiles;
  const float* xs;             // up, W8A8: per-token activation scale
  const float* wscale;         // W8A8: per-output-channel weight scale, [E, 2I] up / [E, H] down
  const float* hs;             // down, W8A8: per-row scale of h
  const float* topk_w;         // down: route weight per slot (NULL: 1)
  void* out;                   // up: h [rows, I] bf16; down: y [rows, H] bf16
  float* rowmax;               // up, W8A8: [n_blocks][max rows] each up workgroup's max |h| of
                               // its rows over its columns (of the bf16-rounded values)
  int rowmax_stride;           // rows of rowmax per N block
                               // (W4A16: wscale as for W8A8, w packed two codes per byte)
  void* partial;               // down, last-round split: raw partial tiles [conc][BM * BN]
  int H, I, k;
  int n_blocks, max_tiles;
  int conc;                    // down: workgroups resident at once (0: no last-round split)
};

// Last-round split (down GEMM).  With conc workgroups resident at once, the
// nwork units run in ceil(nwork / conc) rounds.  When the last round is at
// most half full, each of its units is split into ks K-parts (ks <= conc /
// units, <= 8, >= 2 stages each) so that round fills the machine.  Units
// [0, nmain) run whole; the parts, dispatched after them, write raw partial
// tiles that tail_reduce_kernel sums in part order before the epilogue.
struct TailPlan {
  int nmain, ks;
};
__device__ __forceinline__ TailPlan tail_plan(int nwork, int conc, int nk) {
  TailPlan p{nwork, 1};
  if (conc <= 0 || nwork <= 0) return p;
  const int tail = nwork - ((nwork - 1) / conc) * conc;
  if (2 * tail > conc) return p;
  const int ks = min(min(conc / tail, 8), nk / 2);
  if (ks >= 2) {
    p.nmain = nwork - tail;
    p.ks = ks;
  }
  return p;
}

// unit L0 -> (row tile, N block): groups of GN N blocks, row tiles fastest
template <int GN>
__device__ __forceinline__ int2 raster(int L0, int nt, int n_blocks) {
  const int per_group = nt * GN;
  const int g = L0 / per_group;
  const int rem = L0 - g * per_group;
  const int gs = min(GN, n_blocks - g * GN);
  const int tile = rem / gs;
  return make_int2(tile, g * GN + (rem - tile * gs));
}

// Max of each of 16 values over the 16 lanes of each 16-lane row, by a
// butterfly over lane bits 3, 2, 1, 0 (DPP row_mirror, row_half_mirror,
// quad_perm xor 2 and xor 1; each step's partner differs in that bit): a lane
// keeps the half of its values its bit selects and takes the partner's copy
// of that half.  Lane l returns the max of value l % 16.
template <int S>
__device__ __forceinline__ float bfly16_partner(float v) {
  if constexpr (S == 0) return dpp_f32<0x140>(v);
  else if constexpr (S == 1) return dpp_f32<0x141>(v);
  else if constexpr (S == 2) return dpp_f32<0x4E>(v);
  else return dpp_f32<0xB1>(v);
}
template <int S = 0>
__device__ __forceinline__ float rows_max16x16(float (&m)[16], int lane) {
  if constexpr (S == 4) {
    return m[0];
  } else {
    constexpr int h = 8 >> S;
    const bool up = ((lane >> (3 - S)) & 1) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float send = up ? m[i] : m[i + h];
      const float keep = up ? m[i + h] : m[i];
      m[i] = fmaxf(keep, bfly16_partner<S>(send));
    }
    return rows_max16x16<S + 1>(m, lane);
  }
}

// One BM x BN output tile of one row tile (one expert).  Waves form a WM x WN
// grid; each owns (BM/WM) x (BN/WN) outputs as 32x32 MFMA fragments; with
// four waves per SIMD one wave's MFMAs cover another's copy and LDS waits.
// Raster: groups of GN N blocks; within a group the row tiles run fastest,
// so consecutive workgroups (one XCD) share A rows across GN N blocks and
// B rows across the row tiles of one expert.
//  up:   the B tile stacks BN/2 rows of W1 over the same BN/2 rows of W3, each
//        wave holds matching G and U fragments, and the epilogue writes
//        h = silu(G) * U;
//  down: the B tile is BN rows of W2 and the epilogue writes w_r * acc.
// K advances ROWB bytes per stage.  Stages are copied from
// global memory straight into LDS (16 bytes per lane per instruction, lane i
// landing at 16*i of a 1 KiB block), S stages deep: stage kt+S-1 is in flight
// while stage kt computes, with no staging registers.  Each wave issues the
// same number of copies per stage, waits for its own copies of stage kt with
// an exact vmcnt, and a barrier then publishes them to the workgroup.
// 32-row fragments wholly past the tile's valid rows skip their MFMAs (the
// K loop is specialised on their number), and rows past the valid ones copy
// the tile's first row: their accumulators are never stored (an MFMA output
// row depends only on its A row).
template <bool I8, bool UP, int BM, int BN, int WM, int WN, int S, int ROWB, int GN, bool W4 = false>
__global__ __launch_bounds__(WM* WN * 64)
__attribute__((amdgpu_waves_per_eu(
    (BM / WM) * (BN / WN) <= 128 * 64 && 2 * S * (BM * ROWB + BN * (W4 ? ROWB / 4 : ROWB)) <= 160 * 1024 ? 2
                                                                                                        : 1)))
void gg_kernel(const GemmArgs a) {
  constexpr int NT = WM * WN * 64, NW = WM * WN;
  constexpr int WROWS = BM / WM, FM = WROWS / 32;
  constexpr int WCOLS = BN / WN, NF = WCOLS / 32;
  constexpr int HB = BN / 2, HW = WCOLS / 2;
  constexpr int CPR = ROWB / 16;                     // 16-byte chunks per row
  constexpr int RPB = 1024 / ROWB;                   // rows per 1 KiB copy block
  constexpr int SUB = ROWB / 32;                     // MFMA k-substeps per stage
  // B bytes per row per stage (packed int4: half the int8 bytes, a quarter
  // of the bf16 ones for the same K)
  constexpr int BROWB = W4 ? (I8 ? ROWB / 2 : ROWB / 4) : ROWB;
  constexpr int STAGE = BM * ROWB + BN * BROWB;
  constexpr int EB = I8 ? 1 : 2;
  // 1 KiB copy blocks per stage.  bf16/int8: A and B blocks are split evenly,
  // L per wave.  W4A16: each wave copies LA A blocks, and B block w + NW*j
  // for every j that exists (LB or LB + 1 of them), so each wave's count is
  // a constant of its index and its waits stay exact.
  constexpr int ABLK = BM * ROWB / 1024, BBLK = BN * BROWB / 1024;
  constexpr int NBLK = ABLK + BBLK;
  constexpr int L = W4 ? 1 : NBLK / NW;
  constexpr int LA = ABLK / NW, LB = BBLK / NW, LBR = BBLK % NW;
  static_assert(W4 ? (LA * NW == ABLK && BBLK >= 1 && BBLK * 1024 == BN * BROWB)
                   : (L * NW == NBLK),
                "copies must split evenly over the waves");
  static_assert(S >= 2, "at least two stages");
  static_assert(FM >= 1 && NF >= 1, "wave tile too small");
  // Decode tile (64 rows, whole 128-byte lines per weight row and K step):
  // the weight copies are non-temporal.  Each weight line is read once there,
  // and the streaming hint measured 458 -> 417 us for the decode layer (T =
  // 16, E = 256, k = 8).  Tiles whose weight lines are read by several
  // workgroups, or in two 64-byte halves, keep the default: the same hint
  // made those layers 2-34% slower.
  constexpr int BAUX = (!W4 && BM == 64 && ROWB == 128) ? 2 : 0;
  static_assert(!UP || (NF % 2 == 0), "up needs paired G/U fragments");
  static_assert(S * STAGE <= 160 * 1024, "LDS stages");
  // One LDS allocation: with a second LDS object the compiler can no longer
  // tell the stage reads from the in-flight copies and drains every copy
  // (vmcnt(0)) before each stage.
  __shared__ __attribute__((aligned(16))) uint8_t smem[S * STAGE];
  // per-row epilogue scale (up W8A8: the token's activation scale; down: the
  // route weight, times the row's h scale for W8A8): loaded into a register
  // before the K loop, moved to the freed stage memory after it, so the
  // epilogue does no dependent global loads
  constexpr bool ROWSCALE = (UP && I8) || !UP;
  static_assert(!ROWSCALE || NT >= BM, "one thread per row scale");
  float* row_scale = reinterpret_cast<float*>(smem);

  // The grid covers the host's bound on tiles (plus conc split parts); only
  // the first num_tiles * n_blocks units have work.  The whole units are
  // renumbered over exactly their count, so the real work spreads evenly over
  // the XCDs (renumbering over the whole grid would pile it onto the first
  // few); split parts follow; idle workgroups, dispatched last, exit at once.
  const int nt = __builtin_amdgcn_readfirstlane(*a.num_tiles);
  const int nwork = nt * a.n_blocks;
  const int64_t kbytes = (int64_t)(UP ? a.H : a.I) * EB;
  const int64_t kbytes_b = W4 ? kbytes / (I8 ? 2 : 4) : kbytes;   // a packed int4 weight row
  const int nk_all = (int)(kbytes / ROWB);
  TailPlan tp{nwork, 1};
  if constexpr (!UP) tp = tail_plan(nwork, a.conc, nk_all);
  int L0, part = -1, kb = 0, nk = nk_all;
  if ((int)blockIdx.x < tp.nmain) {
    L0 = xcd_remap(blockIdx.x, tp.nmain);
  } else {
    const int idx = (int)blockIdx.x - tp.nmain;
    if (idx >= (nwork - tp.nmain) * tp.ks) return;
    const int u = idx / tp.ks, z = idx - u * tp.ks;
    L0 = tp.nmain + u;
    kb = (int)((int64_t)nk_all * z / tp.ks);
    nk = (int)((int64_t)nk_all * (z + 1) / tp.ks) - kb;
    part = idx;
  }
  L0 = __builtin_amdgcn_readfirstlane(L0);
  part = __builtin_amdgcn_readfirstlane(part);
  kb = __builtin_amdgcn_readfirstlane(kb);
  nk = __builtin_amdgcn_readfirstlane(nk);
  const int2 tn = raster<GN>(L0, nt, a.n_blocks);
  const int tile = tn.x, nb = tn.y;
  // the tile descriptor is uniform: keep it in scalar registers so every
  // branch on it below is a scalar branch
  const int4 td = reinterpret_cast<const int4*>(a.tiles)[tile];
  const int e = __builtin_amdgcn_readfirstlane(td.x);
  const int r0 = __builtin_amdgcn_readfirstlane(td.y);
  const int rows = __builtin_amdgcn_readfirstlane(td.z);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / WN, wn = wv - (wv / WN) * WN;

  // This wave's copies: block q = wv*L + j; blocks [0, BM/RPB) are A rows,
  // the rest B rows.  Lane i copies row RPB*blk + i/CPR into LDS chunk
  // i%CPR, which holds logical chunk (i%CPR) ^ sw(row).
  const uint8_t* abase = (UP ? a.act : a.act + (int64_t)r0 * kbytes) + (int64_t)kb * ROWB;
  const uint8_t* bbase = a.w + (int64_t)e * (UP ? 2 * a.I : a.H) * kbytes_b + (int64_t)kb * BROWB;
  // A wave whose copy blocks hold only A rows past the tile's valid rows
  // issues no copies at all (those rows are never stored); any other wave
  // issues all of its copies per stage, so its vmcnt waits stay exact.
  bool copies = false;
  // W4A16: this wave's B blocks (wv, wv + NW, ...), and the prefix of its A
  // blocks that hold valid rows: only those are copied, and the per-stage
  // count nva + nbw is what the waits use
  const int nbw = W4 ? LB + (wv < LBR ? 1 : 0) : 0;
  int nva = 0;
  if constexpr (W4) {
    nva = (rows - wv * LA * RPB + RPB - 1) / RPB;
    nva = nva < 0 ? 0 : (nva > LA ? LA : nva);
    copies = nva + nbw > 0;
  } else {
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int q = wv * L + j;
      copies |= q >= BM / RPB || q * RPB < rows;
    }
  }
  auto a_off = [&](int trow) -> uint32_t {
    const int c = (lane % CPR) ^ swr<ROWB>(trow);
    const int r = trow < rows ? trow : 0;
    const uint32_t row = UP ? (uint32_t)(a.sorted_slot[r0 + r] / a.k) : (uint32_t)r;
    return row * (uint32_t)kbytes + c * 16;
  };
  auto b_row = [&](int trow) -> uint32_t {
    if (UP) return (uint32_t)(trow < HB ? nb * HB + trow : a.I + nb * HB + (trow - HB));
    return (uint32_t)(nb * BN + trow);
  };
  constexpr int NG = W4 ? LA + LB + (LBR > 0 ? 1 : 0) : L;
  uint32_t goff[NG];
  if constexpr (W4) {
    // packed B rows are not swizzled: BROWB bytes, lane i copies row
    // i / (BROWB/16), chunk i % (BROWB/16) of its 1 KiB block
    constexpr int CPRB = BROWB / 16, RPBB = 1024 / BROWB;
#pragma unroll
    for (int j = 0; j < LA; ++j) goff[j] = a_off((wv * LA + j) * RPB + lane / CPR);
#pragma unroll
    for (int j = 0; j < NG - LA; ++j) {
      const int qb = wv + NW * j;                      // B block (may not exist)
      const int trow = (qb < BBLK ? qb : 0) * RPBB + lane / CPRB;
      goff[LA + j] = b_row(trow) * (uint32_t)kbytes_b + ((lane % CPRB) ^ swz4<I8>(trow)) * 16;
    }
  } else {
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int q = wv * L + j;
      const bool is_a = q < BM / RPB;                  // uniform
      const int trow = (is_a ? q : q - BM / RPB) * RPB + lane / CPR;
      if (is_a) {
        goff[j] = a_off(trow);
      } else {
        const int c = (lane % CPR) ^ swr<ROWB>(trow);
        goff[j] = b_row(trow) * (uint32_t)kbytes + c * 16;
      }
    }
  }
  auto issue = [&](int kt) {
    if (!copies) return;
    uint8_t* st = smem + (kt % S) * STAGE;
    if constexpr (W4) {
#pragma unroll
      for (int j = 0; j < LA; ++j)
        if (j < nva)
          __builtin_amdgcn_global_load_lds((glb_void*)(abase + (size_t)kt * ROWB + goff[j]),
                                           (lds_void*)(st + (wv * LA + j) * 1024), 16, 0, 0);
#pragma unroll
      for (int j = 0; j < NG - LA; ++j)
        if (j < nbw)
          __builtin_amdgcn_global_load_lds((glb_void*)(bbase + (size_t)kt * BROWB + goff[LA + j]),
                                           (lds_void*)(st + BM * ROWB + (wv + NW * j) * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < L; ++j) {
        const int q = wv * L + j;
        const bool isa = q < BM / RPB;                   // uniform
        const uint8_t* src = (isa ? abase : bbase) + (size_t)kt * ROWB + goff[j];
        if constexpr (BAUX == 0) {
          __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(st + q * 1024), 16, 0, 0);
        } else {
          if (isa)
            __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(st + q * 1024), 16, 0, 0);
          else
            __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(st + q * 1024), 16, 0, BAUX);
        }
      }
    }
  };
  // exact wait for stage kt with `after` later stages in flight
  auto wait_stage = [&](int after) {
    if constexpr (W4) {
      wait_vm_dyn<LA + LB + (LBR > 0 ? 1 : 0), S - 2>(nva + nbw, after);
    } else {
      wait_vm_stages<L, S - 2>(after);
    }
  };

  float rs = 0.f;
  if constexpr (ROWSCALE) {
    if (tid < rows) {
      const int slot = a.sorted_slot[r0 + tid];
      if constexpr (UP) {
        rs = a.xs[slot / a.k];
      } else {
        rs = a.topk_w ? a.topk_w[slot] : 1.f;
        if (I8) rs *= a.hs[r0 + tid];
      }
    }
  }
  // number of this wave's 32-row fragments that hold valid rows (uniform)
  int fmv = (rows - wm * WROWS + 31) / 32;
  fmv = fmv < 0 ? 0 : (fmv > FM ? FM : fmv);

  typename Mma<I8>::Acc acc[FM][NF];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) acc[fm][nf] = typename Mma<I8>::Acc{};

  auto brow_of = [&](int nf) -> int {
    if (UP) return nf < NF / 2 ? wn * HW + nf * 32 : HB + wn * HW + (nf - NF / 2) * 32;
    return wn * WCOLS + nf * 32;
  };
  // fragment rows start at multiples of 32 (the swizzle period), so a lane's
  // address within a fragment depends on the lane and the substep only
  // The MFMA's K slots may be fed in any order that A and B share.  bf16 and
  // int8 tiles: substep s, lane half h takes 16-byte chunk 2s + h of the stage
  // row.  Packed int4 B (W4): half h takes the contiguous half [h/2, (h+1)/2)
  // of the stage's K and substep s its s-th quarter, i.e. A chunk 4h + s, so
  // a lane's packed codes for all substeps are one (bf16) or two (int8)
  // contiguous 16-byte chunks.
  static_assert(!W4 || (ROWB == 128 && SUB == 4), "W4 tiles use 128-byte A rows");
  int lo[SUB];
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    const int r = lane & 31, c = W4 ? 4 * (lane >> 5) + s : 2 * s + (lane >> 5);
    lo[s] = r * ROWB + ((c ^ swr<ROWB>(r)) << 4);
  }

  auto kloop = [&](auto vtag) {
    constexpr int V = decltype(vtag)::value;
#pragma unroll
    for (int p = 0; p < S - 1; ++p)
      if (p < nk) issue(p);
    for (int kt = 0; kt < nk; ++kt) {
      // stages issued after kt: min(S-2, nk-1-kt)
      const int after = nk - 1 - kt < S - 2 ? nk - 1 - kt : S - 2;
      wait_stage(after);
      lds_barrier();
      if (kt + S - 1 < nk) issue(kt + S - 1);
      const uint8_t* As = smem + (kt % S) * STAGE;
      const uint8_t* Bs = As + BM * ROWB;
      if constexpr (V > 0 && W4) {
        // packed B: row (lane % 32), lane half h's codes for all four
        // substeps, one (bf16: 4 bytes per substep) or two (int8: 8 bytes)
        // 16-byte chunks, widened in registers per substep
        constexpr int NCH = I8 ? 2 : 1;
        const int h = lane >> 5, sw = swz4<I8>(lane & 31);
        u32x4 af[SUB][V];
        u32x4 bq[NF][NCH];
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int j = 0; j < NCH; ++j)
            bq[nf][j] = *reinterpret_cast<const u32x4*>(Bs + (brow_of(nf) + (lane & 31)) * BROWB +
                                                        16 * ((NCH * h + j) ^ sw));
#pragma unroll
        for (int s = 0; s < SUB; ++s)
#pragma unroll
          for (int fm = 0; fm < V; ++fm)
            af[s][fm] = *reinterpret_cast<const u32x4*>(As + lo[s] + (wm * WROWS + fm * 32) * ROWB);
#pragma unroll
        for (int s = 0; s < SUB; ++s)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            u32x4 b;
            if constexpr (I8) {
              const u32x4 q = bq[nf][s >> 1];
              const uint32_t w0 = (s & 1) ? q[2] : q[0], w1 = (s & 1) ? q[3] : q[1];
              b = widen_i4_i8(w0, w1);
            } else {
              const u32x4 q = bq[nf][0];
              b = widen_i4(q[s]);
            }
#pragma unroll
            for (int fm = 0; fm < V; ++fm) acc[fm][nf] = Mma<I8>::run(af[s][fm], b, acc[fm][nf]);
          }
      } else if constexpr (V > 0) {
        u32x4 af[SUB][V], bfr[SUB][NF];
        // read order A0, B0..B(NF-1), A1..A(V-1): the first MFMA (A0 x B0)
        // waits for two reads only
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
          af[s][0] = *reinterpret_cast<const u32x4*>(As + lo[s] + (wm * WROWS) * ROWB);
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            bfr[s][nf] = *reinterpret_cast<const u32x4*>(Bs + lo[s] + brow_of(nf) * ROWB);
#pragma unroll
          for (int fm = 1; fm < V; ++fm)
            af[s][fm] = *reinterpret_cast<const u32x4*>(As + lo[s] + (wm * WROWS + fm * 32) * ROWB);
        }
#pragma unroll
        for (int s = 0; s < SUB; ++s)
#pragma unroll
          for (int fm = 0; fm < V; ++fm)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
              acc[fm][nf] = Mma<I8>::run(af[s][fm], bfr[s][nf], acc[fm][nf]);
        // schedule: substep-0 fragment reads, then each later substep's reads
        // spread over the previous substep's MFMAs (LDS latency hidden behind
        // matrix work), then the last substep's MFMAs
        constexpr int R = V + NF, M = V * NF, PER = (M + R - 1) / R;
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
        for (int s = 1; s < SUB; ++s) {
#pragma unroll
          for (int i = 0; i < R; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if constexpr (M - R * PER > 0) __builtin_amdgcn_sched_group_barrier(0x008, M - R * PER, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
      }
    }
  };
  dispatch_valid<FM>(fmv, kloop);
  if constexpr (!UP) {
    if (part >= 0) {
      // a split part: the raw accumulators of the tile's valid rows
      int32_t* pp = reinterpret_cast<int32_t*>(a.partial) + (size_t)part * BM * BN;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (fm >= fmv) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WROWS + fm * 32 + acc_row(v, lane);
          if (row >= rows) continue;
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            // the element by value: __builtin_bit_cast of a vector-element
            // lvalue reads element 0 with this compiler
            int32_t bits;
            if constexpr (I8)
              bits = acc[fm][f][v];
            else
              bits = __float_as_int(acc[fm][f][v]);
            pp[row * BN + wn * WCOLS + f * 32 + (lane & 31)] = bits;
          }
        }
      }
      return;
    }
  }
  if constexpr (ROWSCALE) {
    lds_barrier();   // every wave is done with the stages (all copies have landed)
    if (tid < BM) row_scale[tid] = rs;
    lds_barrier();
  }
  bool fv[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) fv[fm] = fm < fmv;

  if constexpr (UP) {
    // SwiGLU, h = silu(g) * u with g = ag * cg, u = au * cu (ag, au the
    // accumulators; cg, cu the dequantisation: the token's scale times the
    // channel's for W8A8, the channel's for int4 weights, else 1), as
    //   h = (ag * au) * (cg * cu) / (1 + 2^(ag * cg * -log2 e)),
    // one product, one exponential and one (hardware) reciprocal per value.
    // h is stored in bf16.  W8A8 also takes each row's max |h| for the
    // quantisation of h: on the fp32 values, rounded once (rounding to
    // nearest is monotone and symmetric, so max |RN(h_i)| = RN(max |h_i|)).
    constexpr float kNegLog2e = -1.44269504088896341f;
    uint8_t* const hbase = reinterpret_cast<uint8_t*>(a.out) + (int64_t)r0 * a.I * 2;
    float* pm = row_scale + BM;   // [WN][BM] per-wave row maxima (freed stage memory)
    float kg[NF / 2], kgu[NF / 2];
#pragma unroll
    for (int f = 0; f < NF / 2; ++f) {
      const int col = nb * HB + wn * HW + f * 32 + (lane & 31);
      const bool scaled = I8 || W4;
      const float sg = scaled ? a.wscale[(int64_t)e * 2 * a.I + col] : 1.f;
      const float su = scaled ? a.wscale[(int64_t)e * 2 * a.I + a.I + col] : 1.f;
      kg[f] = sg * kNegLog2e;
      kgu[f] = sg * su;
    }
    // Rows v and v + 1 (v even) of a fragment are consecutive rows, and
    // lanes l and l ^ 1 consecutive columns: each lane packs its two rows'
    // bf16 values, swaps the pack with its neighbour, and a byte permute
    // forms one row's two columns, row v on the even lane, row v + 1 on the
    // odd one: one 32-bit store per two values.
    const bool odd = (lane & 1) != 0;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (!fv[fm]) continue;
      float xr[16], mv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        xr[v] = I8 ? row_scale[wm * WROWS + fm * 32 + acc_row(v, lane)] : 1.f;
        mv[v] = 0.f;
      }
      // this lane's store row for v = 0 (even lanes) or 1 (odd lanes)
      const int rl = wm * WROWS + fm * 32 + 4 * (lane >> 5) + (odd ? 1 : 0);
#pragma unroll
      for (int f = 0; f < NF / 2; ++f) {
        const int colp = (nb * HB + wn * HW + f * 32 + (lane & 31)) & ~1;
        // element offset of this lane's store for v = 0; row v adds a
        // wave-uniform multiple of I
        uint32_t obase = (uint32_t)(rl * a.I + colp);
        // (kept opaque so the compiler does not fold the row offsets back
        // into one 32-bit multiply per store)
        asm volatile("" : "+v"(obase));
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          float hh[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float ag = (float)acc[fm][f][v + j], au = (float)acc[fm][NF / 2 + f][v + j];
            const float t = I8 ? ag * (xr[v + j] * kg[f]) : ag * kg[f];
            const float q = I8 ? (ag * au) * (xr[v + j] * xr[v + j] * kgu[f])
                               : ((W4 ? ag * au * kgu[f] : ag * au));
            hh[j] = q * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(t));
            if constexpr (I8) mv[v + j] = fmaxf(mv[v + j], fabsf(hh[j]));
          }
          const uint32_t mine = pack_bf16x2(hh[0], hh[1]);
          const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp((int)mine, (int)mine, 0xB1, 0xF, 0xF, false);
          const uint32_t pair = __builtin_amdgcn_perm(other, mine, sel);
          const int dv = 8 * (v >> 2) + (v & 3);   // unrolled: a constant
          if (rl + dv < rows)
            *reinterpret_cast<uint32_t*>(hbase + (obase + (uint32_t)(dv * a.I)) * 2u) = pair;
        }
      }
      if constexpr (I8) {
        // the 16 rows' maxima over the 32 columns of each half-wave at once:
        // lane l ends with row v = l % 16 over its 16-lane row, the other
        // 16-lane row of the half is folded in; lanes 0-15 and 32-47 hold the
        // fragment's 32 rows
        const int v = lane & 15;
        const float r16 = rows_max16x16(mv, lane);
        const float m = fmaxf(r16, lane_xor16(r16));
        const int row = wm * WROWS + fm * 32 + acc_row(v, lane);
        if ((lane & 16) == 0) pm[wn * BM + row] = __uint_as_float(f32_to_bf16_bits(m) << 16);
      }
    }
    if constexpr (I8) {
      static_assert((1 + WN) * BM * 4 <= S * STAGE, "row scales and per-wave row maxima fit the stages");
      // the workgroup's row maxima over its columns: one plain store per row
      // (the quantisation step takes the maximum over the N blocks)
      lds_barrier();
      if (tid < rows) {
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < WN; ++q) m = fmaxf(m, pm[q * BM + tid]);
        a.rowmax[(int64_t)nb * a.rowmax_stride + r0 + tid] = m;
      }
    }
  } else {
    // y = acc * channel scale * row scale, one bf16 rounding, stored two
    // columns per 32-bit store as in the up epilogue (rows v and v + 1 of a
    // fragment packed per lane, swapped with lane l ^ 1, byte-permuted)
    uint8_t* const ybase = reinterpret_cast<uint8_t*>(a.out) + (int64_t)r0 * a.H * 2;
    float sc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
      sc[f] = (I8 || W4) ? a.wscale[(int64_t)e * a.H + nb * BN + wn * WCOLS + f * 32 + (lane & 31)] : 1.f;
    const bool odd = (lane & 1) != 0;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (!fv[fm]) continue;
      float wr[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) wr[v] = row_scale[wm * WROWS + fm * 32 + acc_row(v, lane)];
      // this lane's store row for v = 0 (even lanes) or 1 (odd lanes)
      const int rl = wm * WROWS + fm * 32 + 4 * (lane >> 5) + (odd ? 1 : 0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int colp = (nb * BN + wn * WCOLS + f * 32 + (lane & 31)) & ~1;
        uint32_t obase = (uint32_t)(rl * a.H + colp);
        // (kept opaque so the compiler does not fold the row offsets back
        // into one 32-bit multiply per store)
        asm volatile("" : "+v"(obase));
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float y0 = (float)acc[fm][f][v] * sc[f] * wr[v];
          const float y1 = (float)acc[fm][f][v + 1] * sc[f] * wr[v + 1];
          const uint32_t mine = pack_bf16x2(y0, y1);
          const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp((int)mine, (int)mine, 0xB1, 0xF, 0xF, false);
          const uint32_t pair = __builtin_amdgcn_perm(other, mine, sel);
          const int dv = 8 * (v >> 2) + (v & 3);   // unrolled: a constant
          if (rl + dv < rows)
            *reinterpret_cast<uint32_t*>(ybase + (obase + (uint32_t)(dv * a.H)) * 2u) = pair;
        }
      }
    }
  }
}

// ------------------------------------------------- last-round split sum ---
// Sums the ks partial tiles of each split unit in part order (int32 exactly
// for W8A8) and applies the down epilogue: y = acc * channel scale * row
// scale, one bf16 rounding.  8 rows per 256-thread block, 8 columns per thread.
template <bool I8, int BM, int BN, int ROWB, int GN>
__global__ __launch_bounds__(256) void tail_reduce_kernel(const GemmArgs a) {
  constexpr int EB = I8 ? 1 : 2;
  const int nt = *a.num_tiles;
  const int nwork = nt * a.n_blocks;
  const TailPlan tp = tail_plan(nwork, a.conc, (int)((int64_t)a.I * EB / ROWB));
  const int u = blockIdx.x / (BM / 8);
  if (u >= nwork - tp.nmain) return;
  const int2 tn = raster<GN>(tp.nmain + u, nt, a.n_blocks);
  const int4 td = reinterpret_cast<const int4*>(a.tiles)[tn.x];
  const int row = (blockIdx.x - u * (BM / 8)) * 8 + (threadIdx.x >> 5);
  if (row >= td.z) return;
  const int c = (threadIdx.x & 31) * 8;
  const int32_t* pp = reinterpret_cast<const int32_t*>(a.partial) + (size_t)u * tp.ks * BM * BN + row * BN + c;
  float acc[8];
  if constexpr (I8) {
    int32_t s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int z = 0; z < tp.ks; ++z) {
      const i32x4 p0 = *reinterpret_cast<const i32x4*>(pp + (size_t)z * BM * BN);
      const i32x4 p1 = *reinterpret_cast<const i32x4*>(pp + (size_t)z * BM * BN + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] += p0[i];
        s[4 + i] += p1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (float)s[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int z = 0; z < tp.ks; ++z) {
      float v[8];
      load8(reinterpret_cast<const float*>(pp + (size_t)z * BM * BN), v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
  }
  const int r = td.y + row;
  float wr = a.topk_w ? a.topk_w[a.sorted_slot[r]] : 1.f;
  if (I8) wr *= a.hs[r];
  const int col = tn.y * BN + c;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = acc[i] * (I8 ? a.wscale[(int64_t)td.x * a.H + col + i] : 1.f) * wr;
  store8(reinterpret_cast<uint16_t*>(a.out) + (int64_t)r * a.H + col, o);
}

// ----------------------------------------------------- W8A8 h quantise ---
// One wave per sorted row: s = max|h| / 127 (1 if 0), q = round-half-even(h / s)
// clamped to [-128, 127]; fp32 IEEE arithmetic.  The tile list covers rows
// [0, N) in order, so N is the end of the last tile; waves past it exit.
__global__ __launch_bounds__(256) void quant_h_kernel(const uint16_t* __restrict__ h,
                                                      const float* __restrict__ rowmax, int nparts,
                                                      int64_t stride, const int32_t* __restrict__ tiles,
                                                      const int32_t* __restrict__ num_tiles, int I,
                                                      int8_t* __restrict__ hq, float* __restrict__ hs) {
  const int nt = *num_tiles;
  if (nt <= 0) return;
  const int4 last = reinterpret_cast<const int4*>(tiles)[nt - 1];
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= (int64_t)last.y + last.z) return;
  const int lane = threadIdx.x & 63;
  // the row's max |h|: the up workgroups' partial maxima, one per N block
  float am = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += 64)
    am = fmaxf(am, wave_max(p0 + lane < nparts ? rowmax[(int64_t)(p0 + lane) * stride + r] : 0.f));
  const float s = am == 0.f ? 1.f : am / 127.f;
  const float rs = 1.f / s;
  for (int c = lane * 8; c < I; c += 512) {
    float v[8];
    load8(h + r * I + c, v);
    uint32_t b[2] = {0u, 0u};
#pragma unroll
    for (int q = 0; q < 8; ++q) b[q >> 2] |= (uint32_t)(quant_code(v[q], s, rs) & 0xFF) << (8 * (q & 3));
    *reinterpret_cast<uint2*>(hq + r * I + c) = make_uint2(b[0], b[1]);
  }
  if (lane == 0) hs[r] = s;
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
  // P chunks of 32 K values in flight in registers: the chunk loads are
  // latency-bound at these sizes, so each chunk is loaded P chunks ahead of
  // its use (slot j of the ring is chunk c0 + j, a compile-time index)
  constexpr int P = 4;
  const int nk = K / 32;
  float4 ra[P], rg[P], ru[P];
  auto load = [&](int c, float4& va, float4& vg, float4& vu) {
    va = lval ? *reinterpret_cast<const float4*>(arow + c * 32 + lc) : make_float4(0, 0, 0, 0);
    vg = *reinterpret_cast<const float4*>(grow + c * 32 + lc);
    if (UP) vu = *reinterpret_cast<const float4*>(urow + c * 32 + lc);
  };
#pragma unroll
  for (int j = 0; j < P; ++j)
    if (j < nk) load(j, ra[j], rg[j], ru[j]);
  for (int c0 = 0; c0 < nk; c0 += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int c = c0 + j;
      if (c >= nk) break;
      As[lr][lc] = ra[j].x; As[lr][lc + 1] = ra[j].y; As[lr][lc + 2] = ra[j].z; As[lr][lc + 3] = ra[j].w;
      Bg[lr][lc] = rg[j].x; Bg[lr][lc + 1] = rg[j].y; Bg[lr][lc + 2] = rg[j].z; Bg[lr][lc + 3] = rg[j].w;
      if (UP) {
        Bu[lr][lc] = ru[j].x; Bu[lr][lc + 1] = ru[j].y; Bu[lr][lc + 2] = ru[j].z; Bu[lr][lc + 3] = ru[j].w;
      }
      if (c + P < nk) load(c + P, ra[j], rg[j], ru[j]);
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
  float* rowmax;   // W8A8: [parts][n] partial row maxima of |h|, one row block per up N block
  int8_t* hq;
  float* hs;
  void* partial;   // down, last-round split
};

// the down GEMM's last-round split is used by the prefill tile (variant 0):
// at most kTailParts partial 256 x 256 tiles of 4 bytes
constexpr int kTailParts = 256;
constexpr size_t kTailBytes = (size_t)kTailParts * 256 * 256 * 4;

// workgroups resident at once for the one-per-CU prefill tile: the device's
// compute units, capped at kTailParts (queried once per device)
int resident_tiles() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  n = n < kTailParts ? n : kTailParts;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  return n;
}

struct Variant {
  int bm, bn, wm, wn, stages, rowb, gn;
};
// Rows: tile family (BN) by the divisibility of I (up) or H (down); columns:
// prefill (256 x BN, 16 waves of 64 x 64 where BN allows, 128-byte stage rows:
// every 1 KiB copy is 8 whole cache lines; raster groups of 4 N blocks up, 2
// down, measured best), mid
// (one 256-row tile per expert: 4 stages of 64-byte rows, groups of 8 N
// blocks so the expert's rows are shared by more of them), decode (64 x BN:
// weight streaming; for BN = 256 two stages of 128-byte rows, 80 KiB of LDS,
// so two workgroups share a CU and one streams while the other waits, and
// raster groups over all N blocks; measured 6% faster per layer than one
// workgroup per CU with six 64-byte stages).  Where a family has no distinct
// mid tile the prefill one is reused (entries 4 up, 7 down).
constexpr Variant kUpVar[] = {{256, 256, 4, 4, 2, 128, 4}, {256, 256, 4, 4, 4, 64, 8},
                              {64, 256, 1, 4, 2, 128, 16},  {256, 128, 2, 2, 3, 128, 8},
                              {256, 128, 2, 2, 3, 128, 8},  {64, 128, 1, 2, 6, 64, 8}};
constexpr Variant kDownVar[] = {{256, 256, 4, 4, 2, 128, 2}, {256, 256, 4, 4, 4, 64, 8},
                                {64, 256, 1, 4, 2, 128, 16},  {256, 128, 2, 2, 3, 128, 8},
                                {256, 128, 1, 4, 4, 64, 8},   {64, 128, 1, 4, 6, 64, 8},
                                {256, 64, 2, 2, 3, 128, 8},   {256, 64, 2, 2, 3, 128, 8},
                                {64, 64, 1, 2, 6, 64, 8}};

// W4A16 tiles, three per N family (BN = 256, 128, 64): prefill, mid, decode.
// Packed B stages are a quarter of the bf16 ones and each B fragment is
// widened by every wave that uses it, so waves own 128 x 64 (two waves share
// a fragment in the prefill tile, one in the others).  All stages are
// 128-byte A rows (64 values of K), which halves the barriers per byte of
// weights against 64-byte rows.  Mid tiles are 128 rows (one per expert at
// ~128 rows); decode tiles are 64 rows with small stages, so several
// workgroups share a CU: at decode the K loop is latency-bound and more
// independent workgroups stream faster than one deep pipeline (measured);
// for BN = 256 three stages and raster groups over all N blocks measured 3-5%
// faster per layer than two stages in groups of 8.  Prefill and mid tiles
// take two stages (with them two mid workgroups share a CU: the W4A8 one's
// three stages held a CU alone), except the bf16 prefill down GEMM, which
// keeps three (measured per
// layer: fine-grained W4A8 -15%, W4A16 -3.5%; skewed W4A8 -6%; Mixtral W4A16
// up -1.5%, its down +4% with two).
constexpr Variant kUpVarW4[] = {{256, 256, 2, 4, 2, 128, 4}, {128, 256, 1, 4, 2, 128, 4},
                                {64, 256, 1, 4, 3, 128, 16}, {256, 128, 2, 2, 3, 128, 8},
                                {128, 128, 1, 2, 3, 128, 8}, {64, 128, 1, 2, 3, 128, 8}};
constexpr Variant kDownVarW4[] = {{256, 256, 2, 4, 3, 128, 2}, {128, 256, 1, 4, 2, 128, 4},
                                  {64, 256, 1, 4, 3, 128, 16}, {256, 128, 2, 2, 3, 128, 8},
                                  {128, 128, 1, 2, 3, 128, 8}, {64, 128, 1, 2, 3, 128, 8},
                                  {256, 64, 2, 2, 3, 128, 8},  {128, 64, 1, 2, 3, 128, 8},
                                  {64, 64, 1, 2, 3, 128, 8},
                                  {256, 256, 2, 4, 2, 128, 2}};   // W4A8 prefill (entry 9)

// the up GEMM's N blocks (each writes one partial row maximum per row of h)
int up_parts(int I, int w_dtype, int up_var) {
  const int bn = (w_dtype == kI4 || w_dtype == kI4A8 ? kUpVarW4 : kUpVar)[up_var].bn;
  return I / (bn / 2);
}

FfnBufs carve_ffn(void* ws, int64_t n, int I, int w_dtype, int up_var, int down_var) {
  uint8_t* wsb = (uint8_t*)ws;
  FfnBufs b{wsb, nullptr, nullptr, nullptr, nullptr};
  const bool a8 = w_dtype == kI8 || w_dtype == kI4A8;   // int8 activations: bf16 h, then hq
  size_t off = align256((size_t)n * I * (w_dtype == kF32 ? 4 : 2));
  if (a8) {
    b.rowmax = (float*)(wsb + off);
    off += align256((size_t)n * 4 * up_parts(I, w_dtype, up_var));
    b.hq = (int8_t*)(wsb + off);
    off += align256((size_t)n * I);
    b.hs = (float*)(wsb + off);
    off += align256((size_t)n * 4);
  }
  if ((w_dtype == kBF16 || w_dtype == kI8) && down_var == 0) b.partial = wsb + off;
  return b;
}

#define MOE_GG_CASE(IDX, BM, BN, WM, WN, S, R, G) \
  case IDX:                                       \
    gg_kernel<I8, UP, BM, BN, WM, WN, S, R, G><<<grid, WM * WN * 64, 0, s>>>(a); \
    break;

template <bool I8, bool UP>
hipError_t launch_gg(int var, const GemmArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)a.max_tiles * (unsigned)a.n_blocks + (unsigned)a.conc;
  if constexpr (UP) {
    switch (var) {
      MOE_GG_CASE(0, 256, 256, 4, 4, 2, 128, 4)
      MOE_GG_CASE(1, 256, 256, 4, 4, 4, 64, 8)
      MOE_GG_CASE(2, 64, 256, 1, 4, 2, 128, 16)
      MOE_GG_CASE(3, 256, 128, 2, 2, 3, 128, 8)
      MOE_GG_CASE(5, 64, 128, 1, 2, 6, 64, 8)
      default:
        return hipErrorInvalidValue;
    }
  } else {
    switch (var) {
      MOE_GG_CASE(0, 256, 256, 4, 4, 2, 128, 2)
      MOE_GG_CASE(1, 256, 256, 4, 4, 4, 64, 8)
      MOE_GG_CASE(2, 64, 256, 1, 4, 2, 128, 16)
      MOE_GG_CASE(3, 256, 128, 2, 2, 3, 128, 8)
      MOE_GG_CASE(4, 256, 128, 1, 4, 4, 64, 8)
      MOE_GG_CASE(5, 64, 128, 1, 4, 6, 64, 8)
      MOE_GG_CASE(6, 256, 64, 2, 2, 3, 128, 8)
      MOE_GG_CASE(8, 64, 64, 1, 2, 6, 64, 8)
      default:
        return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}
#undef MOE_GG_CASE

#define MOE_GG4_CASE(IDX, BM, BN, WM, WN, S, R, G) \
  case IDX:                                        \
    gg_kernel<I8, UP, BM, BN, WM, WN, S, R, G, true><<<grid, WM * WN * 64, 0, s>>>(a); \
    break;

template <bool I8, bool UP>
hipError_t launch_gg_w4(int var, const GemmArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)a.max_tiles * (unsigned)a.n_blocks;
  if constexpr (UP) {
    switch (var) {
      MOE_GG4_CASE(0, 256, 256, 2, 4, 2, 128, 4)
      MOE_GG4_CASE(1, 128, 256, 1, 4, 2, 128, 4)
      MOE_GG4_CASE(2, 64, 256, 1, 4, 3, 128, 16)
      MOE_GG4_CASE(3, 256, 128, 2, 2, 3, 128, 8)
      MOE_GG4_CASE(4, 128, 128, 1, 2, 3, 128, 8)
      MOE_GG4_CASE(5, 64, 128, 1, 2, 3, 128, 8)
      default:
        return hipErrorInvalidValue;
    }
  } else {
    switch (var) {
      MOE_GG4_CASE(0, 256, 256, 2, 4, 3, 128, 2)
      MOE_GG4_CASE(1, 128, 256, 1, 4, 2, 128, 4)
      MOE_GG4_CASE(2, 64, 256, 1, 4, 3, 128, 16)
      MOE_GG4_CASE(3, 256, 128, 2, 2, 3, 128, 8)
      MOE_GG4_CASE(4, 128, 128, 1, 2, 3, 128, 8)
      MOE_GG4_CASE(5, 64, 128, 1, 2, 3, 128, 8)
      MOE_GG4_CASE(6, 256, 64, 2, 2, 3, 128, 8)
      MOE_GG4_CASE(7, 128, 64, 1, 2, 3, 128, 8)
      MOE_GG4_CASE(8, 64, 64, 1, 2, 3, 128, 8)
      MOE_GG4_CASE(9, 256, 256, 2, 4, 2, 128, 2)
      default:
        return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}
#undef MOE_GG4_CASE

template <bool I8, bool W4>
hipError_t launch_up(const FfnPlan& p, const void* act, const float* xs, const void* w13,
                     const float* s13, const int32_t* sorted_slot, const int32_t* tiles,
                     const int32_t* num_tiles, int64_t T, int H, int I, int k, const FfnBufs& b,
                     hipStream_t s) {
  GemmArgs a{};
  a.act = (const uint8_t*)act;
  a.w = (const uint8_t*)w13;
  a.sorted_slot = sorted_slot;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.xs = xs;
  a.wscale = s13;
  a.out = b.h;
  a.rowmax = b.rowmax;
  a.rowmax_stride = (int)(T * k);
  a.H = H;
  a.I = I;
  a.k = k;
  a.n_blocks = I / ((W4 ? kUpVarW4 : kUpVar)[p.up_var].bn / 2);
  a.max_tiles = (int)p.max_tiles;
  if constexpr (W4) return launch_gg_w4<I8, true>(p.up_var, a, s);
  return launch_gg<I8, true>(p.up_var, a, s);
}

template <bool I8, bool W4>
hipError_t launch_down(const FfnPlan& p, const void* w2, const float* s2, const int32_t* sorted_slot,
                       const int32_t* tiles, const int32_t* num_tiles, const float* topk_w, int64_t rows,
                       int H, int I, void* y, const FfnBufs& b, hipStream_t s) {
  if (I8)
    quant_h_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(
        (const uint16_t*)b.h, b.rowmax, up_parts(I, W4 ? kI4A8 : kI8, p.up_var), rows, tiles, num_tiles, I,
        b.hq, b.hs);
  GemmArgs a{};
  a.act = I8 ? (const uint8_t*)b.hq : (const uint8_t*)b.h;
  a.w = (const uint8_t*)w2;
  a.sorted_slot = sorted_slot;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.wscale = s2;
  a.hs = b.hs;
  a.topk_w = topk_w;
  a.out = y;
  a.H = H;
  a.I = I;
  a.k = 1;
  a.n_blocks = H / ((W4 ? kDownVarW4 : kDownVar)[p.down_var].bn);
  a.max_tiles = (int)p.max_tiles;
  if constexpr (W4) return launch_gg_w4<I8, false>(p.down_var, a, s);
  a.partial = b.partial;
  a.conc = (p.down_var == 0 && b.partial) ? resident_tiles() : 0;
  hipError_t err = launch_gg<I8, false>(p.down_var, a, s);
  if (err != hipSuccess || a.conc == 0) return err;
  // variant 0: 256 x 256, 128-byte rows, raster groups of 2
  tail_reduce_kernel<I8, 256, 256, 128, 2><<<(unsigned)(a.conc / 2) * (256 / 8), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

namespace {
// int4 packing (offline weight preparation for W4A16): 16 codes per thread,
// byte j of the output holds code 2j in its low nibble and code 2j+1 in its
// high nibble.
__global__ __launch_bounds__(256) void pack_i4_kernel(const int8_t* __restrict__ codes, int64_t n16,
                                                      uint8_t* __restrict__ packed) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const uint4 c = reinterpret_cast<const uint4*>(codes)[i];
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[2] = {0u, 0u};
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const uint32_t nib = (w[b >> 2] >> (8 * (b & 3))) & 0xFu;
    o[b >> 3] |= nib << (4 * (b & 7));
  }
  reinterpret_cast<uint2*>(packed)[i] = make_uint2(o[0], o[1]);
}
}  // namespace

hipError_t launch_pack_i4(const int8_t* codes, int64_t n, uint8_t* packed, hipStream_t s) {
  const int64_t n16 = n / 16;
  pack_i4_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, s>>>(codes, n16, packed);
  return hipGetLastError();
}

FfnPlan plan_ffn(int64_t T, int H, int I, int E, int k, int w_dtype) {
  FfnPlan p{};
  const int64_t n = T * k;
  if (w_dtype == kF32) {
    p.block_m = 32;
    p.ws_bytes = align256((size_t)n * I * 4);
    snprintf(p.up_name, sizeof p.up_name, "ffn_f32_kernel<up>");
    snprintf(p.down_name, sizeof p.down_name, "ffn_f32_kernel<down>");
  } else if (w_dtype == kI4 || w_dtype == kI4A8) {
    const double mean_rows = (double)n / E;
    const int cls = mean_rows <= 24.0 ? 2 : (mean_rows <= 192.0 ? 1 : 0);
    p.up_var = (I % 128 == 0 ? 0 : 3) + cls;
    p.down_var = (H % 256 == 0 ? 0 : (H % 128 == 0 ? 3 : 6)) + cls;
    p.block_m = cls == 2 ? 64 : (cls == 1 ? 128 : 256);
    // the int8 prefill down GEMM measured faster with two stages, the bf16 one
    // with three
    if (w_dtype == kI4A8 && p.down_var == 0) p.down_var = 9;
    const Variant u = kUpVarW4[p.up_var], d = kDownVarW4[p.down_var];
    const char* t = w_dtype == kI4 ? "w4a16" : "w4a8";
    snprintf(p.up_name, sizeof p.up_name, "gg_kernel<%s,up,%dx%d,%dx%d,S%d,R%d,G%d>", t, u.bm, u.bn, u.wm,
             u.wn, u.stages, u.rowb, u.gn);
    snprintf(p.down_name, sizeof p.down_name, "gg_kernel<%s,down,%dx%d,%dx%d,S%d,R%d,G%d>", t, d.bm, d.bn,
             d.wm, d.wn, d.stages, d.rowb, d.gn);
    if (w_dtype == kI4)
      p.ws_bytes = align256((size_t)n * I * 2);
    else
      p.ws_bytes = align256((size_t)n * I * 2) + align256((size_t)n * 4 * up_parts(I, w_dtype, p.up_var)) +
                   align256((size_t)n * I) + align256((size_t)n * 4);
  } else {
    // shape class from the mean rows per expert: decode-sized (weight
    // streaming, short tiles), mid (one 256-row tile per expert, waves split
    // N), prefill (256 x 256 tiles, 4 x 4 waves of 64 x 64)
    const double mean_rows = (double)n / E;
    const int cls = mean_rows <= 24.0 ? 2 : (mean_rows <= 192.0 ? 1 : 0);
    p.up_var = (I % 128 == 0 ? 0 : 3) + cls;
    p.down_var = (H % 256 == 0 ? 0 : (H % 128 == 0 ? 3 : 6)) + cls;
    if (p.up_var == 4) p.up_var = 3;
    if (p.down_var == 7) p.down_var = 6;
    p.block_m = cls == 2 ? 64 : 256;
    const char* t = w_dtype == kI8 ? "i8" : "bf16";
    const Variant u = kUpVar[p.up_var], d = kDownVar[p.down_var];
    snprintf(p.up_name, sizeof p.up_name, "gg_kernel<%s,up,%dx%d,%dx%d,S%d,R%d,G%d>", t, u.bm, u.bn,
             u.wm, u.wn, u.stages, u.rowb, u.gn);
    snprintf(p.down_name, sizeof p.down_name, "gg_kernel<%s,down,%dx%d,%dx%d,S%d,R%d,G%d>", t, d.bm,
             d.bn, d.wm, d.wn, d.stages, d.rowb, d.gn);
    if (w_dtype == kBF16)
      p.ws_bytes = align256((size_t)n * I * 2);
    else
      p.ws_bytes = align256((size_t)n * I * 2) + align256((size_t)n * 4 * up_parts(I, w_dtype, p.up_var)) +
                   align256((size_t)n * I) + align256((size_t)n * 4);
    if (p.down_var == 0) p.ws_bytes += kTailBytes;
  }
  p.max_tiles = align_max_tiles(T, k, E, p.block_m);
  return p;
}

hipError_t launch_ffn_up(const FfnPlan& p, const void* x, const float* xs, const void* w13,
                         int w_dtype, const float* s13, const int32_t* sorted_slot,
                         const int32_t* tiles, const int32_t* num_tiles, int64_t T, int H, int I,
                         int k, void* ws, hipStream_t s) {
  const FfnBufs b = carve_ffn(ws, T * k, I, w_dtype, p.up_var, p.down_var);
  if (w_dtype == kF32) {
    const unsigned mt = (unsigned)p.max_tiles;
    ffn_f32_kernel<true><<<mt * (I / 32), 256, 0, s>>>((const float*)x, (const float*)w13, sorted_slot,
                                                        tiles, num_tiles, nullptr, H, I, k, I / 32,
                                                        (float*)b.h);
    return hipGetLastError();
  }
  if (w_dtype == kI4)
    return launch_up<false, true>(p, x, xs, w13, s13, sorted_slot, tiles, num_tiles, T, H, I, k, b, s);
  if (w_dtype == kI4A8)
    return launch_up<true, true>(p, x, xs, w13, s13, sorted_slot, tiles, num_tiles, T, H, I, k, b, s);
  if (w_dtype == kBF16)
    return launch_up<false, false>(p, x, xs, w13, s13, sorted_slot, tiles, num_tiles, T, H, I, k, b, s);
  return launch_up<true, false>(p, x, xs, w13, s13, sorted_slot, tiles, num_tiles, T, H, I, k, b, s);
}

hipError_t launch_ffn_down(const FfnPlan& p, const void* w2, int w_dtype, const float* s2,
                           const int32_t* sorted_slot, const int32_t* tiles,
                           const int32_t* num_tiles, const float* topk_w, int64_t T, int H, int I,
                           int k, void* y, void* ws, hipStream_t s) {
  const FfnBufs b = carve_ffn(ws, T * k, I, w_dtype, p.up_var, p.down_var);
  if (w_dtype == kF32) {
    const unsigned mt = (unsigned)p.max_tiles;
    ffn_f32_kernel<false><<<mt * (H / 32), 256, 0, s>>>((const float*)b.h, (const float*)w2,
                                                         sorted_slot, tiles, num_tiles, topk_w, H, I,
                                                         k, H / 32, (float*)y);
    return hipGetLastError();
  }
  if (w_dtype == kI4)
    return launch_down<false, true>(p, w2, s2, sorted_slot, tiles, num_tiles, topk_w, T * k, H, I, y, b, s);
  if (w_dtype == kI4A8)
    return launch_down<true, true>(p, w2, s2, sorted_slot, tiles, num_tiles, topk_w, T * k, H, I, y, b, s);
  if (w_dtype == kBF16)
    return launch_down<false, false>(p, w2, s2, sorted_slot, tiles, num_tiles, topk_w, T * k, H, I, y, b, s);
  return launch_down<true, false>(p, w2, s2, sorted_slot, tiles, num_tiles, topk_w, T * k, H, I, y, b, s);
}

}  // namespace moe
