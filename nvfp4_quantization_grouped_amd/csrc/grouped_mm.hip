// MXFP4 grouped GEMM ("nemo_automodel.components.quantization.mxfp4",
// class MXFP4GroupedMM): per expert e owning token rows [offs[e-1], offs[e]),
//   forward   y[rows_e]      = x[rows_e]        @ W_e^T     (reduce over k)
//   backward  grad_x[rows_e] = grad_out[rows_e] @ W_e       (reduce over n)
// with W_e [n, k] stored as mxfp4 (packed [E, n, k/2] + E8M0 scales
// [E, n, k/32]) and dequantized on the fly with gfx950's scaled fp4
// conversion straight into bf16 MFMA operands (v_mfma_f32_32x32x16_bf16).
// The bf16 weight never exists in HBM.  fp32 accumulation, bf16
// nearest-even output.
//
// Every wave owns a 128-row x 64-column output tile (4 x 2 MFMA tiles, 128
// fp32 accumulators per lane) and runs two to a SIMD, so one's memory phase
// overlaps the other's MFMAs.  Forward workgroups of 4 waves (128 x 256
// tiles, two per CU) serve every shape; the backward uses 8-wave 256 x 256
// tiles whose two row halves share the decoded weights.  The reduction runs
// in steps of
// 64, and inside a step lane-half h of a wave covers the 32 consecutive
// reduction indices [32h, 32h + 32) -- for the forward exactly one E8M0
// scale block -- with sub-step kk taking the 8 values 32h + 8kk ..; both
// operands use the same assignment, so the sum is unchanged.
//
// Scheduling: a one-dimensional grid of output-column tiles x "row-tile
// slots", column-tile index fastest.  Each workgroup reads the device
// offsets and finds which expert and which row tile of it its slot is (sum
// over experts of ceil(rows_e / 128) <= ceil(T / 128) + E slots are
// launched).  Slots past the last tile zero the rows no expert owns.  No host
// synchronization.  With the default round-robin dispatch of workgroups over
// the 8 XCDs and a multiple of 8 column tiles, column tile x runs on XCD
// x % 8 for every row slot, so each XCD's L2 keeps the same weight columns hot while the
// activation blocks it shares with the other XCDs are served from the
// Infinity Cache (this measured faster than giving each XCD a contiguous
// range of row slots).  The backward remaps its workgroups the other way
// (an XCD takes whole row slots with all their column tiles): its grad_out
// tiles are the larger operand to re-fetch, and this measured 2-4% faster.
#include <cstddef>
#include <type_traits>

#include "launch.hpp"
#include "mxq_device.hpp"

namespace mxq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kGemmThreads = 256;
constexpr int kBK = 64;                 // reduction step
constexpr int kLdsRow = kBK * 2 + 16;   // bytes per LDS row (128 data + 16 pad)

struct TileInfo {
  int64_t row0;    // first token row of the tile
  int64_t row_end; // one past the last valid row of its expert (or zero range end)
  int expert;      // -1: zero-fill slot, -2: nothing to do
};

// Which expert / row range a row-tile slot covers.
template <int BM>
__device__ __forceinline__ TileInfo find_tile(const int32_t* __restrict__ offs, int experts, int64_t tokens,
                                              int slot) {
  int64_t start = 0;
  int acc = 0;
  for (int e = 0; e < experts; ++e) {
    // offsets outside [previous, tokens] are clamped into it, so no tile ever
    // reaches past the activation rows whatever offs holds
    int64_t end = offs[e];
    end = end < start ? start : (end > tokens ? tokens : end);
    const int tiles = (int)((end - start + BM - 1) / BM);
    if (slot < acc + tiles) return TileInfo{start + (int64_t)(slot - acc) * BM, end, e};
    acc += tiles;
    start = end;
  }
  // zero-fill slots: rows [offs[E-1], tokens)
  const int64_t z = start + (int64_t)(slot - acc) * BM;
  if (z < tokens) return TileInfo{z, tokens, -1};
  return TileInfo{0, 0, -2};
}

// Inclusive prefix maximum (MAX) or sum over the 64 lanes of a wave, for
// values >= 0: a Hillis-Steele scan inside each row of 16 lanes with DPP
// row shifts (lanes shifted in from outside the row read 0), then each row
// takes the totals of the rows before it.
template <bool MAX, int D>
__device__ __forceinline__ int scan_row_step(int v) {
  const int u = __builtin_amdgcn_update_dpp(0, v, 0x110 + D, 0xF, 0xF, true);   // row_shr:D
  return MAX ? max(v, u) : v + u;
}
template <bool MAX>
__device__ __forceinline__ int wave_scan(int v) {
  v = scan_row_step<MAX, 1>(v);
  v = scan_row_step<MAX, 2>(v);
  v = scan_row_step<MAX, 4>(v);
  v = scan_row_step<MAX, 8>(v);
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31),
            t2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  const int p1 = t0, p2 = MAX ? max(t0, t1) : t0 + t1, p3 = MAX ? max(p2, t2) : p2 + t2;
  const int pre = row == 0 ? 0 : row == 1 ? p1 : row == 2 ? p2 : p3;
  return MAX ? max(v, pre) : v + pre;
}

// Row-tile lookup, built once per wave from the device offsets when there
// are at most 64 experts: lane e holds expert e's clamped segment end and the
// number of row tiles of experts 0..e.  Clamping each offset into [previous
// end, tokens] makes expert e's end the running maximum of 0 and offs[0..e],
// capped at tokens, so both are prefix scans over the lanes; the table costs
// one load of the offsets, and a lookup is one ballot (the first expert whose
// tiles reach past the slot).  A walk over the offsets (find_tile: a
// dependent scalar load per expert) measured 2.7-3.0 us per workgroup with
// 32 experts on MI355X, over half of a forward workgroup's time before its
// first step.  With more than 64 experts the lookup walks them.
template <int BM>
struct TileTable {
  int end;    // lane e < experts: clamped end of expert e's rows; lanes past: the last end
  int incl;   // lane e < experts: row tiles of experts 0..e; lanes past: all row tiles
  const int32_t* offs;
  int experts;
  int64_t tokens;

  __device__ __forceinline__ void build(const int32_t* __restrict__ o, int e_count, int64_t t) {
    offs = o;
    experts = e_count;
    tokens = t;
    end = 0;
    incl = 0;
    if (e_count > 64) return;
    const int lane = threadIdx.x & 63;
    const int v = wave_scan<true>(lane < e_count ? max(o[lane], 0) : 0);
    end = (int)min((int64_t)v, t);
    int prev = __shfl_up(end, 1);
    if (lane == 0) prev = 0;
    incl = wave_scan<false>(lane < e_count ? (int)(((int64_t)end - prev + BM - 1) / BM) : 0);
  }

  // the same result as find_tile<BM>(offs, experts, tokens, slot); every lane active
  __device__ __forceinline__ TileInfo lookup(int slot) const {
    if (experts > 64) return find_tile<BM>(offs, experts, tokens, slot);
    const uint64_t live = experts == 64 ? ~0ull : ((1ull << experts) - 1);
    const uint64_t m = __ballot(incl > slot) & live;
    if (m) {
      const int e = __builtin_ctzll(m);
      const int before = e ? __builtin_amdgcn_readlane(incl, e - 1) : 0;
      const int start = e ? __builtin_amdgcn_readlane(end, e - 1) : 0;
      return TileInfo{start + (int64_t)(slot - before) * BM, __builtin_amdgcn_readlane(end, e), e};
    }
    const int64_t z = __builtin_amdgcn_readlane(end, 63) + (int64_t)(slot - __builtin_amdgcn_readlane(incl, 63)) * BM;
    if (z < tokens) return TileInfo{z, tokens, -1};
    return TileInfo{0, 0, -2};
  }
};

__device__ __forceinline__ const uint8_t* packed_e_of(const uint8_t* packed, int e, int64_t ndim, int64_t kdim) {
  return packed + (int64_t)e * ndim * (kdim / 2);
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  const f32x2_t v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Output of a wave's MT x 2 tiles of 32 x 32 (a 32*MT x 64 block) through
// LDS.  The MFMAs compute each tile transposed (weight fragment as the first
// operand), so lane (r, h) element 4g + e holds row r, column 8g + 4h + e.
// Per pair of column groups, one v_permlane32_swap per dword trades the
// halves so lane (r, 0) holds columns 8g..8g+7 and lane (r, 1) columns
// 8g+8..8g+15 of row r; they go into a row-major LDS block (128 bytes per
// row, 16-byte chunks XOR-swizzled by (row >> 1) & 7, conflict-free both
// ways) and come back 16 bytes per lane, 8 lanes per row, so every global
// store writes 8 whole 128-byte rows (the 2-byte stores of the plain MFMA
// layout touch each row's cache line in 64-byte halves, 4x as many
// instructions).  The stores are non-temporal: the output is not read again
// here, and streaming it past the caches measured 2-3% faster on the
// routed-expert forwards.  ep: this wave's 32*MT*128 bytes of LDS, free of
// pending DMA and other waves' reads.  ncols % 8 == 0, ld % 8 == 0, out
// 16-byte aligned.
template <int MT>
__device__ __forceinline__ void store_block_lds(uint8_t* ep, const f32x16_t (&acc)[MT][2], int lane,
                                                uint8_t* __restrict__ out, int64_t ld, int64_t row0, int64_t row_end,
                                                int64_t col0, int64_t ncols) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g0 = 0; g0 < 4; g0 += 2) {
        const f32x16_t& c = acc[i][j];
        const u32x2_t s0 = __builtin_amdgcn_permlane32_swap(pack_bf16x2(c[4 * g0], c[4 * g0 + 1]),
                                                            pack_bf16x2(c[4 * g0 + 4], c[4 * g0 + 5]), false, false);
        const u32x2_t s1 = __builtin_amdgcn_permlane32_swap(pack_bf16x2(c[4 * g0 + 2], c[4 * g0 + 3]),
                                                            pack_bf16x2(c[4 * g0 + 6], c[4 * g0 + 7]), false, false);
        const int row = 32 * i + r, chunk = 4 * j + g0 + h;
        *reinterpret_cast<u32x4_t*>(ep + row * 128 + 16 * (chunk ^ ((row >> 1) & 7))) = u32x4_t{s0[0], s1[0], s0[1], s1[1]};
      }
#pragma unroll
  for (int it = 0; it < MT * 4; ++it) {
    const int row = 8 * it + (lane >> 3), chunk = lane & 7;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ep + row * 128 + 16 * (chunk ^ ((row >> 1) & 7)));
    const int64_t grow = row0 + row, gcol = col0 + 8 * chunk;
    if (grow < row_end && gcol < ncols)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + (grow * ld + gcol) * 2));
  }
}

// ---------------------------------------------------------------- A operand
// A tile: BM rows x 64 bf16 of a row-major [rows, ld] bf16 matrix.
template <int BM>
struct ALoader {
  static constexpr int kLoads = BM * 8 / kGemmThreads;   // 16-byte chunks per thread
  u32x4_t r[kLoads];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ src, int64_t ld, int64_t row0, int64_t row_end,
                                       int64_t k0, int64_t kdim) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = threadIdx.x + i * kGemmThreads;
      const int row = c >> 3, cc = c & 7;
      const int64_t gr = row0 + row, gk = k0 + cc * 8;
      if (gr < row_end && gk < kdim)
        r[i] = *reinterpret_cast<const u32x4_t*>(src + (gr * ld + gk) * 2);
      else
        r[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = threadIdx.x + i * kGemmThreads;
      const int row = c >> 3, cc = c & 7;
      *reinterpret_cast<u32x4_t*>(lds + row * kLdsRow + cc * 16) = r[i];
    }
  }
};

// ------------------------------------------------- forward, general shapes
// Forward with the weight operand kept out of LDS (any K % 32 == 0).  The workgroup owns a
// 128 x 256 output tile; its 4 waves split the columns (wave tile 128 x 64,
// 4 x 2 MFMA tiles).  Within a reduction step of 64, lane-half h takes the
// 32 consecutive k [k0 + 32h, k0 + 32h + 32) -- one E8M0 scale block -- and
// sub-step kk the 8 values k0 + 32h + 8kk .. +7; A and B use the same
// assignment, so the sum is unchanged.  A lane therefore fetches its weight
// row's 16 packed bytes and one scale byte per column tile and step straight
// from global memory and decodes them into its four B fragments; only the
// activation tile goes through (double-buffered) LDS.  37 KB of LDS and
// <= 256 registers per lane let two workgroups share a CU.
constexpr int kFwdBM = 128, kFwdBN = 256;

__global__ void __launch_bounds__(kGemmThreads, 2)
k_grouped_mm_fwd_general(const uint8_t* __restrict__ a, const uint8_t* __restrict__ packed,
                 const uint8_t* __restrict__ scales, const int32_t* __restrict__ offs, int experts,
                 int64_t tokens, int64_t ndim, int64_t kdim, uint8_t* __restrict__ out, int gx) {
  constexpr int BM = kFwdBM, BN = kFwdBN, MT = BM / 32, NT = BN / 4 / 32;
  // one-dimensional grid: workgroup b takes column tile b % gx of row slot b / gx
  const int64_t col0 = (int64_t)(blockIdx.x % gx) * BN;
  TileTable<BM> tt;
  tt.build(offs, experts, tokens);
  const TileInfo ti = tt.lookup((int)(blockIdx.x / gx));
  if (ti.expert == -2) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r = lane & 31;

  if (ti.expert == -1) {
    for (int i = threadIdx.x; i < BM * BN / 8; i += kGemmThreads) {
      const int rr = i / (BN / 8), c = (i % (BN / 8)) * 8;
      const int64_t gr = ti.row0 + rr, gc = col0 + c;
      if (gr < ti.row_end && gc < ndim) {
        unsigned short* dst = reinterpret_cast<unsigned short*>(out + (gr * ndim + gc) * 2);
        for (int q = 0; q < 8 && gc + q < ndim; ++q) dst[q] = 0;
      }
    }
    return;
  }

  __shared__ uint8_t lds_a[2][BM * kLdsRow];
  const uint8_t* packed_e = packed + (int64_t)ti.expert * ndim * (kdim / 2);
  const uint8_t* scales_e = scales + (int64_t)ti.expert * ndim * (kdim / 32);

  ALoader<BM> al;
  // this lane's weight rows (one per column tile) and their validity
  int64_t wrow[NT];
  bool wok[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    wrow[j] = col0 + wave * (BN / 4) + j * 32 + r;
    wok[j] = wrow[j] < ndim;
  }
  u32x4_t pb[NT];
  uint32_t sb[NT];
  auto load_b = [&](int64_t k0) {
    const int64_t kb = k0 + 32 * h;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (wok[j] && kb < kdim) {
        pb[j] = *reinterpret_cast<const u32x4_t*>(packed_e + wrow[j] * (kdim / 2) + kb / 2);
        sb[j] = scales_e[wrow[j] * (kdim / 32) + kb / 32];
      } else {
        pb[j] = u32x4_t{0u, 0u, 0u, 0u};
        sb[j] = 127u;
      }
    }
  };

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16_t{};

  const int nsteps = (int)((kdim + kBK - 1) / kBK);
  al.load(a, kdim, ti.row0, ti.row_end, 0, kdim);
  load_b(0);
  al.store(lds_a[0]);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    // decode this step's weights into B fragments
    bf16x8_t fb[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const float sc = e8m0_to_f32(sb[j]);
      const uint32_t w[4] = {pb[j].x, pb[j].y, pb[j].z, pb[j].w};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4_t v = {dec_fp4_bf16x2<0>(w[kk], sc), dec_fp4_bf16x2<1>(w[kk], sc), dec_fp4_bf16x2<2>(w[kk], sc),
                     dec_fp4_bf16x2<3>(w[kk], sc)};
        fb[j][kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    if (s + 1 < nsteps) {
      al.load(a, kdim, ti.row0, ti.row_end, (int64_t)(s + 1) * kBK, kdim);
      load_b((int64_t)(s + 1) * kBK);
    }
    const uint8_t* la = lds_a[cur] + r * kLdsRow + 64 * h;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t fa[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(la + i * 32 * kLdsRow + kk * 16);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j][kk], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nsteps) al.store(lds_a[cur ^ 1]);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t gc = wrow[j];
#pragma unroll
      for (int q = 0; q < 16; q += 2) {
        const int64_t gr0 = ti.row0 + i * 32 + 8 * (q >> 2) + 4 * h + (q & 3);
        f32x2_t v = {acc[i][j][q], acc[i][j][q + 1]};
        const uint32_t bb = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
        if (wok[j]) {
          if (gr0 < ti.row_end) *reinterpret_cast<unsigned short*>(out + (gr0 * ndim + gc) * 2) = (unsigned short)(bb & 0xFFFFu);
          if (gr0 + 1 < ti.row_end) *reinterpret_cast<unsigned short*>(out + ((gr0 + 1) * ndim + gc) * 2) = (unsigned short)(bb >> 16);
        }
      }
    }
  }
}

// ------------------------------------------------------ forward, K % 128 == 0
// Same wave tile and fragment scheme as the general forward, with W waves
// side by side along the columns (W = 4 in use: 128 x 512 tiles of 8 waves,
// one per CU, measured 2% slower on the routed-expert layer) and BM = 128 or
// 96 rows, and every global transfer of the main loop a direct global->LDS
// DMA (buffer_load ... lds: the buffer descriptor carries the row base and
// the valid range, the scalar offset the step), issued two steps ahead into
// a ring of three LDS stages:
//  * activations: the BM x 64 bf16 tile as BM / 8 blocks of 1 KB; a
//    block holds 8 rows, and within a row the eight 16-byte chunks are
//    XOR-swizzled by ((row >> 1) & 7): LDS serves 16 lanes x 16 bytes (256
//    bytes, two 128-byte rows) per cycle, and with this swizzle any 16
//    consecutive rows read at one logical chunk hit 16 distinct 16-byte bank
//    groups, so the fragment reads are conflict-free without padding;
//  * weights: each wave fetches the packed bytes of its own 64 weight rows
//    (2 blocks of 1 KB, laid out [row/32][half][row%32] x 16 bytes, so a
//    lane's 16 bytes -- one 32-k scale block -- sit next to its neighbours')
//    and their scale bytes, either the aligned dword holding this step's
//    two 32-k blocks and the neighbouring step's (4 bytes per lane, every
//    step) or, when K % 512 == 0, 16 bytes covering 8 steps, every 8 steps.
//    The per-lane cost of these transfers follows the cache lines they
//    touch (a weight block touches 32 lines for 1 KB, a scale dword
//    transfer 64 lines for 256 bytes), so the 8-step scale chunks matter;
//  * each step waits for exactly the DMA of the step it is about to use
//    (s_waitcnt vmcnt(N), N = operations issued after it), then barriers.
// With no register-destined loads in the loop, no other waits are needed.
// Every step but the last STAGES - 1 issues the same operations (keeping N
// constant); those last steps issue none and wait for everything pending.
// Rows past the expert's segment and weight rows past N lie past their
// buffer's range and read zeros; they are never stored.  Needs K % 128 == 0
// (4-byte aligned scale rows).
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt immediate: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits
  // 15:14, expcnt bits 6:4 (left at its maximum), lgkmcnt bits 11:8 = 0:
  // this wave's LDS reads of the stage are complete before anyone passes the
  // barrier and starts refilling it.
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
  asm volatile("s_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void_t;


// LDS of the DMA forward for a workgroup of W waves (W x 64 output columns).
// A stage holds one step's activation tile and packed weight bytes (32 per
// column).  Scales come in chunks of SCH steps: SCH = 2 puts each column's
// dword (2 steps x 2 blocks) in every stage; SCH = 8 keeps a separate
// double buffer of 16 bytes (8 steps) per column, refilled every 8 steps,
// so the scale transfer touches each column's cache line once per 8 steps
// instead of once per step.
template <int BM, int W, int SCH>
struct DmaStage {                                           // SCH == 8: no scales per stage
  uint8_t a[BM * 128];                                      // activation tile, unpadded (swizzled)
  uint8_t b[W * 64 * 32];
};
template <int BM, int W>
struct DmaStage<BM, W, 2> {
  uint8_t a[BM * 128];
  uint8_t b[W * 64 * 32];
  uint8_t s[W * 64 * 4];
};
template <int BM, int W, int STAGES, int SCH>
struct DmaSmem {
  static constexpr int kCols = W * 64;
  static constexpr int kABlocksPerWave = BM / 8 / W;        // 1 KB activation blocks (8 rows) each wave moves
  static_assert(BM % (8 * W) == 0, "activation blocks per wave");
  using Stage = DmaStage<BM, W, SCH>;
  Stage st[STAGES];
  uint8_t s8[2][kCols * 16];
};
template <int BM, int W, int STAGES>
struct DmaSmem<BM, W, STAGES, 2> {
  static constexpr int kCols = W * 64;
  static constexpr int kABlocksPerWave = BM / 8 / W;
  static_assert(BM % (8 * W) == 0, "activation blocks per wave");
  using Stage = DmaStage<BM, W, 2>;
  Stage st[STAGES];
};

// Global sides of one wave's transfers, as raw buffers: the descriptors
// (scalar registers) hold the tile's, or the wave's, first row and the
// valid range, each lane a fixed 32-bit offset, and a step only moves the
// scalar offset, so no vector address arithmetic runs per transfer; reads
// past the range (rows past the expert's end, weight rows past n) return
// zeros.
template <int QA>
struct DmaSrc {
  __amdgpu_buffer_rsrc_t a, b, s;   // activations, packed weights, scales
  uint32_t a_off[QA];
  uint32_t b_off[2];
  uint32_t s_off;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(bytes > 0 ? bytes : 0), 0x00020000);
}

// Op q of one step's transfers of one wave, straight into LDS (q < QA:
// activation block q; then the 2 weight blocks; then, with SCH == 2, the
// scale dword).
template <int QA, int SCH, class StageT>
__device__ __forceinline__ void fwd_dma_op(StageT& d, const DmaSrc<QA>& src, int wave, int step, int q) {
  if (q < QA) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.a, (lds_void_t*)(d.a + 1024 * (QA * wave + q)), 16, src.a_off[q],
                                             step * kBK * 2, 0, 0);
  } else if (q < QA + 2) {
    const int j = q - QA;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.b, (lds_void_t*)(d.b + 2048 * wave + 1024 * j), 16, src.b_off[j],
                                             step * 32, 0, 0);
  } else if constexpr (SCH == 2) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.s, (lds_void_t*)(d.s + 256 * wave), 4, src.s_off, 4 * (step >> 1), 0,
                                             0);
  }
}

// All of one step's transfers of one wave.
template <int QA, int SCH, class StageT>
__device__ __forceinline__ void fwd_dma_issue(StageT& d, const DmaSrc<QA>& src, int wave, int step) {
#pragma unroll
  for (int q = 0; q < QA + 2 + (SCH == 2 ? 1 : 0); ++q) fwd_dma_op<QA, SCH>(d, src, wave, step, q);
}

// The 16-byte scale chunk c (steps 8c .. 8c+7) of this wave's 64 columns,
// into dst (this wave's 1 KB of the chunk's buffer).
__device__ __forceinline__ void fwd_dma_scales8(lds_void_t* dst, __amdgpu_buffer_rsrc_t s, uint32_t s_off, int chunk) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(s, dst, 16, s_off, 16 * chunk, 0, 0);
}

// SPREAD: issue a step's transfers one or two at a time behind each
// sub-step's fragment reads, so they go out between MFMAs instead of as one
// burst ahead of them (a transfer cannot move past LDS reads of the ring on
// its own: the compiler keeps LDS writes and reads in order).  With buffer
// transfers it is as fast or faster at every K measured (MI355X: +3% at
// K = 7168, +2% at K = 2048); the burst form (SPREAD = false) is kept as
// the reference schedule.
template <int BM, int W, int STAGES, int MINWG, int SCH, bool SPREAD>
__global__ void __launch_bounds__(W * 64, MINWG)
k_grouped_mm_fwd_dma(const uint8_t* __restrict__ a, const uint8_t* __restrict__ packed,
                     const uint8_t* __restrict__ scales, const int32_t* __restrict__ offs, int experts,
                     int64_t tokens, int64_t ndim, int64_t kdim, uint8_t* __restrict__ out, int gx) {
  static_assert(SCH == 2 || SCH == 8, "scale chunk");
  // with SCH == 8 the step-end wait below counts the scale transfer of this
  // step only, which is exact for a ring of three stages
  static_assert(SCH == 2 || STAGES == 3, "scale chunk accounting assumes 3 stages");
  using Smem = DmaSmem<BM, W, STAGES, SCH>;
  constexpr int BN = Smem::kCols, MT = BM / 32, NT = 2, QA = Smem::kABlocksPerWave;
  constexpr int kOps = QA + 2 + (SCH == 2 ? 1 : 0);   // per wave and step (plus 1 every 8 steps when SCH == 8)
  constexpr int kThreads = W * 64;
  // one-dimensional grid: workgroup b takes column tile b % gx of row slot b / gx
  const int64_t col0 = (int64_t)(blockIdx.x % gx) * BN;
  TileTable<BM> tt;
  tt.build(offs, experts, tokens);
  const TileInfo ti = tt.lookup((int)(blockIdx.x / gx));
  if (ti.expert == -2) return;
  // wave index in a scalar register: the LDS destinations of the DMA are scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, r = lane & 31;

  if (ti.expert == -1) {
    for (int i = threadIdx.x; i < BM * BN / 8; i += kThreads) {
      const int rr = i / (BN / 8), c = (i % (BN / 8)) * 8;
      const int64_t gr = ti.row0 + rr, gc = col0 + c;
      if (gr < ti.row_end && gc < ndim) {
        unsigned short* dst = reinterpret_cast<unsigned short*>(out + (gr * ndim + gc) * 2);
        for (int q = 0; q < 8 && gc + q < ndim; ++q) dst[q] = 0;
      }
    }
    return;
  }

  __shared__ __attribute__((aligned(1024))) Smem sm;

  // activation DMA: this wave fills A blocks QA*wave .. QA*wave+QA-1; block b
  // holds rows 8b .. 8b+7: lane l -> row 8b + l/8, LDS chunk l%8 <- global
  // chunk (l%8) ^ ((row >> 1) & 7).  Ranges and offsets fit 31 bits (the
  // launcher checks K and one expert's packed weights; the activation range
  // covers this tile's rows only, since an expert's whole segment could pass
  // 2^31 bytes).
  DmaSrc<QA> src;
  src.a = dma_rsrc(a + ti.row0 * kdim * 2, min(ti.row_end - ti.row0, (int64_t)BM) * kdim * 2);
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int row = 8 * (QA * wave + q) + (lane >> 3);
    src.a_off[q] = (uint32_t)(((int64_t)row * kdim + ((lane & 7) ^ ((row >> 1) & 7)) * 8) * 2);
  }
  // weight DMA: this wave's rows n = col0 + 64*wave + 32*j + r (j = 0, 1);
  // block j holds [half h][row r] x 16 bytes.  Scales: lane l covers column
  // 64*wave + l (a dword per step pair, or 16 bytes per 8 steps).
  const int64_t n0 = col0 + wave * 64;
  src.b = dma_rsrc(packed_e_of(packed, ti.expert, ndim, kdim) + n0 * (kdim / 2), (ndim - n0) * (kdim / 2));
#pragma unroll
  for (int j = 0; j < NT; ++j) src.b_off[j] = (uint32_t)((j * 32 + r) * (kdim / 2) + 16 * h);
  // 4-byte aligned rows for SCH == 2 (K % 128 == 0), 16-byte for SCH == 8 (K % 512 == 0)
  src.s = dma_rsrc(scales + ((int64_t)ti.expert * ndim + n0) * (kdim / 32), (ndim - n0) * (kdim / 32));
  src.s_off = (uint32_t)(lane * (kdim / 32));

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16_t{};

  const int nsteps = (int)(kdim / kBK);
  const int last = nsteps - 1;
  const int last_chunk = (nsteps - 1) >> 3;
  if constexpr (SCH == 8) fwd_dma_scales8((lds_void_t*)(sm.s8[0] + 1024 * wave), src.s, src.s_off, 0);
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t)
    fwd_dma_issue<QA, SCH>(sm.st[t], src, wave, min(t, last));
  // step 0 (and scale chunk 0) have landed once only steps 1 .. STAGES-2 may be in flight
  wait_vmcnt_barrier<kOps * (STAGES - 2)>();

  const int swz_base = r * 128;
  int stage = 0;
  for (int s = 0; s < nsteps; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    // scale chunk c+1 goes out at the first step of chunk c, ahead of this
    // step's activation and weight transfers (vmcnt counts in issue order)
    const bool chunk_start = SCH == 8 && (s & 7) == 0;
    if constexpr (SCH == 8) {
      if (chunk_start) {
        const int c = min((s >> 3) + 1, last_chunk);
        fwd_dma_scales8((lds_void_t*)(sm.s8[c & 1] + 1024 * wave), src.s, src.s_off, c);
      }
    }
    // refill the stage step s-1 used with step s + STAGES - 1 (none in the
    // last STAGES - 1 steps: nothing is left to fetch)
    typename Smem::Stage& nxt = sm.st[stage == 0 ? STAGES - 1 : stage - 1];
    const int nstep = s + STAGES - 1;
    const bool refill = nstep <= last;
    if constexpr (!SPREAD) {
      if (refill) fwd_dma_issue<QA, SCH>(nxt, src, wave, nstep);
    }
    const typename Smem::Stage& c = sm.st[stage];
    // decode this wave's weights for the step into B fragments
    bf16x8_t fb[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const u32x4_t p = *reinterpret_cast<const u32x4_t*>(c.b + 2048 * wave + 1024 * j + 512 * h + 16 * r);
      const int col = wave * 64 + j * 32 + r;
      uint8_t sb;
      if constexpr (SCH == 2)
        sb = c.s[4 * col + 2 * (s & 1) + h];
      else
        sb = sm.s8[(s >> 3) & 1][16 * col + 2 * (s & 7) + h];
      const float sc = e8m0_to_f32(sb);
      const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4_t v = {dec_fp4_bf16x2<0>(w[kk], sc), dec_fp4_bf16x2<1>(w[kk], sc), dec_fp4_bf16x2<2>(w[kk], sc),
                     dec_fp4_bf16x2<3>(w[kk], sc)};
        fb[j][kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    const uint8_t* la = c.a + swz_base;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int off = 16 * ((4 * h + kk) ^ ((r >> 1) & 7));   // rows 32i + r share the swizzle
      bf16x8_t fa[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(la + i * 32 * 128 + off);
      if constexpr (SPREAD) {
        // this sub-step's share of the next stage's transfers (same ops, same
        // order, so the step-end vmcnt count is unchanged)
        constexpr int kOpsAll = QA + 2 + (SCH == 2 ? 1 : 0);
        if (refill) {
#pragma unroll
          for (int q = kk * kOpsAll / 4; q < (kk + 1) * kOpsAll / 4; ++q)
            fwd_dma_op<QA, SCH>(nxt, src, wave, nstep, q);
        }
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j][kk], fa[i], acc[i][j], 0, 0, 0);
    }
    // step s+1 (and its scale chunk) have landed once only the transfers
    // issued after step s+1's may be in flight: steps s+2 .. s+STAGES-1, and
    // this step's scale chunk
    if (!refill)
      wait_vmcnt_barrier<0>();   // nothing issued this step: all that is pending is needed
    else if (chunk_start)
      wait_vmcnt_barrier<kOps * (STAGES - 2) + 1>();
    else
      wait_vmcnt_barrier<kOps * (STAGES - 2)>();
    __builtin_amdgcn_sched_barrier(0);
    stage = stage == STAGES - 1 ? 0 : stage + 1;
  }
  // drain the clamped tail transfers; once every wave has, the ring is free
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);
  __syncthreads();
  static_assert(sizeof(Smem) >= (size_t)W * BM * 128, "epilogue block fits the ring");
  store_block_lds<MT>(reinterpret_cast<uint8_t*>(&sm) + wave * BM * 128, acc, lane, out, ndim, ti.row0, ti.row_end,
                      col0 + wave * 64, ndim);
}

// ------------------------------------------------------ forward, W4A4
// y[rows_e] = x_q[rows_e] @ W_e^T with the activations quantized to MXFP4 as
// well ("NVIDIA Model Optimizer: from mtq.quantize to a 4.95-bit
// DeepSeek-R1", section "The claims, marked reported": the weight-and-
// activation FP4 form is the one that runs on the FP4 matrix units; the
// activations as "nemo_automodel.components.quantization.mxfp4"
// quantize_mxfp4 writes them: packed [T, K/2], E8M0 scales [T, K/32]), on gfx950's
// block-scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 with both operands fp4
// e2m1.  Its operand layout (pinned by an in-bounds probe against a float64
// reference, to fp32 rounding): lane l carries row (or column) l % 32 and
// the 32 consecutive k of block l / 32 of the 64-k sub-step, two codes per
// byte with the even k in the low nibble -- exactly one stored row segment
// and its E8M0 block -- and byte 0 of its scale register scales that block
// (a 0xFF scale gives NaN).  So no code is decoded here: both operands go
// from global memory through LDS into the MFMA as stored.  Products of two
// e2m1 codes and two power-of-two scales are exact, sums run in fp32, the
// output rounds to bf16 nearest-even.
//
// Workgroup: 8 waves, a 256 x 256 output tile; wave (wm, wn) = (wave / 4,
// wave % 4) owns rows [128 wm, +128) and columns [64 wn, +64), 4 x 2 MFMA
// tiles computed transposed (weight fragment first, as in the bf16 kernels,
// so the LDS-staged epilogue is shared).  The reduction runs in stages of
// 128 k (64 bytes of each row), 2 MFMA sub-steps each, through a ring of 4
// LDS stages filled by buffer->LDS DMA three stages ahead; a stage row's four
// 16-byte chunks are XOR-swizzled by (row >> 2) & 3, so the 16 rows one
// fragment read touches per LDS cycle hit 16 distinct bank groups.  Scales
// come 16 bytes (512 k, 4 stages) per row at a time into a double buffer.
// Needs K % 512 == 0 (16-byte aligned scale rows).
constexpr int kW4BM = 256, kW4BN = 256, kW4Threads = 512, kW4Stages = 4;

struct W4Smem {
  uint8_t a[kW4Stages][kW4BM * 64];   // activation codes: 256 rows x 64 bytes (128 k) per stage
  uint8_t b[kW4Stages][kW4BN * 64];   // weight codes: 256 columns x 64 bytes
  uint8_t sa[2][kW4BM * 16];          // activation scales: 16 bytes (512 k) per row
  uint8_t sb[2][kW4BN * 16];          // weight scales
};

typedef int v8i32_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16_t mfma_w4(const u32x4_t& w, const u32x4_t& x, uint32_t sw, uint32_t sx,
                                            const f32x16_t& c) {
  const v8i32_t a = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  const v8i32_t b = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, (int)sw, 0, (int)sx);
}

__global__ void __launch_bounds__(kW4Threads, 1)
k_grouped_mm_fwd_w4a4(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                      const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
                      const int32_t* __restrict__ offs, int experts, int64_t tokens, int64_t ndim, int64_t kdim,
                      uint8_t* __restrict__ out, int gx) {
  constexpr int BM = kW4BM, BN = kW4BN, MT = 4, NT = 2, S = kW4Stages, kThreads = kW4Threads;
  const int64_t col0 = (int64_t)(blockIdx.x % gx) * BN;
  TileTable<BM> tt;
  tt.build(offs, experts, tokens);
  const TileInfo ti = tt.lookup((int)(blockIdx.x / gx));
  if (ti.expert == -2) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5, r = lane & 31;

  if (ti.expert == -1) {
    for (int i = threadIdx.x; i < BM * BN / 8; i += kThreads) {
      const int rr = i / (BN / 8), c = (i % (BN / 8)) * 8;
      const int64_t gr = ti.row0 + rr, gc = col0 + c;
      if (gr < ti.row_end && gc < ndim) {
        unsigned short* dst = reinterpret_cast<unsigned short*>(out + (gr * ndim + gc) * 2);
        for (int q = 0; q < 8 && gc + q < ndim; ++q) dst[q] = 0;
      }
    }
    return;
  }

  __shared__ __attribute__((aligned(1024))) W4Smem sm;

  // buffers over this tile's activation rows and weight columns (reads past
  // the expert's rows or past n return zeros); ranges fit 31 bits (the
  // launcher checks one expert's packed weights, and K < 2^22)
  const int64_t prow = kdim / 2, srow = kdim / 32;
  const int64_t nrows = min(ti.row_end - ti.row0, (int64_t)BM);
  const __amdgpu_buffer_rsrc_t rs_a = dma_rsrc(xq + ti.row0 * prow, nrows * prow);
  const __amdgpu_buffer_rsrc_t rs_sa = dma_rsrc(xs + ti.row0 * srow, nrows * srow);
  const __amdgpu_buffer_rsrc_t rs_b = dma_rsrc(packed_e_of(packed, ti.expert, ndim, kdim) + col0 * prow, (ndim - col0) * prow);
  const __amdgpu_buffer_rsrc_t rs_sb =
      dma_rsrc(scales + ((int64_t)ti.expert * ndim + col0) * srow, (ndim - col0) * srow);
  // code transfers: op q (16 rows) of a stage, wave w moves ops 2w and 2w+1
  // of both operands; lane l -> row 16q + l/4, LDS chunk l%4 <- global chunk
  // (l%4) ^ ((row >> 2) & 3)
  uint32_t c_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * (2 * wave + j) + (lane >> 2);
    c_off[j] = (uint32_t)(row * prow + 16 * ((lane & 3) ^ ((row >> 2) & 3)));
  }
  // scale transfers: wave w < 4 moves activation rows 64w .. 64w+63, wave
  // w >= 4 weight columns 64(w-4) ..; 16 bytes per lane
  const bool s_is_a = wave < 4;
  const uint32_t s_off = (uint32_t)((64 * (wave & 3) + lane) * srow);
  auto issue_codes = [&](int st, int stage, int j) {   // j = 0, 1: the wave's two ops of one operand pair
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void_t*)(sm.a[st] + 1024 * (2 * wave + j)), 16, c_off[j],
                                             stage * 64, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void_t*)(sm.b[st] + 1024 * (2 * wave + j)), 16, c_off[j],
                                             stage * 64, 0, 0);
  };
  auto issue_scales = [&](int chunk) {
    uint8_t* dst = (s_is_a ? sm.sa[chunk & 1] : sm.sb[chunk & 1]) + 1024 * (wave & 3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s_is_a ? rs_sa : rs_sb, (lds_void_t*)dst, 16, s_off, 16 * chunk, 0, 0);
  };

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16_t{};

  const int last = (int)(kdim / 128) - 1, last_chunk = last >> 2;
  issue_scales(0);
#pragma unroll
  for (int t = 0; t < S - 1; ++t) {
    issue_codes(t, t, 0);
    issue_codes(t, t, 1);
  }
  // stage 0 and scale chunk 0 have landed once only stages 1, 2 (4 ops each) may be in flight
  wait_vmcnt_barrier<8>();

  // fragment addresses: rows 128 wm + 32 i + r share (row >> 2) & 3 = (r >> 2) & 3
  const int swz = (r >> 2) & 3;
  const int a_row = (128 * wm + r) * 64, b_row = (64 * wn + r) * 64;
  const int sa_row = (128 * wm + r) * 16, sb_row = (64 * wn + r) * 16;
  struct Half {                  // one sub-step's fragments
    u32x4_t x[MT], w[NT];
  };
  struct Scl {                   // a stage's scale dwords: blocks of (sub-step 0, half 0), (0, 1), (1, 0), (1, 1)
    uint32_t x[MT], w[NT];
  };
  auto read_half = [&](Half& f, int s, int kk) {
    const int st = s & (S - 1), off = 16 * ((2 * kk + h) ^ swz);
#pragma unroll
    for (int i = 0; i < MT; ++i) f.x[i] = *reinterpret_cast<const u32x4_t*>(sm.a[st] + a_row + i * 32 * 64 + off);
#pragma unroll
    for (int j = 0; j < NT; ++j) f.w[j] = *reinterpret_cast<const u32x4_t*>(sm.b[st] + b_row + j * 32 * 64 + off);
  };
  auto read_scales = [&](Scl& c, int s) {
    const uint8_t* sa_c = sm.sa[(s >> 2) & 1] + 4 * (s & 3);
    const uint8_t* sb_c = sm.sb[(s >> 2) & 1] + 4 * (s & 3);
#pragma unroll
    for (int i = 0; i < MT; ++i) c.x[i] = *reinterpret_cast<const uint32_t*>(sa_c + sa_row + i * 32 * 16);
#pragma unroll
    for (int j = 0; j < NT; ++j) c.w[j] = *reinterpret_cast<const uint32_t*>(sb_c + sb_row + j * 32 * 16);
  };
  auto mfmas = [&](const Half& f, const Scl& c, int kk) {
    const int sh = 8 * (2 * kk + h);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = mfma_w4(f.w[j], f.x[i], (c.w[j] >> sh) & 0xFF, (c.x[i] >> sh) & 0xFF, acc[i][j]);
  };
  // Stage s, entered with its sub-step 0 fragments and its scales in
  // registers (k0, sc): read its sub-step 1 fragments; refill ring slot
  // (s + 3) % 4 -- stage s - 1's, whose reads every wave finished before the
  // barrier in the middle of stage s - 1 -- with stage s + 3; sub-step 0's
  // MFMAs; wait for stage s + 1 and barrier; read stage s + 1's sub-step 0
  // fragments and scales into (nk0, nsc); sub-step 1's MFMAs.  Each batch of
  // reads is covered by 8 MFMAs per wave, and the MFMA pipe keeps sub-step
  // 1's work across the barrier (with one workgroup per CU, a barrier at the
  // end of the stage drained the pipe every stage).  Stage s's reads all
  // precede the barrier in its middle, and its slot is refilled only in
  // stage s + 1.
  auto stage = [&](const Half& k0, const Scl& sc, Half& nk0, Scl& nsc, int s) {
    __builtin_amdgcn_sched_barrier(0);
    Half k1;
    read_half(k1, s, 1);
    const bool chunk_start = (s & 3) == 0;
    if (chunk_start) issue_scales(min((s >> 2) + 1, last_chunk));
    const bool refill = s + S - 1 <= last;
    const int nstg = (s + S - 1) & (S - 1);
    if (refill) issue_codes(nstg, s + S - 1, 0);
    mfmas(k0, sc, 0);
    if (refill) issue_codes(nstg, s + S - 1, 1);
    if (s + 1 <= last) {
      // stage s+1 (and its scale chunk) have landed once only the transfers
      // issued after stage s+1's may be in flight: stages s+2 and s+3 (4 ops
      // each, when they exist) and the scale chunks issued at stages s-1, s
      const bool c_prev = s >= 1 && ((s - 1) & 3) == 0;
      const int pend = (s + 2 <= last ? 4 : 0) + (refill ? 4 : 0) + (chunk_start ? 1 : 0) + (c_prev ? 1 : 0);
      __builtin_amdgcn_sched_barrier(0);
      switch (pend) {
        case 9: wait_vmcnt_barrier<9>(); break;
        case 8: wait_vmcnt_barrier<8>(); break;
        case 5: wait_vmcnt_barrier<5>(); break;
        case 4: wait_vmcnt_barrier<4>(); break;
        case 1: wait_vmcnt_barrier<1>(); break;
        default: wait_vmcnt_barrier<0>(); break;
      }
      __builtin_amdgcn_sched_barrier(0);
      read_half(nk0, s + 1, 0);
      read_scales(nsc, s + 1);
    }
    mfmas(k1, sc, 1);
  };

  const int nst = (int)(kdim / 128);      // >= 4 and even (K % 512 == 0)
  Half h0, h1;
  Scl c0, c1;
  read_half(h0, 0, 0);
  read_scales(c0, 0);
  for (int s = 0; s < nst; s += 2) {
    stage(h0, c0, h1, c1, s);
    stage(h1, c1, h0, c0, s + 1);
  }
  // every wave's fragment reads of the ring are done before any wave stages
  // its output there (no code transfer is pending: the last one, stage
  // last's, was waited for in the middle of stage last - 1); drain the
  // clamped scale transfer too (it lands outside the epilogue block)
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
  static_assert(offsetof(W4Smem, sa) >= (size_t)8 * 128 * 128, "epilogue block fits in front of the scales");
  store_block_lds<MT>(reinterpret_cast<uint8_t*>(&sm) + wave * 128 * 128, acc, lane, out, ndim, ti.row0 + 128 * wm,
                      ti.row_end, col0 + wn * 64, ndim);
}

// ----------------------------------------------------------------- backward
// grad_x = grad_out @ W_e.  Tile: 256 token rows x 256 output columns (k),
// reduction over n in steps of 64; 8 waves, one workgroup per CU.  Wave
// (wm, wn) = (wave / 4, wave % 4) owns rows [128 wm, 128 wm + 128) and
// columns [64 wn, 64 wn + 64) of the tile (4 x 2 MFMA tiles), so the two
// waves of a column block share its decoded weights: each step's 64 x 256
// weight block is decoded once for 256 rows.  Global loads are raw buffer
// loads over the tile's valid range: the hardware returns zeros past it, so
// rows past the expert's end, n past the weight rows and column halves past
// k need no masking (an out-of-range chunk gets an offset past every range).
//  * grad_out tile (256 x 64 bf16) is loaded into registers one step ahead
//    and stored into a double-buffered LDS tile (same (row >> 1) & 7 chunk
//    swizzle as the DMA forward);
//  * weights: wave (wm, wn) fetches, two steps ahead, rows [32 wm, 32 wm +
//    32) of the step's 64 in its 64 columns -- one piece of 16 packed bytes
//    (32 values of one row) and its scale byte per lane -- decodes it along
//    k (the direction the scaled fp4 conversion and the E8M0 block both run)
//    a step later, between that step's MFMAs, and writes it in 16-byte
//    chunks into the column block's tile Wd[n][k] of the step after
//    (double-buffered, so the barrier that ends the step publishes it);
//  * the B fragments, which need 8 consecutive n of one column per lane,
//    come out of Wd with gfx950's transposing LDS read ds_read_b64_tr_b16:
//    within each group of 16 lanes, output lane i, element e is element
//    i % 4 of source lane 4e + i / 4, so source lanes pointing at
//    Wd[n0 + s/4][c0 + 4(s%4)] (s = lane % 16) hand lane i the four values
//    Wd[n0 .. n0+3][c0 + i]; two reads give the 8 values of a fragment;
//  * MFMA fragments as in the forward: lane-half h covers n in
//    [32h, 32h + 32) of the step, sub-step kk the 8 values 32h + 8kk ..;
//  * Wd's 16-byte chunk c of row n sits at chunk c ^ swz(n), swz(n) =
//    4 * ((n >> 1) & 1) + ((n >> 1) & 3): the piece writes (8 consecutive
//    rows, both column halves, one chunk each) and the transposing reads
//    (4 consecutive rows, one aligned quad of chunks) hit distinct 16-byte
//    groups of the 64 LDS banks.
constexpr int kBwdBM = 256, kBwdBN = 256, kBwdThreads = 512;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ int wd_swz(int n) { return (((n >> 1) & 1) << 2) | ((n >> 1) & 3); }

// raw buffer over [base, base + bytes) (bytes < 2^31): loads at offsets past
// the range return zeros
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kBufOob = 0x80000000u;   // offset past every range used here

struct WRaw {          // one step's weight piece of a lane (16 packed bytes + scale byte)
  u32x4_t pk;
  uint32_t sb;
};

struct BwdSmem {
  uint8_t g[2][kBwdBM * 128];                // grad_out tiles, 256 rows x 128 bytes
  uint8_t w[2][4][64 * 128];                 // decoded weights per column block, 64 n x 64 k bf16
};

__global__ void __launch_bounds__(kBwdThreads, 1)
k_grouped_mm_bwd(const uint8_t* __restrict__ g, const uint8_t* __restrict__ packed,
                 const uint8_t* __restrict__ scales, const int32_t* __restrict__ offs, int experts,
                 int64_t tokens, int64_t ndim, int64_t kdim, uint8_t* __restrict__ out, int gx) {
  constexpr int BM = kBwdBM, BN = kBwdBN, MT = 4, NT = 2, kThreads = kBwdThreads;
  constexpr int GC = BM * 8 / kThreads;                // 16-byte grad_out chunks per thread and step
  // XCD-major remap: the workgroups the round-robin dispatch puts on XCD x
  // (linear id % 8 == x) take row slots x, x + 8, ..., each with all its
  // column tiles, so a row tile's grad_out is fetched into one L2 only
  // (one-dimensional grid of gx column tiles x a multiple of 8 row slots)
  const int64_t lin = blockIdx.x, kx = lin >> 3;
  const int slot_y = (int)((kx / gx) * 8 + (lin & 7));
  const int64_t col0 = (int64_t)(kx % gx) * BN;
  TileTable<BM> tt;
  tt.build(offs, experts, tokens);
  const TileInfo ti = tt.lookup(slot_y);
  if (ti.expert == -2) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, r = lane & 31;

  if (ti.expert == -1) {
    for (int i = threadIdx.x; i < BM * BN / 8; i += kThreads) {
      const int rr = i / (BN / 8), c = (i % (BN / 8)) * 8;
      const int64_t gr = ti.row0 + rr, gc = col0 + c;
      if (gr < ti.row_end && gc < kdim) {
        unsigned short* dst = reinterpret_cast<unsigned short*>(out + (gr * kdim + gc) * 2);
        for (int q = 0; q < 8 && gc + q < kdim; ++q) dst[q] = 0;
      }
    }
    return;
  }

  __shared__ __attribute__((aligned(1024))) BwdSmem sm;

  // grad_out: thread t owns chunks c = t + 512 i: tile row c / 8 = t / 8 + 64 i, chunk t % 8
  // the range covers this tile's rows only (an expert's whole segment could pass 2^31 bytes)
  const __amdgpu_buffer_rsrc_t rs_g =
      buf_rsrc(g + ti.row0 * ndim * 2, min(ti.row_end - ti.row0, (int64_t)BM) * ndim * 2);
  const int g_col = (threadIdx.x & 7) * 8;
  const uint32_t g_off0 = (uint32_t)((threadIdx.x >> 3) * ndim + g_col) * 2;
  const uint32_t g_row_step = (uint32_t)(64 * ndim * 2);
  u32x4_t gr_regs[GC];
  // the step moves the scalar offset only; lane offsets are fixed
  uint32_t g_voff[GC];
#pragma unroll
  for (int i = 0; i < GC; ++i) g_voff[i] = g_off0 + i * g_row_step;
  auto load_g = [&](int64_t n0) {
    // N % 8 == 0: a chunk is wholly in or out of range
    const bool ok = n0 + g_col < ndim;
    const uint32_t soff = (uint32_t)(min(n0, ndim) * 2);
#pragma unroll
    for (int i = 0; i < GC; ++i)
      gr_regs[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_g, ok ? g_voff[i] : kBufOob,
                                                                                     soff, 0));
  };
  // (row >> 1) & 7 of the rows t / 8 + 64 i does not depend on i
  const int g_st = (threadIdx.x >> 3) * 128 + 16 * ((threadIdx.x & 7) ^ ((threadIdx.x >> 4) & 7));
  auto store_g = [&](uint8_t* dst) {
#pragma unroll
    for (int i = 0; i < GC; ++i) *reinterpret_cast<u32x4_t*>(dst + g_st + i * 64 * 128) = gr_regs[i];
  };

  // weights: lane l of wave (wm, wn) takes row 32 wm + l / 2 of the step, column half l & 1
  const int wrow = 32 * wm + (lane >> 1), whalf = lane & 1;
  const int64_t kc = col0 + wn * 64;
  const bool wvalid = kc + 32 * (whalf + 1) <= kdim;             // K % 32 == 0: halves all in or all out
  const int64_t prow = kdim / 2, srow = kdim / 32;               // bytes per weight row (packed, scales)
  const __amdgpu_buffer_rsrc_t rs_w = buf_rsrc(packed_e_of(packed, ti.expert, ndim, kdim), ndim * prow);
  const __amdgpu_buffer_rsrc_t rs_s = buf_rsrc(scales + (int64_t)ti.expert * ndim * srow, ndim * srow);
  const uint32_t wcol = (uint32_t)(kc / 2 + 16 * whalf), scol = (uint32_t)(kc / 32 + whalf);
  const uint32_t w_voff = (uint32_t)(wrow * prow) + wcol, s_voff = (uint32_t)(wrow * srow) + scol;
  auto load_w = [&](WRaw& w, int64_t n0) {
    const bool ok = wvalid && n0 + wrow < ndim;
    const int64_t nc = min(n0, ndim);   // scalar offsets stay below the range (no 32-bit wrap)
    w.pk = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_w, ok ? w_voff : kBufOob,
                                                                             (uint32_t)(nc * prow), 0));
    w.sb = __builtin_amdgcn_raw_buffer_load_b8(rs_s, ok ? s_voff : kBufOob, (uint32_t)(nc * srow), 0);
  };
  const int wd_st = wrow * 128, wd_swz_row = wd_swz(wrow);
  // decode a piece (32 values) and write it into Wd, 16 bytes at a time
  auto put_piece = [&](const WRaw& w, uint8_t* wd) {
    const float sc = e8m0_to_f32(w.sb);
    const uint32_t w4[4] = {w.pk.x, w.pk.y, w.pk.z, w.pk.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4_t*>(wd + wd_st + 16 * ((4 * whalf + q) ^ wd_swz_row)) =
          u32x4_t{dec_fp4_bf16x2<0>(w4[q], sc), dec_fp4_bf16x2<1>(w4[q], sc), dec_fp4_bf16x2<2>(w4[q], sc),
                  dec_fp4_bf16x2<3>(w4[q], sc)};
  };
  // transposing-read addresses: group gq = lane / 16 -> h = gq / 2, column
  // half gq % 2; source lane s = lane % 16 -> row a = s / 4, columns 4 (s % 4).
  // Rows tr_row + 8 kk + 4 u: the swizzle depends on u only, so sub-step kk
  // is the immediate offset 1024 kk.
  const int gq = lane >> 4, sl = lane & 15;
  const int tr_row = 32 * (gq >> 1) + (sl >> 2);
  const int tr_col = 16 * (gq & 1) + 4 * (sl & 3);
  int tr_off[2][NT];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = tr_row + 4 * u, col = tr_col + 32 * j;
      tr_off[u][j] = n * 128 + 16 * ((col >> 3) ^ wd_swz(n)) + 2 * (col & 7);
    }

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16_t{};

  const int swz_g = (r >> 1) & 7;
  struct Frags { bf16x8_t fa[MT], fb[NT]; };
  auto read_frags = [&](Frags& f, const uint8_t* la, const uint8_t* wd, int kk) {
    const int off = 16 * ((4 * h + kk) ^ swz_g);
#pragma unroll
    for (int i = 0; i < MT; ++i) f.fa[i] = *reinterpret_cast<const bf16x8_t*>(la + i * 32 * 128 + off);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      v4i16_t t[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        t[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(wd + tr_off[u][j] + 1024 * kk));
      f.fb[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.fb[j], f.fa[i], acc[i][j], 0, 0, 0);
  };

  const int nsteps = (int)((ndim + kBK - 1) / kBK);
  WRaw w0, w1;
  load_w(w1, 0);
  load_w(w0, kBK);
  load_g(0);
  put_piece(w1, sm.w[0][wn]);
  store_g(sm.g[0]);
  __syncthreads();
  // step s: MFMAs on the grad_out tile and Wd of buffer s & 1, with each
  // sub-step's fragments read one sub-step ahead.  All waves reach the LDS
  // at once after the barrier, so the first fragment reads go out before
  // the next step's global loads: grad_out of step s + 1 (through registers
  // into the other tile, stored behind sub-step 2) and the raw weights of
  // step s + 2 (into `nxt`).  `cur` holds the raw weights of step s + 1,
  // fetched a step earlier and decoded into the other Wd buffer behind
  // sub-step 1.  Both buffers of step s + 1 were last read in step s - 1,
  // so the barrier that ends step s is the only one.  Loads past the last
  // step read zeros.
  auto step = [&](WRaw& cur, WRaw& nxt, int s) {
    const uint8_t* la = sm.g[s & 1] + (128 * wm + r) * 128;
    const uint8_t* wd = sm.w[s & 1][wn];
    Frags f[2];
    read_frags(f[0], la, wd, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) read_frags(f[(kk + 1) & 1], la, wd, kk + 1);
      mfmas(f[kk & 1]);
      if (kk == 0) {
        __builtin_amdgcn_sched_barrier(0);
        load_g((int64_t)(s + 1) * kBK);
        load_w(nxt, (int64_t)(s + 2) * kBK);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kk == 1) put_piece(cur, sm.w[(s & 1) ^ 1][wn]);
      if (kk == 2) {
        // the grad_out loads issued after sub-step 0 have had two sub-steps
        __builtin_amdgcn_sched_barrier(0);
        store_g(sm.g[(s & 1) ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  };
  for (int s = 0; s < nsteps; s += 2) {
    step(w0, w1, s);
    if (s + 1 < nsteps) step(w1, w0, s + 1);
  }

  // the last step's barrier has retired every read of the tiles
  static_assert(sizeof(BwdSmem) >= (size_t)8 * 128 * 128, "epilogue block fits");
  store_block_lds<MT>(reinterpret_cast<uint8_t*>(&sm) + wave * 128 * 128, acc, lane, out, kdim, ti.row0 + 128 * wm,
                      ti.row_end, col0 + wn * 64, kdim);
}

// ------------------------------------------------------------------ launcher
static int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return n;
}

// One-dimensional grids of column tiles x row slots (the dispatch order of
// the x-major two-dimensional grid, without its 65535 limit on slots); the
// hardware counts a grid's work-items in 32 bits.
static bool grid_fits(int64_t workgroups, int threads) {
  return workgroups > 0 && workgroups * threads < (int64_t(1) << 32);
}

hipError_t launch_grouped_mm(bool bwd, const void* a, int64_t tokens, const int8_t* packed, const uint8_t* scales,
                             int64_t experts, int64_t wn_dim, int64_t wk_dim, const int32_t* offs, void* out,
                             hipStream_t st) {
  if (!bwd) {
    const int64_t gx = (wn_dim + kFwdBN - 1) / kFwdBN;
    const int64_t gy = (tokens + kFwdBM - 1) / kFwdBM + experts;   // 128-row tiles
    if (wk_dim % 128 == 0 && wk_dim < (int64_t(1) << 22) && wn_dim * (wk_dim / 2) < (int64_t(1) << 31) &&
        ((uintptr_t)scales & 3) == 0) {
      // scale bytes in 8-step chunks when whole chunks exist (16-byte aligned
      // rows); 128 x 256 tiles of 4 waves, two per CU (measured faster on
      // the routed-expert layer than 128 x 512 tiles of 8 waves, one per CU:
      // +2% gate/up, +2% down).  96-row tiles when they take no more rounds
      // of two workgroups per CU: the same rounds, each 3/4 as long (a
      // problem of 288 tiles of 128 rows on 256 CUs leaves 32 CUs running two
      // while 384 tiles of 96 rows spread evenly)
      const bool sch8 = wk_dim % 512 == 0 && ((uintptr_t)scales & 15) == 0;
      const int cus = device_cus();
      const int64_t slots = 2 * (int64_t)(cus > 0 ? cus : 256);
      const int64_t gy96 = (tokens + 95) / 96 + experts;
      const bool bm96 = (gx * gy96 + slots - 1) / slots <= (gx * gy + slots - 1) / slots;
      const int64_t n128 = gx * gy, n96 = gx * gy96;
      if (!grid_fits(bm96 ? n96 : n128, kGemmThreads)) return hipErrorInvalidConfiguration;
#define MXQ_FWD_LAUNCH(BM, SCH, NWG)                                                                               \
  hipLaunchKernelGGL((k_grouped_mm_fwd_dma<BM, 4, 3, 2, SCH, true>), dim3((unsigned)(NWG)), dim3(kGemmThreads), 0, st, \
                     (const uint8_t*)a, (const uint8_t*)packed, scales, offs, (int)experts, tokens, wn_dim, wk_dim,      \
                     (uint8_t*)out, (int)gx)
      if (bm96) {
        if (sch8) MXQ_FWD_LAUNCH(96, 8, n96);
        else MXQ_FWD_LAUNCH(96, 2, n96);
      } else {
        if (sch8) MXQ_FWD_LAUNCH(128, 8, n128);
        else MXQ_FWD_LAUNCH(128, 2, n128);
      }
#undef MXQ_FWD_LAUNCH
      return hipGetLastError();
    }
    if (!grid_fits(gx * gy, kGemmThreads)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_grouped_mm_fwd_general, dim3((unsigned)(gx * gy)), dim3(kGemmThreads), 0, st,
                       (const uint8_t*)a, (const uint8_t*)packed, scales, offs, (int)experts, tokens, wn_dim, wk_dim,
                       (uint8_t*)out, (int)gx);
    return hipGetLastError();
  }
  {
    const int64_t gx = (wk_dim + kBwdBN - 1) / kBwdBN;
    const int64_t gy = ((tokens + kBwdBM - 1) / kBwdBM + experts + 7) / 8 * 8;
    if (!grid_fits(gx * gy, kBwdThreads)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_grouped_mm_bwd, dim3((unsigned)(gx * gy)), dim3(kBwdThreads), 0, st, (const uint8_t*)a,
                       (const uint8_t*)packed, scales, offs, (int)experts, tokens, wn_dim, wk_dim, (uint8_t*)out,
                       (int)gx);
    return hipGetLastError();
  }
}

hipError_t launch_grouped_mm_w4a4(const void* xq, const uint8_t* xs, int64_t tokens, const int8_t* packed,
                                  const uint8_t* scales, int64_t experts, int64_t n, int64_t k, const int32_t* offs,
                                  void* out, hipStream_t st) {
  const int64_t gx = (n + kW4BN - 1) / kW4BN;
  const int64_t gy = (tokens + kW4BM - 1) / kW4BM + experts;
  if (!grid_fits(gx * gy, kW4Threads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_grouped_mm_fwd_w4a4, dim3((unsigned)(gx * gy)), dim3(kW4Threads), 0, st, (const uint8_t*)xq, xs,
                     (const uint8_t*)packed, scales, offs, (int)experts, tokens, n, k, (uint8_t*)out, (int)gx);
  return hipGetLastError();
}

}  // namespace mxq
