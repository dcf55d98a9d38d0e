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
// first step.  With more than 64 experts the lookup runs the same scans
// over chunks of 64 experts, carrying the running end and tile count from
// one chunk to the next, until the chunk holding the slot.
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

  // more than 64 experts: chunk c of the experts is scanned as build() scans
  // the first 64, its ends offset by the running end of the chunks before
  // (a running maximum) and its tile counts by their total
  __device__ __forceinline__ TileInfo lookup_chunked(int slot) const {
    const int lane = threadIdx.x & 63;
    int run_end = 0, run_tiles = 0;
    for (int c0 = 0; c0 < experts; c0 += 64) {
      const int n = min(experts - c0, 64);
      const int v = wave_scan<true>(lane < n ? max(offs[c0 + lane], 0) : 0);
      const int e_end = (int)min((int64_t)max(v, run_end), tokens);
      int prev = __shfl_up(e_end, 1);
      if (lane == 0) prev = run_end;
      const int inc = run_tiles + wave_scan<false>(lane < n ? (int)(((int64_t)e_end - prev + BM - 1) / BM) : 0);
      const uint64_t live = n == 64 ? ~0ull : ((1ull << n) - 1);
      const uint64_t m = __ballot(inc > slot) & live;
      if (m) {
        const int e = __builtin_ctzll(m);
        const int before = e ? __builtin_amdgcn_readlane(inc, e - 1) : run_tiles;
        const int start = e ? __builtin_amdgcn_readlane(e_end, e - 1) : run_end;
        return TileInfo{start + (int64_t)(slot - before) * BM, __builtin_amdgcn_readlane(e_end, e), c0 + e};
      }
      run_end = __builtin_amdgcn_readlane(e_end, n - 1);
      run_tiles = __builtin_amdgcn_readlane(inc, n - 1);
    }
    const int64_t z = run_end + (int64_t)(slot - run_tiles) * BM;
    if (z < tokens) return TileInfo{z, tokens, -1};
    return TileInfo{0, 0, -2};
  }

  // which expert and row range a row-tile slot covers (-1: rows no expert
  // owns, to be zeroed; -2: nothing to do); every lane active
  __device__ __forceinline__ TileInfo lookup(int slot) const {
    if (experts > 64) return lookup_chunked(slot);
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
  // The same tiles in another slot order, for a grid that runs in one round
  // with at most two workgroups per CU: the dispatcher places linear ids 0 ..
  // CUs-1 one per CU and id CUs + j on id j's CU, so tiles are ordered by
  // descending count of 32-row blocks (the whole tiles and the segment tails
  // of BM/32 blocks first, then the tails of fewer blocks), experts ascending
  // within a count: the short tails come last and share CUs with whole
  // tiles.  The zero-fill slots follow as in lookup().  At most 64 experts
  // (more take lookup()'s order).
  __device__ __forceinline__ TileInfo lookup_by_height(int slot) const {
    if (experts > 64) return lookup_chunked(slot);
    constexpr int MB = BM / 32;
    int start = __shfl_up(end, 1);
    if ((threadIdx.x & 63) == 0) start = 0;
    const int rows = end - start;   // 0 on lanes past the experts
    const int nfull = rows / BM, tb = (rows % BM + 31) / 32;
    int s = slot;
#pragma unroll
    for (int b = MB; b >= 1; --b) {
      const int c = (b == MB ? nfull : 0) + (tb == b ? 1 : 0);
      const int inc = wave_scan<false>(c);
      const int tot = __builtin_amdgcn_readlane(inc, 63);
      if (s < tot) {
        const int e = __builtin_ctzll(__ballot(inc > s));
        const int k = s - __builtin_amdgcn_readlane(inc - c, e);   // tile k of expert e in this count
        const int64_t row0 = __builtin_amdgcn_readlane(start, e) +
                             (int64_t)(b == MB ? k : __builtin_amdgcn_readlane(nfull, e)) * BM;
        return TileInfo{row0, __builtin_amdgcn_readlane(end, e), e};
      }
      s -= tot;
    }
    const int64_t z = __builtin_amdgcn_readlane(end, 63) + (int64_t)s * BM;
    if (z < tokens) return TileInfo{z, tokens, -1};
    return TileInfo{0, 0, -2};
  }
};

// Rows no expert owns (a zero-fill slot of the tile table) are written as
// zeros: the BM x BN tile at (row0, col0), rows below row_end, columns below
// ndim, by every thread of the workgroup.
template <int BM, int BN>
__device__ __forceinline__ void zero_tile(const TileInfo& ti, int64_t col0, uint8_t* __restrict__ out, int64_t ndim) {
  for (int i = threadIdx.x; i < BM * BN / 8; i += blockDim.x) {
    const int rr = i / (BN / 8), c = (i % (BN / 8)) * 8;
    const int64_t gr = ti.row0 + rr, gc = col0 + c;
    if (gr < ti.row_end && gc < ndim) {
      unsigned short* dst = reinterpret_cast<unsigned short*>(out + (gr * ndim + gc) * 2);
      for (int q = 0; q < 8 && gc + q < ndim; ++q) dst[q] = 0;
    }
  }
}

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
// a lane offset past every range used here (the lane reads zeros); the range
// check covers the lane offset, so a transfer whose scalar offset moves it
// to other rows takes this offset for blocks past the valid rows
constexpr uint32_t kBufOob = 0x80000000u;

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
    zero_tile<BM, BN>(ti, col0, out, ndim);
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

// ------------------------------------------------ forward, whole weight lines
// BM x 256 tiles (BM = 128 or 96) of 4 waves, two workgroups per CU (their
// waves share the SIMDs, so one's barrier and memory waits overlap the
// other's MFMAs), with every weight transfer a whole 128-byte line.  A
// weight row holds 256 reduction indices (4 steps) per line; a forward that
// fetches only the 32 bytes of a step makes the L1 move the whole line from
// L2 each time -- for the routed-expert gate/up projection (7.7 TFLOP) that
// was 98 GB of L1 <- L2 traffic, two thirds of it weight lines, against 60 GB
// for a dense bf16 library GEMM of the same shape.  MI355X runs these GEMMs
// at its board power limit, where the clock, and so the rate, follows the
// energy spent per flop, and data moved between the caches is a large share
// of it; with whole lines the traffic falls to 45 GB.
//  * Activations: two stages of BM x 64 bf16; the stage step s - 1 used
//    takes step s + 1 right after the barrier that ends step s - 1.
//  * Weights: each wave owns its 64 columns.  A "generation" of 4 steps (64
//    columns x 128 bytes, each DMA lane moving 16 bytes of a line, 8 lanes a
//    whole line; chunk c of column n at c ^ ((n >> 1) & 7)) lands in the
//    wave's own LDS area; at its first step the wave copies its 32 bytes per
//    step and column into registers and then fetches the next generation
//    into the same area, four steps ahead of its use.  No other wave reads
//    the area, so this needs no barrier.
//  * Scales: 16 bytes (8 steps) per column, double-buffered per wave.
// The end of step s waits for exactly this wave's activation transfers of
// step s + 1 (s_waitcnt vmcnt; the generation and scale chunk issued after
// them stay in flight), then the barrier publishes every wave's.
// Needs K % 512 == 0 (whole generations and scale chunks).
constexpr int kFlBN = 256, kFlThreads = 256;

template <int BM>
struct FlSmem {
  uint8_t a[2][BM * 128];              // activation tiles: BM rows x 128 bytes
  uint8_t b[4][64 * 128];              // weight generation per wave: 64 columns x 128 bytes
  uint8_t s8[2][kFlBN * 16];           // E8M0 scales: 16 bytes (8 steps) per column
};

// (the body is a device function template called by one kernel per tile
// height: clang emitted no host launch stub for it as a kernel template)
// MTA: the tile's 32-row blocks that hold rows of its expert (1 .. BM/32);
// the blocks past them take no activation transfers, fragment reads or MFMAs.
// Wave `wave` adds the whole reduction for its 64 columns into acc, through
// the LDS block sm; the caller stores acc.
template <int BM, int MTA>
__device__ __forceinline__ void fwd_fl_body(const uint8_t* __restrict__ a, const uint8_t* __restrict__ packed,
                                            const uint8_t* __restrict__ scales, int64_t ndim, int64_t kdim,
                                            const TileInfo ti, const int64_t col0, FlSmem<BM>& sm,
                                            const int wave, f32x16_t (&acc)[BM / 32][2]) {
  constexpr int MT = BM / 32, NT = 2, QA = BM / 32;   // QA: activation blocks per wave
  static_assert(MTA >= 1 && MTA <= MT && QA == 4, "active row blocks; wave w fills row block w");
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;


  // activations: wave w fills blocks QA w .. QA w + QA - 1 of 8 rows (as in the DMA forward)
  const int64_t prow = kdim / 2, srow = kdim / 32;
  const __amdgpu_buffer_rsrc_t rs_a = dma_rsrc(a + ti.row0 * kdim * 2, min(ti.row_end - ti.row0, (int64_t)BM) * kdim * 2);
  uint32_t a_off[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int row = 8 * (QA * wave + q) + (lane >> 3);
    a_off[q] = (uint32_t)(((int64_t)row * kdim + ((lane & 7) ^ ((row >> 1) & 7)) * 8) * 2);
  }
  // this wave's 64 weight columns: block q (q = 0 .. 7) holds columns 8q .. 8q+7,
  // lane l -> column 8q + l/8, LDS chunk l%8 <- line chunk (l%8) ^ ((column >> 1) & 7)
  const int64_t n0 = col0 + 64 * wave;
  const __amdgpu_buffer_rsrc_t rs_b =
      dma_rsrc(packed_e_of(packed, ti.expert, ndim, kdim) + n0 * prow, (ndim - n0) * prow);
  // (column 8q + bc: ((8q + bc) >> 1) & 7 = (bc >> 1) ^ 4 (q & 1), so even and odd blocks differ in one swizzle bit)
  const int bc = lane >> 3;   // column within a block
  const uint32_t b_off[2] = {(uint32_t)(bc * prow + 16 * ((lane & 7) ^ (bc >> 1))),
                             (uint32_t)(bc * prow + 16 * ((lane & 7) ^ (bc >> 1) ^ 4))};
  const uint32_t b_blk = (uint32_t)(8 * prow);   // 8 columns further
  // scales of this wave's columns: lane l <- column 64 w + l
  const __amdgpu_buffer_rsrc_t rs_s = dma_rsrc(scales + ((int64_t)ti.expert * ndim + n0) * srow, (ndim - n0) * srow);
  const uint32_t s_off = (uint32_t)(lane * srow);

  auto issue_a = [&](int step) {
    if (MTA < MT && wave >= MTA) return;
#pragma unroll
    for (int q = 0; q < QA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void_t*)(sm.a[step & 1] + 1024 * (QA * wave + q)), 16,
                                               a_off[q], step * kBK * 2, 0, 0);
  };
  auto issue_b = [&](int gen) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void_t*)(sm.b[wave] + 1024 * q), 16,
                                               n0 + 8 * q < ndim ? b_off[q & 1] : kBufOob,
                                               gen * 128 + q * b_blk, 0, 0);   // block q: a scalar offset
  };
  auto issue_s = [&](int chunk) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s, (lds_void_t*)(sm.s8[chunk & 1] + 1024 * wave), 16, s_off,
                                             16 * chunk, 0, 0);
  };

  const int nsteps = (int)(kdim / kBK), last = nsteps - 1;   // a multiple of 8
  const int ngen = nsteps >> 2, nchunk = nsteps >> 3;

  issue_s(0);
  issue_b(0);
  issue_a(0);
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);   // vmcnt(0)
  __syncthreads();

  const uint8_t* bw = sm.b[wave];
  u32x4_t pw[NT][4];   // the generation's packed bytes: [column tile][step in generation]
  const int swz_base = r * 128;
  // t = s % 4, passed as a literal: after inlining it indexes the
  // generation's registers at compile time
  auto step = [&](int s, int t) {
    __builtin_amdgcn_sched_barrier(0);
    if (t == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int c = 32 * j + r;
          pw[j][u] = *reinterpret_cast<const u32x4_t*>(bw + c * 128 + 16 * ((2 * u + h) ^ ((c >> 1) & 7)));
        }
    }
    // the stage step s - 1 used is free (barrier that ended it): step s + 1
    const bool refill = s + 1 <= last;
    if (refill) issue_a(s + 1);
    bool gen_issue = false, chunk_issue = false;
    if (t == 0) {
      gen_issue = (s >> 2) + 1 < ngen;
      chunk_issue = (s & 7) == 0 && (s >> 3) + 1 < nchunk;
      // the generation's copy has been read before the area is refilled
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      if (gen_issue) issue_b((s >> 2) + 1);
      if (chunk_issue) issue_s((s >> 3) + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    // decode this step's weights into B fragments
    bf16x8_t fb[NT][4];
    {
      const uint8_t* sc_row = sm.s8[(s >> 3) & 1] + 2 * (s & 7) + h;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float sc = e8m0_to_f32(sc_row[16 * (64 * wave + 32 * j + r)]);
        const u32x4_t p = pw[j][t];
        const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          u32x4_t v = {dec_fp4_bf16x2<0>(w[kk], sc), dec_fp4_bf16x2<1>(w[kk], sc), dec_fp4_bf16x2<2>(w[kk], sc),
                       dec_fp4_bf16x2<3>(w[kk], sc)};
          fb[j][kk] = __builtin_bit_cast(bf16x8_t, v);
        }
      }
    }
    const uint8_t* la = sm.a[s & 1] + swz_base;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int off = 16 * ((4 * h + kk) ^ ((r >> 1) & 7));   // rows 32i + r share the swizzle
      bf16x8_t fa[MTA];
#pragma unroll
      for (int i = 0; i < MTA; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(la + i * 32 * 128 + off);
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j][kk], fa[i], acc[i][j], 0, 0, 0);
    }
    if (s == last) return;
    // step s+1's activations (and everything older) have landed once only the
    // generation and scale chunk issued after them may be in flight
    const int pend = (gen_issue ? 8 : 0) + (chunk_issue ? 1 : 0);
    __builtin_amdgcn_sched_barrier(0);
    switch (pend) {
      case 9: wait_vmcnt_barrier<9>(); break;
      case 8: wait_vmcnt_barrier<8>(); break;
      case 1: wait_vmcnt_barrier<1>(); break;
      default: wait_vmcnt_barrier<0>(); break;
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int s = 0; s < nsteps; s += 4) {   // nsteps % 8 == 0
    step(s, 0);
    step(s + 1, 1);
    step(s + 2, 2);
    step(s + 3, 3);
  }
  // nothing is pending after the last step's wait
}

// The 96-row form with a three-slot activation ring (76 KB: still two
// workgroups per CU; 128-row tiles would need 88 KB): activations get two
// steps of lead and generations three, as in the W4A8 forward.  On the
// 8-expert forward (before its height-ordered 128-row grid), bit-identical,
// 73.5 -> 72.1 us against the two-slot
// body.
template <int BM>
struct Fl3Smem {
  uint8_t a[3][BM * 128];              // activation ring: BM rows x 128 bytes per step
  uint8_t b[4][64 * 128];              // weight generation per wave: 64 columns x 128 bytes
  uint8_t s8[2][kFlBN * 16];           // E8M0 scales: 16 bytes (8 steps) per column
};
static_assert(sizeof(Fl3Smem<96>) <= 80 * 1024, "two workgroups per CU");

template <int BM>
__device__ __forceinline__ void fwd_fl3_body(const uint8_t* __restrict__ a, const uint8_t* __restrict__ packed,
                                            const uint8_t* __restrict__ scales, const int32_t* __restrict__ offs,
                                            int experts, int64_t tokens, int64_t ndim, int64_t kdim,
                                            uint8_t* __restrict__ out, int gx) {
  constexpr int BN = kFlBN, MT = BM / 32, NT = 2, QA = BM / 32;   // QA: activation blocks per wave
  const int64_t col0 = (int64_t)(blockIdx.x % gx) * BN;
  TileTable<BM> tt;
  tt.build(offs, experts, tokens);
  const TileInfo ti = tt.lookup((int)(blockIdx.x / gx));
  if (ti.expert == -2) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, r = lane & 31;

  if (ti.expert == -1) {
    zero_tile<BM, BN>(ti, col0, out, ndim);
    return;
  }

  __shared__ __attribute__((aligned(1024))) Fl3Smem<BM> sm;

  // activations: wave w fills blocks QA w .. QA w + QA - 1 of 8 rows (as in the DMA forward)
  const int64_t prow = kdim / 2, srow = kdim / 32;
  const __amdgpu_buffer_rsrc_t rs_a = dma_rsrc(a + ti.row0 * kdim * 2, min(ti.row_end - ti.row0, (int64_t)BM) * kdim * 2);
  uint32_t a_off[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int row = 8 * (QA * wave + q) + (lane >> 3);
    a_off[q] = (uint32_t)(((int64_t)row * kdim + ((lane & 7) ^ ((row >> 1) & 7)) * 8) * 2);
  }
  // this wave's 64 weight columns: block q (q = 0 .. 7) holds columns 8q .. 8q+7,
  // lane l -> column 8q + l/8, LDS chunk l%8 <- line chunk (l%8) ^ ((column >> 1) & 7)
  const int64_t n0 = col0 + 64 * wave;
  const __amdgpu_buffer_rsrc_t rs_b =
      dma_rsrc(packed_e_of(packed, ti.expert, ndim, kdim) + n0 * prow, (ndim - n0) * prow);
  // (column 8q + bc: ((8q + bc) >> 1) & 7 = (bc >> 1) ^ 4 (q & 1), so even and odd blocks differ in one swizzle bit)
  const int bc = lane >> 3;   // column within a block
  const uint32_t b_off[2] = {(uint32_t)(bc * prow + 16 * ((lane & 7) ^ (bc >> 1))),
                             (uint32_t)(bc * prow + 16 * ((lane & 7) ^ (bc >> 1) ^ 4))};
  const uint32_t b_blk = (uint32_t)(8 * prow);   // 8 columns further
  // scales of this wave's columns: lane l <- column 64 w + l
  const __amdgpu_buffer_rsrc_t rs_s = dma_rsrc(scales + ((int64_t)ti.expert * ndim + n0) * srow, (ndim - n0) * srow);
  const uint32_t s_off = (uint32_t)(lane * srow);

  auto issue_a = [&](int slot, int step) {
#pragma unroll
    for (int q = 0; q < QA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void_t*)(sm.a[slot] + 1024 * (QA * wave + q)), 16,
                                               a_off[q], step * kBK * 2, 0, 0);
  };
  auto issue_b = [&](int gen) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void_t*)(sm.b[wave] + 1024 * q), 16,
                                               n0 + 8 * q < ndim ? b_off[q & 1] : kBufOob,
                                               gen * 128 + q * b_blk, 0, 0);   // block q: a scalar offset
  };
  auto issue_s = [&](int slot, int chunk) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s, (lds_void_t*)(sm.s8[slot] + 1024 * wave), 16, s_off,
                                             16 * chunk, 0, 0);
  };

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16_t{};

  const int nsteps = (int)(kdim / kBK), last = nsteps - 1;   // a multiple of 8
  const int ngen = nsteps >> 2, nchunk = nsteps >> 3;

  issue_s(0, 0);
  issue_b(0);
  issue_a(0, 0);
  issue_a(1, 1);
  wait_vmcnt_barrier<QA>();   // all but step 1

  const uint8_t* bw = sm.b[wave];
  u32x4_t pw[NT][4];   // the generation's packed bytes: [column tile][step in generation]
  const int swz_base = r * 128;
  // T = s % 8 (a literal after inlining), t = T % 4: step within the
  // generation.  Three activation slots: after the barrier that ends step
  // s - 1, step s + 2 goes into that step's slot, first, then (t == 0) the
  // next generation and (T == 0) scale chunk, clamped at the end of the
  // line so that every step issues the same; each step ends by waiting for
  // step s + 1's activations.
  auto step = [&](int s, auto tc, auto lc) __attribute__((always_inline)) {
    constexpr int T = decltype(tc)::value, t = T & 3;
    constexpr bool kLast = decltype(lc)::value;
    __builtin_amdgcn_sched_barrier(0);
    if (t == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int c = 32 * j + r;
          pw[j][u] = *reinterpret_cast<const u32x4_t*>(bw + c * 128 + 16 * ((2 * u + h) ^ ((c >> 1) & 7)));
        }
    }
    if constexpr (!kLast) {
      issue_a((s + 2) % 3, min(s + 2, last));
      if constexpr (t == 0) {
        // the generation's copy has been read before the area is refilled
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        issue_b(min((s >> 2) + 1, ngen - 1));
        if constexpr (T == 0) issue_s(((s >> 3) + 1) & 1, min((s >> 3) + 1, nchunk - 1));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t fb[NT][4];
    {
      const uint8_t* sc_row = sm.s8[(s >> 3) & 1] + 2 * (s & 7) + h;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float sc = e8m0_to_f32(sc_row[16 * (64 * wave + 32 * j + r)]);
        const u32x4_t p = pw[j][t];
        const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          u32x4_t v = {dec_fp4_bf16x2<0>(w[kk], sc), dec_fp4_bf16x2<1>(w[kk], sc), dec_fp4_bf16x2<2>(w[kk], sc),
                       dec_fp4_bf16x2<3>(w[kk], sc)};
          fb[j][kk] = __builtin_bit_cast(bf16x8_t, v);
        }
      }
    }
    const uint8_t* la = sm.a[s % 3] + swz_base;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int off = 16 * ((4 * h + kk) ^ ((r >> 1) & 7));
      bf16x8_t fa[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(la + i * 32 * 128 + off);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j][kk], fa[i], acc[i][j], 0, 0, 0);
    }
    if constexpr (!kLast) {
      // step s + 1's activations have landed when only what was issued after
      // them is in flight: step s - 1's generation and chunk (t == 0 there)
      // and this step's activations, generation and chunk
      constexpr int kG[8] = {9, 0, 0, 0, 8, 0, 0, 0};
      constexpr int kPend = kG[(T + 7) & 7] + QA + kG[T];
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_barrier<kPend>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using B0 = std::false_type;
  auto eight = [&](int s0, auto lc) __attribute__((always_inline)) {
    step(s0, std::integral_constant<int, 0>{}, B0{});
    step(s0 + 1, std::integral_constant<int, 1>{}, B0{});
    step(s0 + 2, std::integral_constant<int, 2>{}, B0{});
    step(s0 + 3, std::integral_constant<int, 3>{}, B0{});
    step(s0 + 4, std::integral_constant<int, 4>{}, B0{});
    step(s0 + 5, std::integral_constant<int, 5>{}, B0{});
    step(s0 + 6, std::integral_constant<int, 6>{}, B0{});
    step(s0 + 7, std::integral_constant<int, 7>{}, lc);
  };
  for (int s0 = 0; s0 < nsteps - 8; s0 += 8) eight(s0, B0{});
  eight(nsteps - 8, std::true_type{});
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);   // vmcnt(0): the clamped transfers of the last steps
  // nothing is pending after the last step's wait; once every wave is here the LDS is free
  __syncthreads();
  static_assert(sizeof(Fl3Smem<BM>) >= (size_t)4 * BM * 128, "epilogue block fits");
  store_block_lds<MT>(reinterpret_cast<uint8_t*>(&sm) + wave * BM * 128, acc, lane, out, ndim, ti.row0, ti.row_end,
                      col0 + 64 * wave, ndim);
}

// The 128-row whole-line forward.  BY_HEIGHT takes the slots in height
// order (TileTable::lookup_by_height), for a grid that runs in one round:
// on the 8-expert forward (288 tiles, 256 of full height) every CU then runs
// one full tile and the 32 one-block tails share CUs with the first 32.
// xr > 0 (one round, 8 xr CUs): the first 8 xr workgroups, one per CU, are
// taken XCD-major -- the dispatcher puts linear id i on XCD i % 8, which
// then runs logical ids (i % 8) xr .. (i % 8) xr + xr - 1, whole row tiles
// with all their column tiles, so each L2 fetches about one expert's
// weights and its share of the activations instead of every activation row
// for one column tile; the ids past them keep their places (and CU pairs).
template <bool BY_HEIGHT>
__device__ __forceinline__ void fwd_fl128(const uint8_t* __restrict__ a, const uint8_t* __restrict__ packed,
                                          const uint8_t* __restrict__ scales, const int32_t* __restrict__ offs,
                                          int experts, int64_t tokens, int64_t ndim, int64_t kdim,
                                          uint8_t* __restrict__ out, int gx, int xr) {
  constexpr int BM = 128, BN = kFlBN;
  const int bid = (xr > 0 && (int)blockIdx.x < 8 * xr) ? (int)(blockIdx.x & 7) * xr + (int)(blockIdx.x >> 3)
                                                        : (int)blockIdx.x;
  const int64_t col0 = (int64_t)(bid % gx) * BN;
  TileTable<BM> tt;
  tt.build(offs, experts, tokens);
  const int slot = bid / gx;
  const TileInfo ti = BY_HEIGHT ? tt.lookup_by_height(slot) : tt.lookup(slot);
  if (ti.expert == -2) return;
  if (ti.expert == -1) {
    zero_tile<BM, BN>(ti, col0, out, ndim);
    return;
  }
  // one LDS block for every instantiation below
  __shared__ __attribute__((aligned(1024))) FlSmem<BM> sm;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  f32x16_t acc[BM / 32][2];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) acc[i][0] = acc[i][1] = f32x16_t{};
  // a segment tail of fewer than BM rows runs only the 32-row blocks it fills
  switch ((int)((min(ti.row_end - ti.row0, (int64_t)BM) + 31) / 32)) {
    case 1: fwd_fl_body<BM, 1>(a, packed, scales, ndim, kdim, ti, col0, sm, wave, acc); break;
    case 2: fwd_fl_body<BM, 2>(a, packed, scales, ndim, kdim, ti, col0, sm, wave, acc); break;
    case 3: fwd_fl_body<BM, 3>(a, packed, scales, ndim, kdim, ti, col0, sm, wave, acc); break;
    default: fwd_fl_body<BM, 4>(a, packed, scales, ndim, kdim, ti, col0, sm, wave, acc); break;
  }
  // once every wave is here the LDS is free
  __syncthreads();
  static_assert(sizeof(FlSmem<BM>) >= (size_t)4 * BM * 128, "epilogue block fits");
  store_block_lds<BM / 32>(reinterpret_cast<uint8_t*>(&sm) + wave * BM * 128, acc, threadIdx.x & 63, out, ndim,
                           ti.row0, ti.row_end, col0 + 64 * wave, ndim);
}
__global__ void __launch_bounds__(kFlThreads, 2)
k_grouped_mm_fwd_fl128(const uint8_t* __restrict__ a, const uint8_t* __restrict__ packed,
                       const uint8_t* __restrict__ scales, const int32_t* __restrict__ offs, int experts,
                       int64_t tokens, int64_t ndim, int64_t kdim, uint8_t* __restrict__ out, int gx) {
  fwd_fl128<false>(a, packed, scales, offs, experts, tokens, ndim, kdim, out, gx, 0);
}
__global__ void __launch_bounds__(kFlThreads, 2)
k_grouped_mm_fwd_fl128_by_height(const uint8_t* __restrict__ a, const uint8_t* __restrict__ packed,
                                 const uint8_t* __restrict__ scales, const int32_t* __restrict__ offs, int experts,
                                 int64_t tokens, int64_t ndim, int64_t kdim, uint8_t* __restrict__ out, int gx,
                                 int xr) {
  fwd_fl128<true>(a, packed, scales, offs, experts, tokens, ndim, kdim, out, gx, xr);
}
__global__ void __launch_bounds__(kFlThreads, 2)
k_grouped_mm_fwd_fl96(const uint8_t* __restrict__ a, const uint8_t* __restrict__ packed,
                      const uint8_t* __restrict__ scales, const int32_t* __restrict__ offs, int experts,
                      int64_t tokens, int64_t ndim, int64_t kdim, uint8_t* __restrict__ out, int gx) {
  fwd_fl3_body<96>(a, packed, scales, offs, experts, tokens, ndim, kdim, out, gx);
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
// and its E8M0 block -- and the byte of its scale register that the
// instruction's byte select names scales that block (a 0xFF scale gives
// NaN).  So no code is decoded here: both operands go
// from global memory through LDS into the MFMA as stored.  Products of two
// e2m1 codes and two power-of-two scales are exact, sums run in fp32, the
// output rounds to bf16 nearest-even.
//
// Workgroup: BM x 256 tiles (BM = 128 or 96) of 4 waves, two workgroups per
// CU, wave w owning columns [64 w, +64) of the tile (BM/32 x 2 MFMA tiles
// computed transposed, weight fragment first, so the LDS-staged epilogue is
// the bf16 kernels').  Organised like the W4A8 forward, with every global
// transfer a whole 128-byte line; for fp4 a line of a row is 256 k, so:
//  * activations: a stage is 128 bytes (256 k) of each of the tile's rows,
//    two stages, 16-byte chunks swizzled by (row >> 1) & 7 as in the bf16
//    kernels (conflict-free 16-lane fragment reads);
//  * weights: per wave, a generation of 64 columns x 128 bytes (the same
//    256 k), copied into registers at the start of its stage, the area then
//    refilled with the next stage's generation;
//  * scales: 16 bytes (512 k = two stages) per row and per column,
//    double-buffered; a lane reads the 8 bytes of its stage once and the
//    MFMA's scale byte select picks each sub-step's block (dwords shifted
//    right by 8h, so the block of sub-step u sits in byte 2(u & 1) of dword
//    u / 2).
// A stage is 4 MFMA sub-steps of 64 k: per wave and stage the same bytes of
// LDS traffic per MFMA cycle as the W4A8 kernel's 128-k stage (at 96 rows,
// 24 fp4 MFMAs of 32 cycles against 12 fp8 x fp4 MFMAs of 64).  Each stage issues
// everything the next needs (scale chunk, weight generation, activation
// stage) and ends by waiting for it (vmcnt(0)) and the barrier.  Needs
// K % 512 == 0.
constexpr int kW4BN = 256, kW4Threads = 256;

template <int BM>
struct W4Smem {
  uint8_t a[2][BM * 128];             // activation stages: BM rows x 128 bytes (256 k of e2m1)
  uint8_t b[4][64 * 128];             // weight generation per wave: 64 columns x 128 bytes (256 k)
  uint8_t sa[2][128 * 16];            // activation scales: 16 bytes (512 k) per row (two 64-row transfers)
  uint8_t sb[2][kW4BN * 16];          // weight scales: 16 bytes (512 k) per column
};

typedef int v8i32_t __attribute__((ext_vector_type(8)));

// fp4 x fp4 block-scaled MFMA; SEL picks the scale byte of both scale operands
template <int SEL>
__device__ __forceinline__ f32x16_t mfma_w4(const u32x4_t& w, const u32x4_t& x, uint32_t sw, uint32_t sx,
                                            const f32x16_t& c) {
  const v8i32_t a = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  const v8i32_t b = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, SEL, (int)sw, SEL, (int)sx);
}

// (a device function template called by one kernel per tile height: clang
// emitted no host launch stub for it as a kernel template)
template <int BM>
__device__ __forceinline__ void w4a4_body(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                          const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
                                          const int32_t* __restrict__ offs, int experts, int64_t tokens, int64_t ndim,
                                          int64_t kdim, uint8_t* __restrict__ out, int gx) {
  constexpr int BN = kW4BN, MT = BM / 32, NT = 2, QA = BM / 32;
  const int64_t col0 = (int64_t)(blockIdx.x % gx) * BN;
  TileTable<BM> tt;
  tt.build(offs, experts, tokens);
  const TileInfo ti = tt.lookup((int)(blockIdx.x / gx));
  if (ti.expert == -2) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, r = lane & 31;

  if (ti.expert == -1) {
    zero_tile<BM, BN>(ti, col0, out, ndim);
    return;
  }

  __shared__ __attribute__((aligned(1024))) W4Smem<BM> sm;

  // buffers over this tile's rows and this wave's weight columns (reads past
  // them return zeros); ranges fit 31 bits (the launcher checks one expert's
  // packed weights, and K < 2^22)
  const int64_t prow = kdim / 2, srow = kdim / 32;
  const int64_t nrows = min(ti.row_end - ti.row0, (int64_t)BM);
  // activations: wave w fills blocks QA w .. QA w + QA - 1 of 8 rows (lane l ->
  // row 8b + l/8, LDS chunk l%8 <- line chunk (l%8) ^ ((row >> 1) & 7))
  const __amdgpu_buffer_rsrc_t rs_a = dma_rsrc(xq + ti.row0 * prow, nrows * prow);
  uint32_t a_off[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int row = 8 * (QA * wave + q) + (lane >> 3);
    a_off[q] = (uint32_t)(row * prow + 16 * ((lane & 7) ^ ((row >> 1) & 7)));
  }
  // activation scales: waves 0 and 1 move rows 64 w + lane (16 bytes each)
  const __amdgpu_buffer_rsrc_t rs_sa = dma_rsrc(xs + ti.row0 * srow, nrows * srow);
  const uint32_t sa_off = (uint32_t)((64 * (wave & 1) + lane) * srow);
  // weights: this wave's 64 columns, block q (0 .. 7) = columns 8q .. 8q+7,
  // lane l -> column 8q + l/8, LDS chunk l%8 <- line chunk (l%8) ^ (column >> 1 & 7)
  // (column 8q + c: ((8q + c) >> 1) & 7 = (c >> 1) ^ 4 (q & 1)); blocks past
  // n take an out-of-range lane offset (the block offset is a scalar offset)
  const int64_t n0 = col0 + 64 * wave;
  const __amdgpu_buffer_rsrc_t rs_b =
      dma_rsrc(packed_e_of(packed, ti.expert, ndim, kdim) + n0 * prow, (ndim - n0) * prow);
  const int bc = lane >> 3;
  const uint32_t b_off[2] = {(uint32_t)(bc * prow + 16 * ((lane & 7) ^ (bc >> 1))),
                             (uint32_t)(bc * prow + 16 * ((lane & 7) ^ (bc >> 1) ^ 4))};
  const uint32_t b_blk = (uint32_t)(8 * prow);
  // weight scales of this wave's columns: lane l <- column 64 w + l
  const __amdgpu_buffer_rsrc_t rs_sb = dma_rsrc(scales + ((int64_t)ti.expert * ndim + n0) * srow, (ndim - n0) * srow);
  const uint32_t sb_off = (uint32_t)(lane * srow);

  const int nst = (int)(kdim / 256);          // stages of 256 k; even (K % 512 == 0)
  const int nchunk = nst / 2;
  auto issue_a = [&](int st) {
#pragma unroll
    for (int q = 0; q < QA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void_t*)(sm.a[st & 1] + 1024 * (QA * wave + q)), 16,
                                               a_off[q], st * 128, 0, 0);
  };
  auto issue_b = [&](int gen) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void_t*)(sm.b[wave] + 1024 * q), 16,
                                               n0 + 8 * q < ndim ? b_off[q & 1] : kBufOob,
                                               gen * 128 + q * b_blk, 0, 0);
  };
  auto issue_scales = [&](int chunk) {
    if (wave < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_sa, (lds_void_t*)(sm.sa[chunk & 1] + 1024 * wave), 16, sa_off,
                                               16 * chunk, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_sb, (lds_void_t*)(sm.sb[chunk & 1] + 1024 * wave), 16, sb_off,
                                             16 * chunk, 0, 0);
  };

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16_t{};

  issue_scales(0);
  issue_b(0);
  issue_a(0);
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);   // vmcnt(0)
  __syncthreads();

  const int swz = (r >> 1) & 7;               // rows 32i + r share the chunk swizzle
  const uint32_t sh = 8u * (uint32_t)h;
  auto stage = [&](int s) {
    __builtin_amdgcn_sched_barrier(0);
    // this stage's weight generation and the 8 scale bytes (256 k) of every
    // column and row tile, landed by the last barrier
    u32x4_t pw[NT][4];
    uint32_t swb[NT][2], sxa[MT][2];
    const int sc_off = 8 * (s & 1);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int c = 32 * j + r;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pw[j][u] = *reinterpret_cast<const u32x4_t*>(sm.b[wave] + c * 128 + 16 * ((2 * u + h) ^ ((c >> 1) & 7)));
      const u32x2_t v = *reinterpret_cast<const u32x2_t*>(sm.sb[(s >> 1) & 1] + 16 * (64 * wave + c) + sc_off);
      swb[j][0] = v.x >> sh;
      swb[j][1] = v.y >> sh;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const u32x2_t v = *reinterpret_cast<const u32x2_t*>(sm.sa[(s >> 1) & 1] + 16 * (32 * i + r) + sc_off);
      sxa[i][0] = v.x >> sh;
      sxa[i][1] = v.y >> sh;
    }
    // everything the next stage needs: scale chunk, weight generation, activations
    if ((s & 1) == 0 && (s >> 1) + 1 < nchunk) issue_scales((s >> 1) + 1);
    if (s + 1 < nst) {
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the copy has read the generation's area
      issue_b(s + 1);
      issue_a(s + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    // sub-step u: the 32 k of block 2u + h of the stage (16-byte chunk 2u + h
    // of the row); each sub-step's fragments are read while the previous
    // sub-step's MFMAs run (two register sets)
    const uint8_t* la = sm.a[s & 1] + r * 128;
    u32x4_t fx[2][MT];
    auto read_fx = [&](u32x4_t (&f)[MT], int u) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
        f[i] = *reinterpret_cast<const u32x4_t*>(la + i * 32 * 128 + 16 * ((2 * u + h) ^ swz));
    };
    read_fx(fx[0], 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < 3) read_fx(fx[(u + 1) & 1], u + 1);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if ((u & 1) == 0)
            acc[i][j] = mfma_w4<0>(pw[j][u], fx[u & 1][i], swb[j][u >> 1], sxa[i][u >> 1], acc[i][j]);
          else
            acc[i][j] = mfma_w4<2>(pw[j][u], fx[u & 1][i], swb[j][u >> 1], sxa[i][u >> 1], acc[i][j]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    // all the next stage needs has landed (nothing is pending after the last
    // stage); unconditional, so that the MFMAs above stay ahead of it (behind
    // a branch the compiler moved them past the wait)
    __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);   // vmcnt(0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int s = 0; s < nst; ++s) stage(s);
  __syncthreads();
  static_assert(sizeof(W4Smem<BM>) >= (size_t)4 * BM * 128, "epilogue block fits");
  store_block_lds<MT>(reinterpret_cast<uint8_t*>(&sm) + wave * BM * 128, acc, lane, out, ndim, ti.row0, ti.row_end,
                      col0 + 64 * wave, ndim);
}

__global__ void __launch_bounds__(kW4Threads, 2)
k_grouped_mm_fwd_w4a4_128(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                          const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
                          const int32_t* __restrict__ offs, int experts, int64_t tokens, int64_t ndim, int64_t kdim,
                          uint8_t* __restrict__ out, int gx) {
  w4a4_body<128>(xq, xs, packed, scales, offs, experts, tokens, ndim, kdim, out, gx);
}
__global__ void __launch_bounds__(kW4Threads, 2)
k_grouped_mm_fwd_w4a4_96(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                         const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
                         const int32_t* __restrict__ offs, int experts, int64_t tokens, int64_t ndim, int64_t kdim,
                         uint8_t* __restrict__ out, int gx) {
  w4a4_body<96>(xq, xs, packed, scales, offs, experts, tokens, ndim, kdim, out, gx);
}

// ------------------------------------------------------------- forward, W4A8
// y[rows_e] = q8(x)[rows_e] @ W_e^T with the activations in fp8: E4M3 codes
// [T, K] with one E8M0 scale per 32 k [T, K/32], as quantize_cache_packed(x,
// "fp8", 32) stores them (the fp8 form of "nemo_automodel.components.models.
// deepseek_v41.quantization" quantize_cache; "NVIDIA Model Optimizer: from
// mtq.quantize to a 4.95-bit DeepSeek-R1", sections "NVFP4 in the code: two
// scales and a nibble" and "The claims, marked reported", for activation
// scales computed at run time and the W4A8 form).  Both operands go as
// stored into gfx950's block-scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4,
// weights (e2m1, 16 bytes per lane: column l % 32, the 32 k of block h =
// l / 32 of the 64-k sub-step) first, activations (E4M3, 32 bytes per lane:
// row l % 32, bytes 0-15 the 16 k of slice h and bytes 16-31 those of slice
// h + 2, slices of 16 k) second, each lane's E8M0 block scale in byte 0 of
// its scale operand.  This pairing of an 8-bit with a 4-bit operand was read
// off the one-hot parity test: with 32 consecutive k per lane the products
// of slices 1 and 2 were crossed.  Products of codes and power-of-two scales
// are exact, sums run in fp32, the output rounds to bf16 nearest-even.
//
// Organised like the whole-line bf16 forward: 96 x 256 tiles of 4 waves, two
// workgroups per CU, wave w owning columns [64 w, +64) of the tile (3 x 2
// MFMA tiles computed transposed).  Every global transfer is a whole
// 128-byte line:
//  * activations: a stage is 128 bytes (128 k) of each of the tile's 96
//    rows, a ring of three stages (12 KB each, 80 KB in all: still two
//    workgroups per CU), 16-byte chunks swizzled by (row >> 1) & 7 as in
//    the bf16 kernels;
//  * weights: per wave, a generation of 64 columns x 128 bytes (256 k = two
//    stages), copied into registers at its first stage, the area then
//    refilled with the next generation;
//  * scales: 16 bytes (512 k = four stages) per row and per column,
//    double-buffered.
// Stage s issues, after the barrier that ends stage s - 1, the activations
// of stage s + 2 (into stage s - 1's slot), then the next weight generation
// (even stages) and scale chunk (every fourth stage), and ends by waiting
// for what stage s + 1 needs, leaving its own transfers in flight: two
// stages of lead for the activations and the generations (one stage with
// a two-slot ring and a vmcnt(0) per stage measured 4% slower on gate/up
// and 2% on down, bit-identical).  Near the end of the line the transfers
// are clamped to the last stage, generation and chunk, into slots nothing
// reads again, so that every stage issues the same and its wait count is a
// constant.  Needs K % 512 == 0.
constexpr int kW8BM = 96, kW8BN = 256, kW8Threads = 256;

struct W8Smem {
  uint8_t a[3][kW8BM * 128];          // activation ring: 96 rows x 128 bytes (128 k of E4M3) per stage
  uint8_t b[4][64 * 128];             // weight generation per wave: 64 columns x 128 bytes (256 k)
  uint8_t sa[2][128 * 16];            // activation scales: 16 bytes (512 k) per row (two 64-row transfers)
  uint8_t sb[2][kW8BN * 16];          // weight scales: 16 bytes (512 k) per column
};
static_assert(sizeof(W8Smem) <= 80 * 1024, "two workgroups per CU");

__global__ void __launch_bounds__(kW8Threads, 2)
k_grouped_mm_fwd_w4a8(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                      const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
                      const int32_t* __restrict__ offs, int experts, int64_t tokens, int64_t ndim, int64_t kdim,
                      uint8_t* __restrict__ out, int gx) {
  constexpr int BM = kW8BM, BN = kW8BN, MT = BM / 32, NT = 2, QA = BM / 32;
  const int64_t col0 = (int64_t)(blockIdx.x % gx) * BN;
  TileTable<BM> tt;
  tt.build(offs, experts, tokens);
  const TileInfo ti = tt.lookup((int)(blockIdx.x / gx));
  if (ti.expert == -2) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, r = lane & 31;

  if (ti.expert == -1) {
    zero_tile<BM, BN>(ti, col0, out, ndim);
    return;
  }

  __shared__ __attribute__((aligned(1024))) W8Smem sm;

  const int64_t prow = kdim / 2, srow = kdim / 32;
  const int64_t nrows = min(ti.row_end - ti.row0, (int64_t)BM);
  // activations: wave w fills blocks QA w .. QA w + QA - 1 of 8 rows (lane l ->
  // row 8b + l/8, LDS chunk l%8 <- global chunk (l%8) ^ ((row >> 1) & 7));
  // ranges cover this tile's rows (reads past them return zeros)
  const __amdgpu_buffer_rsrc_t rs_a = dma_rsrc(xq + ti.row0 * kdim, nrows * kdim);
  uint32_t a_off[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int row = 8 * (QA * wave + q) + (lane >> 3);
    a_off[q] = (uint32_t)(row * kdim + 16 * ((lane & 7) ^ ((row >> 1) & 7)));
  }
  // activation scales: waves 0 and 1 move rows 64 w + lane (16 bytes each)
  const __amdgpu_buffer_rsrc_t rs_sa = dma_rsrc(xs + ti.row0 * srow, nrows * srow);
  const uint32_t sa_off = (uint32_t)((64 * (wave & 1) + lane) * srow);
  // weights: this wave's 64 columns, block q (0 .. 7) = columns 8q .. 8q+7,
  // lane l -> column 8q + l/8, LDS chunk l%8 <- line chunk (l%8) ^ (column >> 1 & 7)
  // (column 8q + c: ((8q + c) >> 1) & 7 = (c >> 1) ^ 4 (q & 1))
  const int64_t n0 = col0 + 64 * wave;
  const __amdgpu_buffer_rsrc_t rs_b =
      dma_rsrc(packed_e_of(packed, ti.expert, ndim, kdim) + n0 * prow, (ndim - n0) * prow);
  const int bc = lane >> 3;
  const uint32_t b_off[2] = {(uint32_t)(bc * prow + 16 * ((lane & 7) ^ (bc >> 1))),
                             (uint32_t)(bc * prow + 16 * ((lane & 7) ^ (bc >> 1) ^ 4))};
  const uint32_t b_blk = (uint32_t)(8 * prow);
  // weight scales of this wave's columns: lane l <- column 64 w + l
  const __amdgpu_buffer_rsrc_t rs_sb = dma_rsrc(scales + ((int64_t)ti.expert * ndim + n0) * srow, (ndim - n0) * srow);
  const uint32_t sb_off = (uint32_t)(lane * srow);

  const int nst = (int)(kdim / 128);          // stages of 128 k; a multiple of 4 (K % 512 == 0)
  const int ngen = nst / 2, nchunk = nst / 4;
  auto issue_a = [&](int slot, int st) {
#pragma unroll
    for (int q = 0; q < QA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void_t*)(sm.a[slot] + 1024 * (QA * wave + q)), 16,
                                               a_off[q], st * 128, 0, 0);
  };
  auto issue_b = [&](int gen) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void_t*)(sm.b[wave] + 1024 * q), 16,
                                               n0 + 8 * q < ndim ? b_off[q & 1] : kBufOob,
                                               gen * 128 + q * b_blk, 0, 0);   // block q: a scalar offset
  };
  auto issue_scales = [&](int slot, int chunk) {
    if (wave < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_sa, (lds_void_t*)(sm.sa[slot] + 1024 * wave), 16, sa_off,
                                               16 * chunk, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_sb, (lds_void_t*)(sm.sb[slot] + 1024 * wave), 16, sb_off,
                                             16 * chunk, 0, 0);
  };

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16_t{};

  issue_scales(0, 0);
  issue_b(0);
  issue_a(0, 0);
  issue_a(1, 1);
  wait_vmcnt_barrier<QA>();                   // all but stage 1

  u32x4_t pw[NT][4];                          // the generation's weight codes: [column tile][sub-step]
  uint32_t swb[NT][2];                        // the generation's 8 weight scale bytes per column tile
  const int swz = (r >> 1) & 7;               // rows 32i + r share the chunk swizzle
  // stage s (T = s % 4, a literal after inlining; g = T % 2: which half of
  // the generation).  Three activation slots: after the barrier that ends
  // stage s - 1 (every read of its slot done), stage s + 2 goes into that
  // slot, first, then the next generation (T even) and scale chunk (T == 0),
  // clamped at the end of the line so that every stage issues the same.
  // Each stage ends by waiting for stage s + 1's activations only.
  auto step = [&](int s, auto tc, auto lc) __attribute__((always_inline)) {
    constexpr int T = decltype(tc)::value, g = T & 1;
    constexpr bool kLast = decltype(lc)::value;
    __builtin_amdgcn_sched_barrier(0);
    if (g == 0) {
      // copy generation s / 2 and its scale bytes (landed by the last barrier)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int c = 32 * j + r;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          pw[j][u] = *reinterpret_cast<const u32x4_t*>(sm.b[wave] + c * 128 + 16 * ((2 * u + h) ^ ((c >> 1) & 7)));
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(sm.sb[(s >> 2) & 1] + 16 * (64 * wave + c) +
                                                            8 * ((s >> 1) & 1));
        swb[j][0] = v.x;
        swb[j][1] = v.y;
      }
    }
    uint32_t sxa[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
      sxa[i] = *reinterpret_cast<const uint32_t*>(sm.sa[(s >> 2) & 1] + 16 * (32 * i + r) + 4 * (s & 3));
    if constexpr (!kLast) {
      issue_a((s + 2) % 3, min(s + 2, nst - 1));
      if constexpr (g == 0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the copy has read the area
        issue_b(min((s >> 1) + 1, ngen - 1));
      }
      if constexpr (T == 0) issue_scales(((s >> 2) + 1) & 1, min((s >> 2) + 1, nchunk - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* la = sm.a[s % 3] + r * 128;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      v8i32_t fx[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(la + i * 32 * 128 + 16 * ((4 * u + h) ^ swz));
        const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(la + i * 32 * 128 + 16 * ((4 * u + 2 + h) ^ swz));
        fx[i] = v8i32_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      }
      const int wu = 2 * g + u;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const u32x4_t p = pw[j][wu];
        const v8i32_t w = {(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
        const uint32_t sw = (swb[j][(2 * wu + h) >> 2] >> (8 * ((2 * wu + h) & 3))) & 0xFFu;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const uint32_t sx = (sxa[i] >> (8 * (2 * u + h))) & 0xFFu;
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, fx[i], acc[i][j], 4, 0, 0, (int)sw, 0,
                                                                       (int)sx);
        }
      }
    }
    if constexpr (!kLast) {
      // stage s + 1 has landed, and so has everything stage s - 1 issued
      // (its generation is copied at stage s + 1, its scales later): only
      // what this stage issued may stay in flight, its activations (QA), and
      // on even stages its generation (8) and on T == 0 its scales (2 on
      // waves 0 and 1, else 1)
      constexpr int kThis = QA + ((T & 1) == 0 ? 8 : 0);
      __builtin_amdgcn_sched_barrier(0);
      if (T == 0 && wave < 2) wait_vmcnt_barrier<kThis + 2>();
      else if (T == 0) wait_vmcnt_barrier<kThis + 1>();
      else wait_vmcnt_barrier<kThis>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using B0 = std::false_type;
  auto four = [&](int s0, auto lc) __attribute__((always_inline)) {
    step(s0, std::integral_constant<int, 0>{}, B0{});
    step(s0 + 1, std::integral_constant<int, 1>{}, B0{});
    step(s0 + 2, std::integral_constant<int, 2>{}, B0{});
    step(s0 + 3, std::integral_constant<int, 3>{}, lc);
  };
  for (int s0 = 0; s0 < nst - 4; s0 += 4) four(s0, B0{});
  four(nst - 4, std::true_type{});
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);   // vmcnt(0): the clamped transfers of the last stages
  __syncthreads();
  static_assert(sizeof(W8Smem) >= (size_t)4 * BM * 128, "epilogue block fits");
  store_block_lds<MT>(reinterpret_cast<uint8_t*>(&sm) + wave * BM * 128, acc, lane, out, ndim, ti.row0, ti.row_end,
                      col0 + 64 * wave, ndim);
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
//    (n & 3) + 4 * ((n >> 1) & 1).  A 16-byte LDS write serves 8 lanes (128
//    bytes) per cycle, a transposing read 32 lanes (256 bytes): the piece
//    writes' 8 lanes (4 consecutive rows, both column halves: chunks q ^ s
//    and (q + 4) ^ s) need s mod 4 distinct over 4 consecutive rows, and
//    the transposing reads (rows n, n + 2 of one parity, one aligned quad of
//    chunks each) need bit 2 of s to differ between them; both then hit
//    distinct banks (an LDS probe counted no conflicts for either, where
//    the former swizzle 4 ((n >> 1) & 1) + ((n >> 1) & 3) gave the writes
//    about 8 conflict cycles each).  swz does not change under n + 4, so a
//    sub-step's rows 8 kk further are an immediate offset.
constexpr int kBwdBM = 256, kBwdBN = 256, kBwdThreads = 512;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ int wd_swz(int n) { return (n & 3) | (((n >> 1) & 1) << 2); }

// raw buffer over [base, base + bytes) (bytes < 2^31): loads at offsets past
// the range return zeros
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

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
  // two register sets, fixed by step parity: even steps load gA and store gB,
  // odd steps the reverse (a set is never copied across the loop)
  u32x4_t gA[GC], gB[GC];
  // the step moves the scalar offset only; lane offsets are fixed
  uint32_t g_voff[GC];
#pragma unroll
  for (int i = 0; i < GC; ++i) g_voff[i] = g_off0 + i * g_row_step;
  auto load_g = [&](u32x4_t (&gr_regs)[GC], int64_t n0) {
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
  auto store_g = [&](const u32x4_t (&gr_regs)[GC], uint8_t* dst) {
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
  // Rows tr_row + 8 kk + 4 u share the swizzle of tr_row, so sub-step kk is
  // the immediate offset 1024 kk.
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
  load_g(gA, 0);
  load_g(gB, kBK);
  put_piece(w1, sm.w[0][wn]);
  store_g(gA, sm.g[0]);
  __syncthreads();
  // step s: MFMAs on the grad_out tile and Wd of buffer s & 1, with each
  // sub-step's fragments read one sub-step ahead.  All waves reach the LDS
  // at once after the barrier, so the first fragment reads go out before
  // the global loads, two steps ahead: grad_out of step s + 2 (into
  // registers `gl`) and the raw weights of step s + 2 (into `nxt`).
  // Behind sub-step 2, grad_out of step s + 1 (`gs`, loaded a step earlier)
  // goes into the other tile: a whole step for its loads measured 1-2%
  // faster than the two sub-steps of loading it one step ahead, and every
  // other load or store position tried was slower.  `cur` holds the raw
  // weights of step s + 1, fetched a step earlier and decoded into the
  // other Wd buffer behind sub-step 1.  Both buffers of step s + 1 were last
  // read in step s - 1, so the barrier that ends step s is the only one.
  // Loads past the last step read zeros.
  auto step = [&](WRaw& cur, WRaw& nxt, u32x4_t (&gl)[GC], const u32x4_t (&gs)[GC], int s) {
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
        load_g(gl, (int64_t)(s + 2) * kBK);
        load_w(nxt, (int64_t)(s + 2) * kBK);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kk == 1) put_piece(cur, sm.w[(s & 1) ^ 1][wn]);
      if (kk == 2) {
        __builtin_amdgcn_sched_barrier(0);
        store_g(gs, sm.g[(s & 1) ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  };
  for (int s = 0; s < nsteps; s += 2) {
    step(w0, w1, gA, gB, s);
    if (s + 1 < nsteps) step(w1, w0, gB, gA, s + 1);
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
#define MXQ_FL_LAUNCH(KERNEL, NWG)                                                                               \
  hipLaunchKernelGGL(KERNEL, dim3((unsigned)(NWG)), dim3(kFlThreads), 0, st, (const uint8_t*)a,                       \
                     (const uint8_t*)packed, scales, offs, (int)experts, tokens, wn_dim, wk_dim, (uint8_t*)out,       \
                     (int)gx)
      // whole weight lines (4 steps per fetch) whenever whole generations and
      // 16-byte scale chunks exist: 3-5% faster on the routed-expert
      // projections and ~15% on the 8-expert forward than the per-step form
      if (sch8) {
        // a grid of 128-row tiles that fits in one round takes them in height
        // order: every CU gets one tile of full height first and the short
        // segment tails double up
        if (n128 <= slots) {
          const int xr = cus > 0 && cus % 8 == 0 && n128 >= cus ? cus / 8 : 0;
          hipLaunchKernelGGL(k_grouped_mm_fwd_fl128_by_height, dim3((unsigned)n128), dim3(kFlThreads), 0, st,
                             (const uint8_t*)a, (const uint8_t*)packed, scales, offs, (int)experts, tokens, wn_dim,
                             wk_dim, (uint8_t*)out, (int)gx, xr);
        }
        else if (bm96) MXQ_FL_LAUNCH(k_grouped_mm_fwd_fl96, n96);   // (several rounds)
        else MXQ_FL_LAUNCH(k_grouped_mm_fwd_fl128, n128);
      } else if (bm96) {
        MXQ_FWD_LAUNCH(96, 2, n96);
      } else {
        MXQ_FWD_LAUNCH(128, 2, n128);
      }
#undef MXQ_FL_LAUNCH
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
  // 96-row tiles when they take no more rounds of two workgroups per CU (as the bf16 forward)
  const int cus = device_cus();
  const int64_t slots = 2 * (int64_t)(cus > 0 ? cus : 256);
  const int64_t n128 = gx * ((tokens + 127) / 128 + experts), n96 = gx * ((tokens + 95) / 96 + experts);
  const bool bm96 = (n96 + slots - 1) / slots <= (n128 + slots - 1) / slots;
  if (!grid_fits(bm96 ? n96 : n128, kW4Threads)) return hipErrorInvalidConfiguration;
  if (bm96)
    hipLaunchKernelGGL(k_grouped_mm_fwd_w4a4_96, dim3((unsigned)n96), dim3(kW4Threads), 0, st, (const uint8_t*)xq, xs,
                       (const uint8_t*)packed, scales, offs, (int)experts, tokens, n, k, (uint8_t*)out, (int)gx);
  else
    hipLaunchKernelGGL(k_grouped_mm_fwd_w4a4_128, dim3((unsigned)n128), dim3(kW4Threads), 0, st, (const uint8_t*)xq,
                       xs, (const uint8_t*)packed, scales, offs, (int)experts, tokens, n, k, (uint8_t*)out, (int)gx);
  return hipGetLastError();
}

hipError_t launch_grouped_mm_w4a8(const void* xq, const uint8_t* xs, int64_t tokens, const int8_t* packed,
                                  const uint8_t* scales, int64_t experts, int64_t n, int64_t k, const int32_t* offs,
                                  void* out, hipStream_t st) {
  const int64_t gx = (n + kW8BN - 1) / kW8BN;
  const int64_t gy = (tokens + kW8BM - 1) / kW8BM + experts;
  if (!grid_fits(gx * gy, kW8Threads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_grouped_mm_fwd_w4a8, dim3((unsigned)(gx * gy)), dim3(kW8Threads), 0, st, (const uint8_t*)xq, xs,
                     (const uint8_t*)packed, scales, offs, (int)experts, tokens, n, k, (uint8_t*)out, (int)gx);
  return hipGetLastError();
}

}  // namespace mxq
