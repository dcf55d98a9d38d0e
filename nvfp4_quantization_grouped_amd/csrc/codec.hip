// Streaming codec kernels: quantize_mxfp4, dequantize_mxfp4, quantize_cache
// and the straight-through copy.  All are HBM-bound streams.
//
// Fast path: a lane owns a "chunk" of 8 consecutive elements (one 16-byte
// load for 16-bit types, two for fp32); a scale block of B elements is B/8
// consecutive lanes, whose amax is combined with DPP.  Every lane of a wave
// runs the same trip count (tails are masked, never branched around) so the
// cross-lane reductions always see whole groups.  Each lane keeps several
// chunks in flight (8 for inputs larger than the Infinity Cache, read
// non-temporally; 4 otherwise).  The general path (misaligned pointers, block sizes that
// are not a power of two in [8, 512], partial final groups) is one thread per
// block with scalar accesses; it shares the element arithmetic.
#include "launch.hpp"
#include "mxq_device.hpp"

namespace mxq {

constexpr int kThreads = 256;
constexpr int kGridCap = 16384;   // workgroups of a grid-stride launch (64 per CU)

// Access mode of a streaming launch, chosen on the host (MI355X measurements
// on data not in any cache).  Inputs of 256 MB and more: 8 chunks in flight
// per lane, non-temporal loads and stores.  Quantizers on smaller inputs (a
// 67 MB KV cache): 16 chunks per lane, so the whole input is requested in one
// round by half as many waves (~6% faster there, ~4% slower on large inputs).
struct StreamBig {
  static constexpr int kUnroll = 8;
  template <typename T> __device__ static __forceinline__ T ld(const T* p) { return __builtin_nontemporal_load(p); }
  template <typename T> __device__ static __forceinline__ void st(T v, T* p) { __builtin_nontemporal_store(v, p); }
};
// Quantizer inputs below 16 MB: one chunk per lane (16 per lane would leave
// a handful of workgroups for the whole GPU).
struct StreamTiny {
  static constexpr int kUnroll = 1;
  template <typename T> __device__ static __forceinline__ T ld(const T* p) { return *p; }
  template <typename T> __device__ static __forceinline__ void st(T v, T* p) { __builtin_nontemporal_store(v, p); }
};
struct StreamSmall {
  static constexpr int kUnroll = 16;
  template <typename T> __device__ static __forceinline__ T ld(const T* p) { return __builtin_nontemporal_load(p); }
  template <typename T> __device__ static __forceinline__ void st(T v, T* p) { __builtin_nontemporal_store(v, p); }
};
// Dequantization (all sizes): 4 chunks per lane, non-temporal loads of the
// packed bytes and stores of the 4x larger output.
struct StreamDequant {
  static constexpr int kUnroll = 4;
  template <typename T> __device__ static __forceinline__ T ld(const T* p) { return __builtin_nontemporal_load(p); }
  template <typename T> __device__ static __forceinline__ void st(T v, T* p) { __builtin_nontemporal_store(v, p); }
};
constexpr int64_t kBigStreamBytes = 256ll << 20, kTinyStreamBytes = 16ll << 20;

template <int DT>
struct Chunk {
  static constexpr int kWords = DT == DT_F32 ? 8 : 4;
  uint32_t w[kWords];
};

template <int DT, class M>
__device__ __forceinline__ void load_chunk(const uint8_t* __restrict__ base, int64_t c, Chunk<DT>& ch) {
  if constexpr (DT == DT_F32) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(base + c * 32);
    u32x4_t a = M::ld(p), b = M::ld(p + 1);
    ch.w[0] = a.x; ch.w[1] = a.y; ch.w[2] = a.z; ch.w[3] = a.w;
    ch.w[4] = b.x; ch.w[5] = b.y; ch.w[6] = b.z; ch.w[7] = b.w;
  } else {
    u32x4_t a = M::ld(reinterpret_cast<const u32x4_t*>(base + c * 16));
    ch.w[0] = a.x; ch.w[1] = a.y; ch.w[2] = a.z; ch.w[3] = a.w;
  }
}

template <int DT, class M>
__device__ __forceinline__ void store_chunk(uint8_t* __restrict__ base, int64_t c, const Chunk<DT>& ch) {
  if constexpr (DT == DT_F32) {
    u32x4_t* p = reinterpret_cast<u32x4_t*>(base + c * 32);
    u32x4_t a = {ch.w[0], ch.w[1], ch.w[2], ch.w[3]}, b = {ch.w[4], ch.w[5], ch.w[6], ch.w[7]};
    M::st(a, p);
    M::st(b, p + 1);
  } else {
    u32x4_t a = {ch.w[0], ch.w[1], ch.w[2], ch.w[3]};
    M::st(a, reinterpret_cast<u32x4_t*>(base + c * 16));
  }
}

// fp32 bit pattern of max |x| over the chunk.
template <int DT>
__device__ __forceinline__ uint32_t chunk_amax_bits(const Chunk<DT>& ch) {
  if constexpr (DT == DT_F32) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, ch.w[i] & 0x7FFFFFFFu);
    return m;
  } else {
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mag_max_h2(acc, ch.w[i]);
    const uint32_t h = max(acc & 0xFFFFu, acc >> 16);
    if constexpr (DT == DT_BF16) return h << 16;
    else return as_u32((float)__builtin_bit_cast(_Float16, (unsigned short)h));
  }
}

// Eight elements -> eight e2m1 codes (one dword, element 0 in the low nibble).
// CANON: map -0.0 inputs to +0.0 first (needed where the code itself is kept).
template <int DT, bool CANON>
__device__ __forceinline__ uint32_t encode_fp4_chunk(const Chunk<DT>& ch, float s) {
  uint32_t c = 0;
  if constexpr (DT == DT_F32) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = CANON ? as_f32(ch.w[i]) + 0.0f : as_f32(ch.w[i]);
    c = enc_fp4_f2<0>(c, v[0], v[1], s);
    c = enc_fp4_f2<1>(c, v[2], v[3], s);
    c = enc_fp4_f2<2>(c, v[4], v[5], s);
    c = enc_fp4_f2<3>(c, v[6], v[7], s);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = CANON ? canon_negzero_h2(ch.w[i]) : ch.w[i];
    c = enc_fp4_h2<DT, 0>(c, w[0], s);
    c = enc_fp4_h2<DT, 1>(c, w[1], s);
    c = enc_fp4_h2<DT, 2>(c, w[2], s);
    c = enc_fp4_h2<DT, 3>(c, w[3], s);
  }
  return c;
}

// Eight e2m1 codes -> eight values of DT (code 8 must already be cleared).
template <int DT>
__device__ __forceinline__ void decode_fp4_chunk(uint32_t c, float s, Chunk<DT>& out) {
  if constexpr (DT == DT_F16) {
    out.w[0] = dec_fp4_f16x2<0>(c, s);
    out.w[1] = dec_fp4_f16x2<1>(c, s);
    out.w[2] = dec_fp4_f16x2<2>(c, s);
    out.w[3] = dec_fp4_f16x2<3>(c, s);
  } else {
    uint32_t b[4];
    b[0] = dec_fp4_bf16x2<0>(c, s);
    b[1] = dec_fp4_bf16x2<1>(c, s);
    b[2] = dec_fp4_bf16x2<2>(c, s);
    b[3] = dec_fp4_bf16x2<3>(c, s);
    if constexpr (DT == DT_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) out.w[i] = b[i];
    } else {  // every e2m1 value times 2^k is a bf16 value: widening is exact
#pragma unroll
      for (int i = 0; i < 4; ++i) { out.w[2 * i] = b[i] << 16; out.w[2 * i + 1] = b[i] & 0xFFFF0000u; }
    }
  }
}

// Eight elements -> E4M3 -> eight values of DT, scale s (nearest-even both ways).
template <int DT>
__device__ __forceinline__ void fake_quant_fp8_chunk(const Chunk<DT>& in, float s, Chunk<DT>& out) {
  if constexpr (DT == DT_BF16) {
    uint32_t c0 = enc_fp8_bf16x2<false>(0u, in.w[0], s);
    c0 = enc_fp8_bf16x2<true>(c0, in.w[1], s);
    uint32_t c1 = enc_fp8_bf16x2<false>(0u, in.w[2], s);
    c1 = enc_fp8_bf16x2<true>(c1, in.w[3], s);
    out.w[0] = dec_fp8_bf16x2<false>(c0, s);
    out.w[1] = dec_fp8_bf16x2<true>(c0, s);
    out.w[2] = dec_fp8_bf16x2<false>(c1, s);
    out.w[3] = dec_fp8_bf16x2<true>(c1, s);
  } else {
    float v[8];
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = as_f32(in.w[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = f16_lo(in.w[i]); v[2 * i + 1] = f16_hi(in.w[i]); }
    }
    float o[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t c = enc_fp8_f2<false>(0u, v[4 * h], v[4 * h + 1], s);
      c = enc_fp8_f2<true>(c, v[4 * h + 2], v[4 * h + 3], s);
      f32x2_t a = dec_fp8_f2<false>(c, s), b = dec_fp8_f2<true>(c, s);
      o[4 * h] = a.x; o[4 * h + 1] = a.y; o[4 * h + 2] = b.x; o[4 * h + 3] = b.y;
    }
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) out.w[i] = as_u32(o[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out.w[i] = pack_f16x2(o[2 * i], o[2 * i + 1]);
    }
  }
}

// ------------------------------------------------------------- quantize_mxfp4
template <int DT, class M>
__global__ void __launch_bounds__(kThreads) k_quantize_mxfp4(const uint8_t* __restrict__ x,
                                                           uint32_t* __restrict__ packed,
                                                           uint8_t* __restrict__ scales, int64_t nchunks) {
  const int64_t step = (int64_t)gridDim.x * kThreads * M::kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * M::kUnroll; base < nchunks; base += step) {
    Chunk<DT> ch[M::kUnroll];
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      if (c < nchunks) load_chunk<DT, M>(x, c, ch[u]);
      else {
#pragma unroll
        for (int i = 0; i < Chunk<DT>::kWords; ++i) ch[u].w[i] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      const uint32_t amax = group_max_u32<4>(chunk_amax_bits<DT>(ch[u]));   // 32 = 4 chunks
      const int e = floor_rule_exponent(amax);
      const uint32_t codes = encode_fp4_chunk<DT, true>(ch[u], pow2f(e));
      if (c < nchunks) {
        M::st(codes, packed + c);
        if ((c & 3) == 0) scales[c >> 2] = (uint8_t)(e + 127);
      }
    }
  }
}

// One thread per 32-element block; any alignment.
template <int DT>
__device__ __forceinline__ float load_elem(const uint8_t* p, int64_t i) {
  if constexpr (DT == DT_F32) return *reinterpret_cast<const float*>(p + 4 * i);
  else {
    const unsigned short h = *reinterpret_cast<const unsigned short*>(p + 2 * i);
    if constexpr (DT == DT_BF16) return as_f32((uint32_t)h << 16);
    else return (float)__builtin_bit_cast(_Float16, h);
  }
}
template <int DT>
__device__ __forceinline__ void store_elem(uint8_t* p, int64_t i, float v, uint32_t bf16_bits) {
  if constexpr (DT == DT_F32) *reinterpret_cast<float*>(p + 4 * i) = v;
  else if constexpr (DT == DT_BF16) *reinterpret_cast<unsigned short*>(p + 2 * i) = (unsigned short)bf16_bits;
  else *reinterpret_cast<unsigned short*>(p + 2 * i) = __builtin_bit_cast(unsigned short, (_Float16)v);
}

template <int DT>
__global__ void __launch_bounds__(kThreads) k_quantize_mxfp4_general(const uint8_t* __restrict__ x,
                                                                   uint8_t* __restrict__ packed,
                                                                   uint8_t* __restrict__ scales, int64_t nblocks) {
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * kThreads) {
    uint32_t amax = 0;
    for (int i = 0; i < 32; ++i) amax = max(amax, as_u32(load_elem<DT>(x, b * 32 + i)) & 0x7FFFFFFFu);
    const int e = floor_rule_exponent(amax);
    const float s = pow2f(e);
    for (int j = 0; j < 16; ++j) {
      const float a = load_elem<DT>(x, b * 32 + 2 * j) + 0.0f, c = load_elem<DT>(x, b * 32 + 2 * j + 1) + 0.0f;
      packed[b * 16 + j] = (uint8_t)(enc_fp4_f2<0>(0u, a, c, s) & 0xFFu);
    }
    scales[b] = (uint8_t)(e + 127);
  }
}

// ----------------------------------------------------------- dequantize_mxfp4
template <int DT, class M>
__global__ void __launch_bounds__(kThreads) k_dequantize_mxfp4(const uint32_t* __restrict__ packed,
                                                             const uint8_t* __restrict__ scales,
                                                             uint8_t* __restrict__ out, int64_t nchunks) {
  const int64_t step = (int64_t)gridDim.x * kThreads * M::kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * M::kUnroll; base < nchunks; base += step) {
    uint32_t codes[M::kUnroll], sb[M::kUnroll];
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      codes[u] = c < nchunks ? M::ld(packed + c) : 0u;
      sb[u] = c < nchunks ? (uint32_t)scales[c >> 2] : 127u;
    }
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      Chunk<DT> o;
      decode_fp4_chunk<DT>(clear_negzero_codes(codes[u]), e8m0_to_f32(sb[u]), o);
      if (c < nchunks) store_chunk<DT, M>(out, c, o);
    }
  }
}

template <int DT>
__global__ void __launch_bounds__(kThreads) k_dequantize_mxfp4_general(const uint8_t* __restrict__ packed,
                                                                     const uint8_t* __restrict__ scales,
                                                                     uint8_t* __restrict__ out, int64_t nblocks) {
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * kThreads) {
    const float s = e8m0_to_f32(scales[b]);
    for (int j = 0; j < 16; ++j) {
      const uint32_t code = clear_negzero_codes((uint32_t)packed[b * 16 + j]);
      if constexpr (DT == DT_F16) {
        const uint32_t h = dec_fp4_f16x2<0>(code, s);
        *reinterpret_cast<unsigned short*>(out + 2 * (b * 32 + 2 * j)) = (unsigned short)(h & 0xFFFFu);
        *reinterpret_cast<unsigned short*>(out + 2 * (b * 32 + 2 * j + 1)) = (unsigned short)(h >> 16);
      } else {
        const uint32_t h = dec_fp4_bf16x2<0>(code, s);
        store_elem<DT>(out, b * 32 + 2 * j, as_f32(h << 16), h & 0xFFFFu);
        store_elem<DT>(out, b * 32 + 2 * j + 1, as_f32(h & 0xFFFF0000u), h >> 16);
      }
    }
  }
}

// ------------------------------------------------------------- quantize_cache
template <int DT, int FMT, int L, class M>
__global__ void __launch_bounds__(kThreads) k_quantize_cache(const uint8_t* __restrict__ x,
                                                           uint8_t* __restrict__ out, int64_t nchunks) {
  const int64_t step = (int64_t)gridDim.x * kThreads * M::kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * M::kUnroll; base < nchunks; base += step) {
    Chunk<DT> ch[M::kUnroll];
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      if (c < nchunks) load_chunk<DT, M>(x, c, ch[u]);
      else {
#pragma unroll
        for (int i = 0; i < Chunk<DT>::kWords; ++i) ch[u].w[i] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      const uint32_t amax = group_max_u32<L>(chunk_amax_bits<DT>(ch[u]));
      const float s = pow2f(ceil_rule_exponent<FMT>(amax));
      Chunk<DT> o;
      if constexpr (FMT == FMT_FP8) fake_quant_fp8_chunk<DT>(ch[u], s, o);
      else decode_fp4_chunk<DT>(clear_negzero_codes(encode_fp4_chunk<DT, false>(ch[u], s)), s, o);
      if (c < nchunks) store_chunk<DT, M>(out, c, o);
    }
  }
}

// One thread per (row, group); handles partial final groups and any alignment.
template <int DT, int FMT>
__global__ void __launch_bounds__(kThreads) k_quantize_cache_general(const uint8_t* __restrict__ x,
                                                                   uint8_t* __restrict__ out, int64_t rows,
                                                                   int64_t channels, int64_t block) {
  const int64_t groups = (channels + block - 1) / block;
  const int64_t total = rows * groups;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < total; g += (int64_t)gridDim.x * kThreads) {
    const int64_t r = g / groups, j0 = (g % groups) * block;
    const int64_t n = min(block, channels - j0);
    const int64_t o0 = r * channels + j0;
    uint32_t amax = 0;
    for (int64_t i = 0; i < n; ++i) amax = max(amax, as_u32(load_elem<DT>(x, o0 + i)) & 0x7FFFFFFFu);
    const float s = pow2f(ceil_rule_exponent<FMT>(amax));
    for (int64_t i = 0; i < n; ++i) {
      const float v = load_elem<DT>(x, o0 + i);
      float y;
      if constexpr (FMT == FMT_FP8) {
        y = dec_fp8_f2<false>(enc_fp8_f2<false>(0u, v, 0.0f, s), s).x;
      } else {
        const uint32_t code = clear_negzero_codes(enc_fp4_f2<0>(0u, v, 0.0f, s) & 0xFu);
        y = as_f32(dec_fp4_bf16x2<0>(code, s) << 16);
      }
      // every value here is exact in fp32; the output cast rounds nearest-even
      uint32_t bfbits;
      if constexpr (DT == DT_BF16) {
        if constexpr (FMT == FMT_FP8) {
          bfbits = dec_fp8_bf16x2<false>(enc_fp8_f2<false>(0u, v, 0.0f, s), s) & 0xFFFFu;
        } else {
          bfbits = as_u32(y) >> 16;
        }
      } else {
        bfbits = 0;
      }
      store_elem<DT>(out, o0 + i, y, bfbits);
    }
  }
}

// ------------------------------------------------------------ STE copy
// 1024-thread workgroups, 4 x 16 bytes per lane, non-temporal both ways
// (measured best at every size: 256 threads x 8 chunks is ~6% slower).
constexpr int kCopyThreads = 1024, kCopyUnroll = 4;
__global__ void __launch_bounds__(kCopyThreads) k_copy16(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                       int64_t n16) {
  const int64_t step = (int64_t)gridDim.x * kCopyThreads * kCopyUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kCopyThreads * kCopyUnroll; base < n16; base += step) {
    u32x4_t v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + u * kCopyThreads + threadIdx.x;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + u * kCopyThreads + threadIdx.x;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}
__global__ void __launch_bounds__(kThreads) k_copy_bytes(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                       int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    dst[i] = src[i];
}

__global__ void __launch_bounds__(kThreads) k_zero_bytes(uint8_t* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    dst[i] = 0;
}

// ------------------------------------------------------------------ launchers
static inline int grid_for(int64_t items, int64_t per_block) {
  const int64_t cap = kGridCap;
  int64_t g = (items + per_block - 1) / per_block;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}
static inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

template <int DT>
static hipError_t launch_quantize_mxfp4_t(const void* x, int64_t rows, int64_t k, int8_t* packed, uint8_t* scales,
                                          hipStream_t st) {
  const int64_t n = rows * k;
  if (aligned(x, 16) && aligned(packed, 4)) {
    const int64_t nchunks = n / 8, bytes = n * (DT == DT_F32 ? 4 : 2);
    if (bytes >= kBigStreamBytes)
      hipLaunchKernelGGL((k_quantize_mxfp4<DT, StreamBig>), dim3(grid_for(nchunks, kThreads * StreamBig::kUnroll)),
                         dim3(kThreads), 0, st, (const uint8_t*)x, (uint32_t*)packed, scales, nchunks);
    else if (bytes >= kTinyStreamBytes)
      hipLaunchKernelGGL((k_quantize_mxfp4<DT, StreamSmall>), dim3(grid_for(nchunks, kThreads * StreamSmall::kUnroll)),
                         dim3(kThreads), 0, st, (const uint8_t*)x, (uint32_t*)packed, scales, nchunks);
    else
      hipLaunchKernelGGL((k_quantize_mxfp4<DT, StreamTiny>), dim3(grid_for(nchunks, kThreads * StreamTiny::kUnroll)),
                         dim3(kThreads), 0, st, (const uint8_t*)x, (uint32_t*)packed, scales, nchunks);
  } else {
    const int64_t nb = n / 32;
    hipLaunchKernelGGL(k_quantize_mxfp4_general<DT>, dim3(grid_for(nb, kThreads)), dim3(kThreads), 0, st,
                       (const uint8_t*)x, (uint8_t*)packed, scales, nb);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const void* x, int dt, int64_t rows, int64_t k, int8_t* packed, uint8_t* scales,
                                 hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_quantize_mxfp4_t<DT_F32>(x, rows, k, packed, scales, st);
    case DT_BF16: return launch_quantize_mxfp4_t<DT_BF16>(x, rows, k, packed, scales, st);
    default: return launch_quantize_mxfp4_t<DT_F16>(x, rows, k, packed, scales, st);
  }
}

template <int DT>
static hipError_t launch_dequantize_mxfp4_t(const int8_t* packed, const uint8_t* scales, int64_t rows, int64_t k,
                                            void* out, hipStream_t st) {
  const int64_t n = rows * k;
  if (aligned(packed, 4) && aligned(out, 16)) {
    // dequantization is write-dominated (1 packed byte -> 4..8 output bytes):
    // plain loads measured best at every size
    const int64_t nchunks = n / 8;
    hipLaunchKernelGGL((k_dequantize_mxfp4<DT, StreamDequant>), dim3(grid_for(nchunks, kThreads * StreamDequant::kUnroll)),
                       dim3(kThreads), 0, st, (const uint32_t*)packed, scales, (uint8_t*)out, nchunks);
  } else {
    const int64_t nb = n / 32;
    hipLaunchKernelGGL(k_dequantize_mxfp4_general<DT>, dim3(grid_for(nb, kThreads)), dim3(kThreads), 0, st,
                       (const uint8_t*)packed, scales, (uint8_t*)out, nb);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize_mxfp4(const int8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, void* out,
                                   int dt, hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_dequantize_mxfp4_t<DT_F32>(packed, scales, rows, k, out, st);
    case DT_BF16: return launch_dequantize_mxfp4_t<DT_BF16>(packed, scales, rows, k, out, st);
    default: return launch_dequantize_mxfp4_t<DT_F16>(packed, scales, rows, k, out, st);
  }
}

template <int DT, int FMT, int L>
static void launch_cache_fast(const void* x, void* out, int64_t nchunks, hipStream_t st) {
  const int64_t bytes = nchunks * 8 * (DT == DT_F32 ? 4 : 2);
  if (bytes >= kBigStreamBytes)
    hipLaunchKernelGGL((k_quantize_cache<DT, FMT, L, StreamBig>), dim3(grid_for(nchunks, kThreads * StreamBig::kUnroll)),
                       dim3(kThreads), 0, st, (const uint8_t*)x, (uint8_t*)out, nchunks);
  else if (bytes >= kTinyStreamBytes)
    hipLaunchKernelGGL((k_quantize_cache<DT, FMT, L, StreamSmall>),
                       dim3(grid_for(nchunks, kThreads * StreamSmall::kUnroll)), dim3(kThreads), 0, st,
                       (const uint8_t*)x, (uint8_t*)out, nchunks);
  else
    hipLaunchKernelGGL((k_quantize_cache<DT, FMT, L, StreamTiny>),
                       dim3(grid_for(nchunks, kThreads * StreamTiny::kUnroll)), dim3(kThreads), 0, st,
                       (const uint8_t*)x, (uint8_t*)out, nchunks);
}

template <int DT, int FMT>
static hipError_t launch_quantize_cache_t(const void* x, void* out, int64_t rows, int64_t channels, int32_t block,
                                          hipStream_t st) {
  const bool pow2 = block >= 8 && block <= 512 && (block & (block - 1)) == 0;
  if (pow2 && channels % block == 0 && aligned(x, 16) && aligned(out, 16)) {
    const int64_t nchunks = rows * channels / 8;
    switch (block) {
      case 8: launch_cache_fast<DT, FMT, 1>(x, out, nchunks, st); break;
      case 16: launch_cache_fast<DT, FMT, 2>(x, out, nchunks, st); break;
      case 32: launch_cache_fast<DT, FMT, 4>(x, out, nchunks, st); break;
      case 64: launch_cache_fast<DT, FMT, 8>(x, out, nchunks, st); break;
      case 128: launch_cache_fast<DT, FMT, 16>(x, out, nchunks, st); break;
      case 256: launch_cache_fast<DT, FMT, 32>(x, out, nchunks, st); break;
      default: launch_cache_fast<DT, FMT, 64>(x, out, nchunks, st); break;
    }
  } else {
    const int64_t groups = rows * ((channels + block - 1) / block);
    hipLaunchKernelGGL((k_quantize_cache_general<DT, FMT>), dim3(grid_for(groups, kThreads)), dim3(kThreads), 0, st,
                       (const uint8_t*)x, (uint8_t*)out, rows, channels, (int64_t)block);
  }
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_quantize_cache_dt(const void* x, void* out, int64_t rows, int64_t channels, int fmt,
                                           int32_t block, hipStream_t st) {
  switch (fmt) {
    case FMT_FP8: return launch_quantize_cache_t<DT, FMT_FP8>(x, out, rows, channels, block, st);
    case FMT_MXFP4: return launch_quantize_cache_t<DT, FMT_MXFP4>(x, out, rows, channels, block, st);
    default: return launch_quantize_cache_t<DT, FMT_NVFP4>(x, out, rows, channels, block, st);
  }
}

hipError_t launch_quantize_cache(const void* x, void* out, int dt, int64_t rows, int64_t channels, int fmt,
                                 int32_t block, hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_quantize_cache_dt<DT_F32>(x, out, rows, channels, fmt, block, st);
    case DT_BF16: return launch_quantize_cache_dt<DT_BF16>(x, out, rows, channels, fmt, block, st);
    default: return launch_quantize_cache_dt<DT_F16>(x, out, rows, channels, fmt, block, st);
  }
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  if (aligned(src, 16) && aligned(dst, 16) && bytes % 16 == 0) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_copy16, dim3(grid_for(n16, kCopyThreads * kCopyUnroll)), dim3(kCopyThreads), 0, st,
                       (const u32x4_t*)src, (u32x4_t*)dst, n16);
  } else {
    hipLaunchKernelGGL(k_copy_bytes, dim3(grid_for(bytes, kThreads * 4)), dim3(kThreads), 0, st,
                       (const uint8_t*)src, (uint8_t*)dst, bytes);
  }
  return hipGetLastError();
}

hipError_t launch_zero(void* dst, int64_t bytes, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_bytes, dim3(grid_for(bytes, kThreads * 4)), dim3(kThreads), 0, st, (uint8_t*)dst, bytes);
  return hipGetLastError();
}

}  // namespace mxq
