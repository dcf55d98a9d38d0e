// Streaming codec kernels: quantize_mxfp4, dequantize_mxfp4, quantize_cache,
// its packed storage form,
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
#include <algorithm>

#include "launch.hpp"
#include "mxq_device.hpp"

namespace mxq {

constexpr int kThreads = 256;
constexpr int kGridCap = 16384;   // workgroups of a grid-stride launch (64 per CU)
// The dequantizers write 4x what they read; with up to 256 workgroups per CU
// in flight over the grid-stride passes the [64, 4096, 4096] weight dequant
// ran 5% faster (bf16 [65536, 7168]: 1%) than with the 64-per-CU cap,
// bit-identical.
constexpr int kDequantGridCap = 65536;

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

// Eight elements -> eight E4M3 codes of x / s, nearest-even, sign kept (c0 holds
// elements 0..3, c1 elements 4..7, element i in byte i of the pair).
template <int DT>
__device__ __forceinline__ void encode_fp8_chunk(const Chunk<DT>& in, float s, uint32_t& c0, uint32_t& c1) {
  if constexpr (DT == DT_BF16) {
    c0 = enc_fp8_bf16x2<true>(enc_fp8_bf16x2<false>(0u, in.w[0], s), in.w[1], s);
    c1 = enc_fp8_bf16x2<true>(enc_fp8_bf16x2<false>(0u, in.w[2], s), in.w[3], s);
  } else {
    float v[8];
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = as_f32(in.w[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = f16_lo(in.w[i]); v[2 * i + 1] = f16_hi(in.w[i]); }
    }
    c0 = enc_fp8_f2<true>(enc_fp8_f2<false>(0u, v[0], v[1], s), v[2], v[3], s);
    c1 = enc_fp8_f2<true>(enc_fp8_f2<false>(0u, v[4], v[5], s), v[6], v[7], s);
  }
}

// Eight E4M3 codes -> eight values of DT: code value times s, rounded
// nearest-even to DT (exact in fp32, then one rounding for f16).
template <int DT>
__device__ __forceinline__ void decode_fp8_chunk(uint32_t c0, uint32_t c1, float s, Chunk<DT>& out) {
  if constexpr (DT == DT_BF16) {
    out.w[0] = dec_fp8_bf16x2<false>(c0, s);
    out.w[1] = dec_fp8_bf16x2<true>(c0, s);
    out.w[2] = dec_fp8_bf16x2<false>(c1, s);
    out.w[3] = dec_fp8_bf16x2<true>(c1, s);
  } else {
    float o[8];
    const uint32_t c[2] = {c0, c1};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x2_t a = dec_fp8_f2<false>(c[h], s), b = dec_fp8_f2<true>(c[h], s);
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

// Eight elements -> E4M3 -> eight values of DT, scale s (nearest-even both ways).
template <int DT>
__device__ __forceinline__ void fake_quant_fp8_chunk(const Chunk<DT>& in, float s, Chunk<DT>& out) {
  uint32_t c0, c1;
  encode_fp8_chunk<DT>(in, s, c0, c1);
  decode_fp8_chunk<DT>(c0, c1, s, out);
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

// ---------------------------------------------------------- two-level NVFP4
// "NVIDIA Model Optimizer: from mtq.quantize to a 4.95-bit DeepSeek-R1",
// section "NVFP4 in the code: two scales and a nibble":
//   g   = max|x| / (6 * 448)                       FP32 per-tensor scale
//   s_b = E4M3(max_{i in b} |x_i| / (6 g))         blocks of 16; a zero scale
//                                                   becomes 1.0, then clamped to [2^-9, 448]
//   x^  = E2M1(x / (s_b g)) * s_b g
// in fp32, each operation rounded nearest-even in the order written.  The
// divisions are IEEE divisions, not products with a reciprocal: where a
// quotient falls against the e2m1 midpoints decides the code, so it has to
// be the correctly rounded one.  Launches: the tensor amax (an atomic max of
// fp32 bit patterns, which order like the values for x >= 0) into the
// caller's 4-byte global-scale slot, the block pass reading it, and a
// one-thread pass that replaces it by g.  A tensor whose amax is 0 has every
// scale 1.0 and every code 0.
constexpr float kNvfp4Den = 6.0f * 448.0f;   // 2688, exact

__global__ void k_nvfp4_amax_init(uint32_t* __restrict__ slot) { *slot = 0u; }
__global__ void k_nvfp4_finalize(uint32_t* __restrict__ slot) { *slot = as_u32(as_f32(*slot) / kNvfp4Den); }

// Wave max, then workgroup max through LDS, then one atomic per workgroup.
__device__ __forceinline__ void nvfp4_amax_publish(uint32_t m, uint32_t* __restrict__ slot) {
  m = group_max_u32<64>(m);
  __shared__ uint32_t wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = wmax[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) b = max(b, wmax[i]);
    if (b) atomicMax(slot, b);
  }
}

template <int DT, class M>
__global__ void __launch_bounds__(kThreads) k_nvfp4_amax(const uint8_t* __restrict__ x, int64_t nchunks,
                                                       uint32_t* __restrict__ slot) {
  // Branch-free loads: a lane past the end reads the last chunk again and
  // leaves it out of the max.  With the loads behind `c < nchunks` the
  // compiler moved each chunk's max into its branch, after a vmcnt(0), so a
  // lane had one load in flight instead of kUnroll.
  uint32_t m = 0;
  const int64_t step = (int64_t)gridDim.x * kThreads * M::kUnroll, last = nchunks - 1;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * M::kUnroll; base < nchunks; base += step) {
    Chunk<DT> ch[M::kUnroll];
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) load_chunk<DT, M>(x, min(base + u * kThreads + threadIdx.x, last), ch[u]);
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const uint32_t a = chunk_amax_bits<DT>(ch[u]);
      m = max(m, base + u * kThreads + threadIdx.x <= last ? a : 0u);
    }
  }
  nvfp4_amax_publish(m, slot);
}

// Block scale of a block with max |x| = ab under the global scale g > 0: its
// E4M3 bits, and the element divisor d = fl(s_b g).
__device__ __forceinline__ uint32_t nvfp4_block_scale(float ab, float g, float& d) {
  float r = ab / (6.0f * g);
  if (r == 0.0f) r = 1.0f;
  r = fminf(fmaxf(r, 0x1p-9f), 448.0f);
  const uint32_t bits = enc_fp8_f2<false>(0u, r, r, 1.0f) & 0xFFu;   // nearest-even E4M3
  d = dec_fp8_f2<false>(bits, 1.0f).x * g;
  return bits;
}

// The same block scale from the reciprocal of 6g.  Per kernel: rlo, rhi =
// rcp(fl(6g)) (1 -+ 2^-20) and fast = 6g in [2^-125, 2^125] (a normal,
// accurate reciprocal).  ab rlo and ab rhi are within ~2 ulp of the nudged
// quotients, so they bracket fl(ab / fl(6g)); where both cast to the same
// E4M3 byte and lie inside (2^-8, 400) -- clear of the zero rule and the
// clamp -- that byte is the cast of the correctly rounded ratio.  Otherwise
// the division decides.
struct Nvfp4Ratio {
  float rlo, rhi;
  bool fast;
};
__device__ __forceinline__ Nvfp4Ratio nvfp4_ratio_setup(float g) {
  const float sixg = 6.0f * g;
  const float r = __builtin_amdgcn_rcpf(sixg);
  return {r * (1.0f - 0x1p-20f), r * (1.0f + 0x1p-20f), sixg >= 0x1p-125f && sixg <= 0x1p125f};
}
__device__ __forceinline__ uint32_t nvfp4_block_scale_fast(float ab, float g, const Nvfp4Ratio& q, float& d) {
  if (q.fast) {
    const float lo = ab * q.rlo, hi = ab * q.rhi;
    if (lo >= 0x1p-8f && hi <= 400.0f) {
      const uint32_t pr = enc_fp8_f2<false>(0u, lo, hi, 1.0f);     // bytes 0, 1: casts of lo, hi
      if (((pr ^ (pr >> 8)) & 0xFFu) == 0u) {
        const uint32_t bits = pr & 0xFFu;
        d = dec_fp8_f2<false>(bits, 1.0f).x * g;
        return bits;
      }
    }
  }
  return nvfp4_block_scale(ab, g, d);
}

// Eight elements -> eight e2m1 codes of the correctly rounded x / d (a
// code's sign bit is x < 0: -0.0 gives code 0).  Fast form: with r the
// hardware reciprocal of d (within 1 ulp), x r is within ~2.5 ulp of x / d, so the codes of
// x r nudged down and up by 2^-20 (8 ulp) bracket the code of fl(x / d);
// where the two agree no e2m1 midpoint lies between them and that is the
// code.  The nudges are folded into the reciprocal (x r(1 -+ 2^-20), ~2 ulp
// from the nudged quotients), and each product is a fused multiply-add with
// +0.0, which maps a -0.0 input to +0.0 (code 0) at no extra cost and keeps
// every other product as is.  A code of magnitude 0 keeps the sign of
// fl(x / d), which is -0.0 (code 0) for a negative x with |x / d| <= 2^-150,
// a boundary the reciprocal product cannot see; with d < 256 only nonzero
// fp32 subnormal inputs are that small (bf16 and f16 values are not).  So
// an element within reach of a midpoint (exact ties among them) takes an
// IEEE division, and chunks with d >= 256 or a reciprocal past 2^126, or
// with a nonzero fp32 subnormal input, take IEEE divisions for all eight.
template <int DT>
__device__ __forceinline__ uint32_t nvfp4_encode_chunk(const Chunk<DT>& ch, float d) {
  float v[8];
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = as_f32(ch.w[i]);
  } else if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(ch.w[i]); v[2 * i + 1] = bf16_hi(ch.w[i]); }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = f16_lo(ch.w[i]); v[2 * i + 1] = f16_hi(ch.w[i]); }
  }
  const float r = __builtin_amdgcn_rcpf(d);
  const float rd = r * (1.0f - 0x1p-20f), ru = r * (1.0f + 0x1p-20f);
  float ql[8], qh[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { ql[i] = __builtin_fmaf(v[i], rd, 0.0f); qh[i] = __builtin_fmaf(v[i], ru, 0.0f); }
  uint32_t lo = 0, hi = 0;
  lo = enc_fp4_f2<0>(lo, ql[0], ql[1], 1.0f);
  hi = enc_fp4_f2<0>(hi, qh[0], qh[1], 1.0f);
  lo = enc_fp4_f2<1>(lo, ql[2], ql[3], 1.0f);
  hi = enc_fp4_f2<1>(hi, qh[2], qh[3], 1.0f);
  lo = enc_fp4_f2<2>(lo, ql[4], ql[5], 1.0f);
  hi = enc_fp4_f2<2>(hi, qh[4], qh[5], 1.0f);
  lo = enc_fp4_f2<3>(lo, ql[6], ql[7], 1.0f);
  hi = enc_fp4_f2<3>(hi, qh[6], qh[7], 1.0f);
  bool exact = !(r <= 0x1p126f) || !(d < 256.0f);
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) exact |= ((as_u32(v[i]) & 0x7FFFFFFFu) - 1u) < 0x007FFFFFu;   // nonzero subnormal
  }
  if (exact) {
    // (+ 0.0f: a quotient that underflows to -0.0 gets code 0)
    uint32_t c = 0;
    c = enc_fp4_f2<0>(c, v[0] / d + 0.0f, v[1] / d + 0.0f, 1.0f);
    c = enc_fp4_f2<1>(c, v[2] / d + 0.0f, v[3] / d + 0.0f, 1.0f);
    c = enc_fp4_f2<2>(c, v[4] / d + 0.0f, v[5] / d + 0.0f, 1.0f);
    c = enc_fp4_f2<3>(c, v[6] / d + 0.0f, v[7] / d + 0.0f, 1.0f);
    return c;
  }
  // The bracket decides each element on its own: where its two codes
  // agree, that is the code.  Only the elements whose codes differ take
  // the division, one element position per branch, so a wave pays for a
  // division at a position only when one of its lanes straddles a midpoint
  // there.  (Exact ties are common: with x in bf16 and d = s_b g, a tensor
  // maximum whose odd part shares a factor with 2688 = 2^7 * 3 * 7 puts
  // quotients on midpoints in up to 3% of the chunks, in most waves.)
  const uint32_t diff = lo ^ hi;
  if (diff != 0u) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((diff >> (4 * i)) & 0xFu) {
        const uint32_t nib = enc_fp4_f2<0>(0u, v[i] / d + 0.0f, 0.0f, 1.0f) & 0xFu;
        lo = (lo & ~(0xFu << (4 * i))) | (nib << (4 * i));
      }
  }
  return lo;
}

template <int DT, class M>
__global__ void __launch_bounds__(kThreads) k_quantize_nvfp4(const uint8_t* __restrict__ x, uint32_t* __restrict__ packed,
                                                           uint8_t* __restrict__ scales, int64_t nchunks,
                                                           const uint32_t* __restrict__ slot) {
  const float g = as_f32(*slot) / kNvfp4Den;
  const Nvfp4Ratio rq = nvfp4_ratio_setup(g);
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
      const uint32_t ab = group_max_u32<2>(chunk_amax_bits<DT>(ch[u]));   // 16 = 2 chunks
      uint32_t codes = 0u, sbits = 0x38u;                                  // g = 0: scale 1.0, codes 0
      if (g != 0.0f) {
        float d;
        sbits = nvfp4_block_scale_fast(as_f32(ab), g, rq, d);
        codes = nvfp4_encode_chunk<DT>(ch[u], d);
      }
      if (c < nchunks) {
        M::st(codes, packed + c);
        if ((c & 1) == 0) scales[c >> 1] = (uint8_t)sbits;
      }
    }
  }
}

// fp32 product a * b, kept as an fp32 value: without the empty asm the
// compiler folds a product that is then narrowed to f16 into one
// mixed-precision multiply-add (with a +0.0 addend, which turns -0.0 into
// +0.0, and one rounding where the method rounds to fp32 first).
__device__ __forceinline__ float mul_f32(float a, float b) {
  float r = a * b;
  asm volatile("" : "+v"(r));
  return r;
}

// fp32 pair -> bf16 pair, nearest-even.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Eight codes (code 8 already cleared) times d -> eight values of DT.
template <int DT>
__device__ __forceinline__ void nvfp4_decode_chunk(uint32_t c, float d, Chunk<DT>& out) {
  float v[8];
  const uint32_t b[4] = {dec_fp4_bf16x2<0>(c, 1.0f), dec_fp4_bf16x2<1>(c, 1.0f), dec_fp4_bf16x2<2>(c, 1.0f),
                         dec_fp4_bf16x2<3>(c, 1.0f)};   // e2m1 values, exact in bf16
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = mul_f32(bf16_lo(b[i]), d); v[2 * i + 1] = mul_f32(bf16_hi(b[i]), d); }
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out.w[i] = as_u32(v[i]);
  } else if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out.w[i] = pack_bf16x2_rne(v[2 * i], v[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out.w[i] = pack_f16x2(v[2 * i], v[2 * i + 1]);
  }
}

template <int DT, class M>
__global__ void __launch_bounds__(kThreads) k_dequantize_nvfp4(const uint32_t* __restrict__ packed,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ gscale,
                                                             uint8_t* __restrict__ out, int64_t nchunks) {
  const float g = *gscale;
  const int64_t step = (int64_t)gridDim.x * kThreads * M::kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * M::kUnroll; base < nchunks; base += step) {
    uint32_t codes[M::kUnroll], sb[M::kUnroll];
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      codes[u] = c < nchunks ? M::ld(packed + c) : 0u;
      sb[u] = c < nchunks ? (uint32_t)scales[c >> 1] : 0x38u;
    }
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      Chunk<DT> o;
      nvfp4_decode_chunk<DT>(clear_negzero_codes(codes[u]), dec_fp8_f2<false>(sb[u], 1.0f).x * g, o);
      if (c < nchunks) store_chunk<DT, M>(out, c, o);
    }
  }
}

// General paths (any alignment): one element / one 16-element block per thread.
template <int DT>
__global__ void __launch_bounds__(kThreads) k_nvfp4_amax_general(const uint8_t* __restrict__ x, int64_t n,
                                                               uint32_t* __restrict__ slot) {
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    m = max(m, as_u32(load_elem<DT>(x, i)) & 0x7FFFFFFFu);
  nvfp4_amax_publish(m, slot);
}

template <int DT>
__global__ void __launch_bounds__(kThreads) k_quantize_nvfp4_general(const uint8_t* __restrict__ x,
                                                                   uint8_t* __restrict__ packed,
                                                                   uint8_t* __restrict__ scales, int64_t nblocks,
                                                                   const uint32_t* __restrict__ slot) {
  const float g = as_f32(*slot) / kNvfp4Den;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * kThreads) {
    uint32_t ab = 0;
    for (int i = 0; i < 16; ++i) ab = max(ab, as_u32(load_elem<DT>(x, b * 16 + i)) & 0x7FFFFFFFu);
    if (g == 0.0f) {
      for (int j = 0; j < 8; ++j) packed[b * 8 + j] = 0;
      scales[b] = 0x38;
      continue;
    }
    float d;
    scales[b] = (uint8_t)nvfp4_block_scale(as_f32(ab), g, d);
    for (int j = 0; j < 8; ++j) {
      const float q0 = load_elem<DT>(x, b * 16 + 2 * j) / d + 0.0f, q1 = load_elem<DT>(x, b * 16 + 2 * j + 1) / d + 0.0f;
      packed[b * 8 + j] = (uint8_t)(enc_fp4_f2<0>(0u, q0, q1, 1.0f) & 0xFFu);
    }
  }
}

template <int DT>
__global__ void __launch_bounds__(kThreads) k_dequantize_nvfp4_general(const uint8_t* __restrict__ packed,
                                                                     const uint8_t* __restrict__ scales,
                                                                     const float* __restrict__ gscale,
                                                                     uint8_t* __restrict__ out, int64_t nblocks) {
  const float g = *gscale;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * kThreads) {
    const float d = dec_fp8_f2<false>((uint32_t)scales[b], 1.0f).x * g;
    for (int j = 0; j < 8; ++j) {
      const uint32_t h = dec_fp4_bf16x2<0>(clear_negzero_codes((uint32_t)packed[b * 8 + j]), 1.0f);
      const float v0 = mul_f32(bf16_lo(h), d), v1 = mul_f32(bf16_hi(h), d);
      const uint32_t bb = pack_bf16x2_rne(v0, v1);
      store_elem<DT>(out, b * 16 + 2 * j, v0, bb & 0xFFFFu);
      store_elem<DT>(out, b * 16 + 2 * j + 1, v1, bb >> 16);
    }
  }
}

// ------------------------------------------------------- NVFP4 MSE scale sweep
// The MSE block-scale rule: each block of 16 tries the 126 positive finite
// E4M3 values (codes 0x01 .. 0x7E, in order) as its scale and keeps the first
// with the least fp32 squared error sum(fl(e^2)), e = x - e2m1(fl(x / d)) d in
// one fused multiply-add, d = fl(s g), squares and sums rounded one by one,
// elements in order.  One lane per block.  The error needs only the code
// magnitudes, which the reciprocal bracket of nvfp4_encode_chunk gives (x
// times rcp(d)(1 -+ 2^-20): where the two codes agree, no midpoint lies
// between them); elements whose bracket straddles a midpoint take a
// division each.  The stored codes are then encoded as the max rule's are.
//
// Candidates that cannot win are skipped without changing the result: the
// terms are non-negative and rounding to nearest is monotone, so a
// candidate's error is at least any one of its terms, computed the same way.
// The lane first evaluates the max rule's scale in full, then computes the
// term of the block's largest element under every candidate (wave-uniform
// d), and evaluates in full only the candidates whose term is below the
// best error so far (or equal to it at a lower code: the first candidate
// with the least error wins, so the selection keeps the least (error, code)
// pair).  On normally distributed weights about a fifth of the 126 survive.

// Squared error of 8 elements (v) whose codes are the dword c, under d; adds
// into err in element order.  The residual is one fused multiply-add; the
// square is kept opaque so that it is not fused into the sum.
__device__ __forceinline__ float sweep_err8(const float* v, uint32_t c, float d, float err) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    f32x2_t e2;
    switch (p) {
      case 0: e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0); break;
      case 1: e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1); break;
      case 2: e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2); break;
      default: e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3); break;
    }
    const float e0 = __builtin_fmaf(-e2.x, d, v[2 * p]), e1 = __builtin_fmaf(-e2.y, d, v[2 * p + 1]);
    err = err + mul_f32(e0, e0);
    err = err + mul_f32(e1, e1);
  }
  return err;
}

// Codes of 8 values under reciprocal bracket factors rd = r(1 - 2^-20), ru =
// r(1 + 2^-20); exact (IEEE division by d) where the bracket does not decide.
__device__ __forceinline__ uint32_t sweep_codes8(const float* v, float rd, float ru, float d, bool force_exact) {
  uint32_t lo = 0, hi = 0;
  lo = enc_fp4_f2<0>(lo, v[0] * rd, v[1] * rd, 1.0f);
  hi = enc_fp4_f2<0>(hi, v[0] * ru, v[1] * ru, 1.0f);
  lo = enc_fp4_f2<1>(lo, v[2] * rd, v[3] * rd, 1.0f);
  hi = enc_fp4_f2<1>(hi, v[2] * ru, v[3] * ru, 1.0f);
  lo = enc_fp4_f2<2>(lo, v[4] * rd, v[5] * rd, 1.0f);
  hi = enc_fp4_f2<2>(hi, v[4] * ru, v[5] * ru, 1.0f);
  lo = enc_fp4_f2<3>(lo, v[6] * rd, v[7] * rd, 1.0f);
  hi = enc_fp4_f2<3>(hi, v[6] * ru, v[7] * ru, 1.0f);
  if (force_exact) {
    uint32_t c = 0;
    c = enc_fp4_f2<0>(c, v[0] / d, v[1] / d, 1.0f);
    c = enc_fp4_f2<1>(c, v[2] / d, v[3] / d, 1.0f);
    c = enc_fp4_f2<2>(c, v[4] / d, v[5] / d, 1.0f);
    c = enc_fp4_f2<3>(c, v[6] / d, v[7] / d, 1.0f);
    return c;
  }
  // per element, as in nvfp4_encode_chunk: only positions whose two codes
  // differ take the division
  const uint32_t diff = lo ^ hi;
  if (diff != 0u) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((diff >> (4 * i)) & 0xFu) {
        const uint32_t nib = enc_fp4_f2<0>(0u, v[i] / d, 0.0f, 1.0f) & 0xFu;
        lo = (lo & ~(0xFu << (4 * i))) | (nib << (4 * i));
      }
  }
  return lo;
}

// The term of one element under d: its code as sweep_codes8 chooses it
// (returned in *code), then the squared residual as sweep_err8 forms it
// (returned in *res before squaring).
__device__ __forceinline__ float sweep_term1(float x, float d, uint32_t* code, float* res) {
  const float r = __builtin_amdgcn_rcpf(d);
  const bool force_exact = !(r <= 0x1p126f);
  const uint32_t lo = enc_fp4_f2<0>(0u, x * (r * (1.0f - 0x1p-20f)), 0.0f, 1.0f) & 0xFu;
  const uint32_t hi = enc_fp4_f2<0>(0u, x * (r * (1.0f + 0x1p-20f)), 0.0f, 1.0f) & 0xFu;
  const uint32_t c = (force_exact || lo != hi) ? enc_fp4_f2<0>(0u, x / d, 0.0f, 1.0f) & 0xFu : lo;
  const float e = __builtin_fmaf(-__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0)[0], d, x);
  *code = c;
  *res = e;
  return mul_f32(e, e);
}

// Squared error of the block v under candidate code (d = its E4M3 value
// times g, nonzero).
__device__ __forceinline__ float sweep_err16(const float* v, uint32_t code, float g) {
  const float d = dec_fp8_f2<false>(code, 1.0f).x * g;
  const float r = __builtin_amdgcn_rcpf(d);
  const bool force_exact = !(r <= 0x1p126f);
  const float rd = r * (1.0f - 0x1p-20f), ru = r * (1.0f + 0x1p-20f);
  const uint32_t c0 = sweep_codes8(v, rd, ru, d, force_exact);
  const uint32_t c1 = sweep_codes8(v + 8, rd, ru, d, force_exact);
  return sweep_err8(v + 8, c1, d, sweep_err8(v, c0, d, 0.0f));
}

template <int DT>
__global__ void __launch_bounds__(kThreads) k_quantize_nvfp4_mse(const uint8_t* __restrict__ x,
                                                               uint8_t* __restrict__ packed,
                                                               uint8_t* __restrict__ scales, int64_t nblocks,
                                                               const uint32_t* __restrict__ slot) {
  const float g = as_f32(*slot) / kNvfp4Den;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * kThreads) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = load_elem<DT>(x, b * 16 + i) + 0.0f;
    uint32_t best = 0x38, w0 = 0, w1 = 0;
    if (g != 0.0f) {
      // the block's largest magnitude (its first element of that magnitude)
      float xm = v[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) xm = __builtin_fabsf(v[i]) > __builtin_fabsf(xm) ? v[i] : xm;
      // the max rule's scale first (any candidate would do; this one is near the optimum)
      uint32_t c_init = enc_fp8_f2<false>(0u, __builtin_fabsf(xm) / (6.0f * g), 0.0f, 1.0f) & 0x7Fu;
      c_init = c_init < 1u ? 1u : (c_init > 0x7Eu ? 0x7Eu : c_init);
      best = 0;                                      // 0: no candidate yet
      float best_err = 0.0f;
      if (dec_fp8_f2<false>(c_init, 1.0f).x * g != 0.0f) {
        best = c_init;
        best_err = sweep_err16(v, c_init, g);
      }
      // the codes whose largest-element term does not rule them out, scanned
      // outwards from c_init.  d grows with the code.  Downwards the scan
      // stops at an underflowed divisor (every lower one underflows too) or
      // once the largest element saturates at 6 with 6d <= |xm| and a term
      // above the best error: every lower code saturates it too, with a
      // residual |xm| - 6d at least as large.  Upwards it stops after the
      // first code whose largest element quantizes to 0: every element does,
      // so every higher code has the same error (sum of x^2) at a higher code.
      uint32_t keep[4] = {0u, 0u, 0u, 0u};
      auto consider = [&](uint32_t code, float t) __attribute__((always_inline)) {
        if (best == 0 || t < best_err || (t == best_err && code < best)) keep[code >> 5] |= 1u << (code & 31);
      };
      for (uint32_t code = c_init - 1; code >= 1; --code) {
        const float d = dec_fp8_f2<false>(code, 1.0f).x * g;
        if (d == 0.0f) break;
        uint32_t cm;
        float e;
        const float t = sweep_term1(xm, d, &cm, &e);
        if (best != 0 && (cm & 7u) == 7u && (e > 0.0f) == (xm > 0.0f) && t > best_err) break;
        consider(code, t);
      }
      for (uint32_t code = c_init + 1; code < 0x7F; ++code) {
        const float d = dec_fp8_f2<false>(code, 1.0f).x * g;
        if (d == 0.0f) continue;                     // an underflowed divisor is not a candidate
        uint32_t cm;
        float e;
        const float t = sweep_term1(xm, d, &cm, &e);
        consider(code, t);
        if ((cm & 7u) == 0u) break;
      }
      // full evaluation of the survivors, lowest code first, per lane
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        while (keep[q] != 0u) {
          const uint32_t code = 32u * q + (uint32_t)__builtin_ctz(keep[q]);
          keep[q] &= keep[q] - 1u;
          const float err = sweep_err16(v, code, g);
          if (best == 0 || err < best_err || (err == best_err && code < best)) { best = code; best_err = err; }
        }
      }
      const float d = dec_fp8_f2<false>(best, 1.0f).x * g;
      Chunk<DT_F32> h0, h1;
#pragma unroll
      for (int i = 0; i < 8; ++i) { h0.w[i] = as_u32(v[i]); h1.w[i] = as_u32(v[8 + i]); }
      w0 = nvfp4_encode_chunk<DT_F32>(h0, d);
      w1 = nvfp4_encode_chunk<DT_F32>(h1, d);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      packed[b * 8 + j] = (uint8_t)(w0 >> (8 * j));
      packed[b * 8 + 4 + j] = (uint8_t)(w1 >> (8 * j));
    }
    scales[b] = (uint8_t)best;
  }
}

// ------------------------------------------------- packed KV-cache storage
// The codes and group scales quantize_cache rounds through, stored: e2m1
// nibbles (even channel low, sign bit for x < 0) or E4M3 bytes, and one scale
// byte per group.  The element arithmetic is quantize_cache's, so decoding
// the stored form gives the fake-quantized values bit for bit.

// Scale byte of 2^k: E8M0 (k + 127) for mxfp4 and fp8; E4M3 bits for nvfp4,
// whose k is in [-9, 8] (normal for k >= -6, else the subnormal 2^(k+9) * 2^-9).
template <int FMT>
__device__ __forceinline__ uint32_t cache_scale_byte(int k) {
  if constexpr (FMT == FMT_NVFP4) return k >= -6 ? (uint32_t)(k + 7) << 3 : 1u << (k + 9);
  else return (uint32_t)(k + 127);
}
// Scale byte -> fp32 scale.  The scaled conversions use only the exponent of
// their scale operand, which is exact for E8M0 but not for an E4M3 byte with
// mantissa bits, so nvfp4 decodes at scale 1 and multiplies in fp32 (e2m1
// times E4M3 is exact in fp32, bf16 and f16).
template <int FMT>
__device__ __forceinline__ float cache_scale_value(uint32_t b) {
  if constexpr (FMT == FMT_NVFP4) return dec_fp8_f2<false>(b, 1.0f).x;   // E4M3 decode; 0x7F/0xFF -> NaN
  else return e8m0_to_f32(b);
}

// Fast path: lane = chunk of 8 elements, group = L consecutive lanes (block 8L).
template <int DT, int FMT, int L, class M>
__global__ void __launch_bounds__(kThreads) k_quantize_cache_packed(const uint8_t* __restrict__ x,
                                                                  uint8_t* __restrict__ codes,
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
      const uint32_t amax = group_max_u32<L>(chunk_amax_bits<DT>(ch[u]));
      const int k = ceil_rule_exponent<FMT>(amax);
      const float s = pow2f(k);
      if constexpr (FMT == FMT_FP8) {
        uint32_t c0, c1;
        encode_fp8_chunk<DT>(ch[u], s, c0, c1);
        if (c < nchunks) M::st(u32x2_t{c0, c1}, reinterpret_cast<u32x2_t*>(codes) + c);
      } else {
        const uint32_t w = encode_fp4_chunk<DT, true>(ch[u], s);
        if (c < nchunks) M::st(w, reinterpret_cast<uint32_t*>(codes) + c);
      }
      if (c < nchunks && (c & (L - 1)) == 0) scales[c / L] = (uint8_t)cache_scale_byte<FMT>(k);
    }
  }
}

template <int DT, int FMT, int L, class M>
__global__ void __launch_bounds__(kThreads) k_dequantize_cache_packed(const uint8_t* __restrict__ codes,
                                                                    const uint8_t* __restrict__ scales,
                                                                    uint8_t* __restrict__ out, int64_t nchunks) {
  const int64_t step = (int64_t)gridDim.x * kThreads * M::kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * M::kUnroll; base < nchunks; base += step) {
    u32x2_t cw[M::kUnroll];
    uint32_t sb[M::kUnroll];
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      if constexpr (FMT == FMT_FP8) cw[u] = c < nchunks ? M::ld(reinterpret_cast<const u32x2_t*>(codes) + c) : u32x2_t{0u, 0u};
      else cw[u].x = c < nchunks ? M::ld(reinterpret_cast<const uint32_t*>(codes) + c) : 0u;
      sb[u] = c < nchunks ? (uint32_t)scales[c / L] : 0u;
    }
    // mxfp4: every load has landed.  Without this wait the compiler sinks
    // the decodes into the conditional stores and waits for vmcnt(0) inside
    // each, where the count includes the stores just issued, so the chunks'
    // stores run one after another: the packed mxfp4 load of the bf16
    // [4, 8192, 512] cache took 7.84 us that way and takes 7.31 us with it
    // (bit-identical).  The fp8 load, compiled the same way, measured 7%
    // slower with the wait, and the nvfp4 load keeps a single wait either
    // way, so only mxfp4 takes it.
    if constexpr (FMT == FMT_MXFP4) __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);   // vmcnt(0)
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int64_t c = base + u * kThreads + threadIdx.x;
      const float s = cache_scale_value<FMT>(sb[u]);
      Chunk<DT> o;
      if constexpr (FMT == FMT_FP8) decode_fp8_chunk<DT>(cw[u].x, cw[u].y, s, o);
      else if constexpr (FMT == FMT_NVFP4) nvfp4_decode_chunk<DT>(clear_negzero_codes(cw[u].x), s, o);
      else decode_fp4_chunk<DT>(clear_negzero_codes(cw[u].x), s, o);
      if (c < nchunks) store_chunk<DT, M>(out, c, o);
    }
  }
}

// General path: one thread per group (whole groups of any size, even for the
// fp4 formats; any alignment).
template <int DT, int FMT>
__global__ void __launch_bounds__(kThreads) k_quantize_cache_packed_general(const uint8_t* __restrict__ x,
                                                                          uint8_t* __restrict__ codes,
                                                                          uint8_t* __restrict__ scales,
                                                                          int64_t groups, int64_t block) {
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups; g += (int64_t)gridDim.x * kThreads) {
    const int64_t o0 = g * block;
    uint32_t amax = 0;
    for (int64_t i = 0; i < block; ++i) amax = max(amax, as_u32(load_elem<DT>(x, o0 + i)) & 0x7FFFFFFFu);
    const int k = ceil_rule_exponent<FMT>(amax);
    const float s = pow2f(k);
    if constexpr (FMT == FMT_FP8) {
      for (int64_t i = 0; i < block; ++i)
        codes[o0 + i] = (uint8_t)(enc_fp8_f2<false>(0u, load_elem<DT>(x, o0 + i), 0.0f, s) & 0xFFu);
    } else {
      for (int64_t j = 0; j < block / 2; ++j) {
        const float a = load_elem<DT>(x, o0 + 2 * j) + 0.0f, b = load_elem<DT>(x, o0 + 2 * j + 1) + 0.0f;
        codes[o0 / 2 + j] = (uint8_t)(enc_fp4_f2<0>(0u, a, b, s) & 0xFFu);
      }
    }
    scales[g] = (uint8_t)cache_scale_byte<FMT>(k);
  }
}

template <int DT, int FMT>
__global__ void __launch_bounds__(kThreads) k_dequantize_cache_packed_general(const uint8_t* __restrict__ codes,
                                                                            const uint8_t* __restrict__ scales,
                                                                            uint8_t* __restrict__ out,
                                                                            int64_t groups, int64_t block) {
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups; g += (int64_t)gridDim.x * kThreads) {
    const int64_t o0 = g * block;
    const float s = cache_scale_value<FMT>(scales[g]);
    if constexpr (FMT == FMT_FP8) {
      for (int64_t i = 0; i < block; ++i) {
        const uint32_t code = codes[o0 + i];
        const float v = dec_fp8_f2<false>(code, s).x;
        store_elem<DT>(out, o0 + i, v, DT == DT_BF16 ? dec_fp8_bf16x2<false>(code, s) & 0xFFFFu : 0u);
      }
    } else {
      for (int64_t j = 0; j < block / 2; ++j) {
        const uint32_t code = clear_negzero_codes((uint32_t)codes[o0 / 2 + j]);
        if constexpr (FMT == FMT_NVFP4) {
          const uint32_t h = dec_fp4_bf16x2<0>(code, 1.0f);
          const float v0 = mul_f32(bf16_lo(h), s), v1 = mul_f32(bf16_hi(h), s);
          const uint32_t bb = pack_bf16x2_rne(v0, v1);
          store_elem<DT>(out, o0 + 2 * j, v0, bb & 0xFFFFu);
          store_elem<DT>(out, o0 + 2 * j + 1, v1, bb >> 16);
        } else if constexpr (DT == DT_F16) {
          const uint32_t h = dec_fp4_f16x2<0>(code, s);
          *reinterpret_cast<unsigned short*>(out + 2 * (o0 + 2 * j)) = (unsigned short)(h & 0xFFFFu);
          *reinterpret_cast<unsigned short*>(out + 2 * (o0 + 2 * j + 1)) = (unsigned short)(h >> 16);
        } else {
          const uint32_t h = dec_fp4_bf16x2<0>(code, s);
          store_elem<DT>(out, o0 + 2 * j, as_f32(h << 16), h & 0xFFFFu);
          store_elem<DT>(out, o0 + 2 * j + 1, as_f32(h & 0xFFFF0000u), h >> 16);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launchers
static inline int grid_for(int64_t items, int64_t per_block, int64_t cap = kGridCap) {
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
    hipLaunchKernelGGL((k_dequantize_mxfp4<DT, StreamDequant>), dim3(grid_for(nchunks, kThreads * StreamDequant::kUnroll, kDequantGridCap)),
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

// Packed cache storage.  Fast path: block a power of two in [8, 512], 16-byte
// aligned x / out and codes aligned to one chunk's codes (4 or 8 bytes).
template <int FMT>
static bool packed_fast(int32_t block, const void* elems, const void* codes) {
  const bool pow2 = block >= 8 && block <= 512 && (block & (block - 1)) == 0;
  return pow2 && aligned(elems, 16) && aligned(codes, FMT == FMT_FP8 ? 8 : 4);
}

template <int DT, int FMT, int L>
static void launch_packed_q(const void* x, uint8_t* codes, uint8_t* scales, int64_t nchunks, hipStream_t st) {
  const int64_t bytes = nchunks * 8 * (DT == DT_F32 ? 4 : 2);
  const uint8_t* xp = (const uint8_t*)x;
  if (bytes >= kBigStreamBytes)
    hipLaunchKernelGGL((k_quantize_cache_packed<DT, FMT, L, StreamBig>),
                       dim3(grid_for(nchunks, kThreads * StreamBig::kUnroll)), dim3(kThreads), 0, st, xp, codes, scales,
                       nchunks);
  else if (bytes >= kTinyStreamBytes && FMT == FMT_FP8)
    hipLaunchKernelGGL((k_quantize_cache_packed<DT, FMT, L, StreamSmall>),
                       dim3(grid_for(nchunks, kThreads * StreamSmall::kUnroll)), dim3(kThreads), 0, st, xp, codes,
                       scales, nchunks);
  else if (bytes >= kTinyStreamBytes)   // e2m1 codes: 4 chunks per lane measured ~8% faster on a 32 MiB cache
    hipLaunchKernelGGL((k_quantize_cache_packed<DT, FMT, L, StreamDequant>),
                       dim3(grid_for(nchunks, kThreads * StreamDequant::kUnroll)), dim3(kThreads), 0, st, xp, codes,
                       scales, nchunks);
  else
    hipLaunchKernelGGL((k_quantize_cache_packed<DT, FMT, L, StreamTiny>),
                       dim3(grid_for(nchunks, kThreads * StreamTiny::kUnroll)), dim3(kThreads), 0, st, xp, codes,
                       scales, nchunks);
}

template <int DT, int FMT, int L>
static void launch_packed_dq(const uint8_t* codes, const uint8_t* scales, void* out, int64_t nchunks,
                             hipStream_t st) {
  hipLaunchKernelGGL((k_dequantize_cache_packed<DT, FMT, L, StreamDequant>),
                     dim3(grid_for(nchunks, kThreads * StreamDequant::kUnroll)), dim3(kThreads), 0, st, codes, scales,
                     (uint8_t*)out, nchunks);
}

template <int DT, int FMT>
static hipError_t launch_cache_packed_t(bool dequant, const void* x, uint8_t* codes, const uint8_t* scales_in,
                                        uint8_t* scales_out, void* out, int64_t n, int32_t block, hipStream_t st) {
  if (packed_fast<FMT>(block, dequant ? out : x, codes)) {
    const int64_t nc = n / 8;
#define MXQ_PACKED_CASE(B, L)                                                        \
  case B:                                                                            \
    if (dequant) launch_packed_dq<DT, FMT, L>(codes, scales_in, out, nc, st);       \
    else launch_packed_q<DT, FMT, L>(x, codes, scales_out, nc, st);                 \
    break;
    switch (block) {
      MXQ_PACKED_CASE(8, 1)
      MXQ_PACKED_CASE(16, 2)
      MXQ_PACKED_CASE(32, 4)
      MXQ_PACKED_CASE(64, 8)
      MXQ_PACKED_CASE(128, 16)
      MXQ_PACKED_CASE(256, 32)
      default: MXQ_PACKED_CASE(512, 64)
    }
#undef MXQ_PACKED_CASE
  } else {
    const int64_t groups = n / block;
    if (dequant)
      hipLaunchKernelGGL((k_dequantize_cache_packed_general<DT, FMT>), dim3(grid_for(groups, kThreads)), dim3(kThreads),
                         0, st, codes, scales_in, (uint8_t*)out, groups, (int64_t)block);
    else
      hipLaunchKernelGGL((k_quantize_cache_packed_general<DT, FMT>), dim3(grid_for(groups, kThreads)), dim3(kThreads),
                         0, st, (const uint8_t*)x, codes, scales_out, groups, (int64_t)block);
  }
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_cache_packed_dt(bool dequant, const void* x, uint8_t* codes, const uint8_t* si, uint8_t* so,
                                         void* out, int64_t n, int fmt, int32_t block, hipStream_t st) {
  switch (fmt) {
    case FMT_FP8: return launch_cache_packed_t<DT, FMT_FP8>(dequant, x, codes, si, so, out, n, block, st);
    case FMT_MXFP4: return launch_cache_packed_t<DT, FMT_MXFP4>(dequant, x, codes, si, so, out, n, block, st);
    default: return launch_cache_packed_t<DT, FMT_NVFP4>(dequant, x, codes, si, so, out, n, block, st);
  }
}

static hipError_t launch_cache_packed(bool dequant, const void* x, uint8_t* codes, const uint8_t* si, uint8_t* so,
                                      void* out, int dt, int64_t n, int fmt, int32_t block, hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_cache_packed_dt<DT_F32>(dequant, x, codes, si, so, out, n, fmt, block, st);
    case DT_BF16: return launch_cache_packed_dt<DT_BF16>(dequant, x, codes, si, so, out, n, fmt, block, st);
    default: return launch_cache_packed_dt<DT_F16>(dequant, x, codes, si, so, out, n, fmt, block, st);
  }
}

hipError_t launch_quantize_cache_packed(const void* x, int dt, int64_t rows, int64_t channels, int fmt, int32_t block,
                                        uint8_t* codes, uint8_t* scales, hipStream_t st) {
  return launch_cache_packed(false, x, codes, nullptr, scales, nullptr, dt, rows * channels, fmt, block, st);
}

hipError_t launch_dequantize_cache_packed(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t channels,
                                          int fmt, int32_t block, void* out, int dt, hipStream_t st) {
  return launch_cache_packed(true, nullptr, const_cast<uint8_t*>(codes), scales, nullptr, out, dt, rows * channels,
                             fmt, block, st);
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

hipError_t copy_to_host_sync(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  const hipError_t e = hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

// At most 1024 workgroups for the amax pass: each ends with one atomic on
// the same word, and 16384 of them (the streaming cap) measured 35% slower.
constexpr int kAmaxGridCap = 1024;

template <int DT, class M>
static void launch_nvfp4_fast(const void* x, int64_t nchunks, uint32_t* packed, uint8_t* scales, uint32_t* slot,
                              hipStream_t st) {
  const int g = grid_for(nchunks, kThreads * M::kUnroll);
  hipLaunchKernelGGL((k_nvfp4_amax<DT, M>), dim3(std::min(g, kAmaxGridCap)), dim3(kThreads), 0, st, (const uint8_t*)x,
                     nchunks, slot);
  hipLaunchKernelGGL((k_quantize_nvfp4<DT, M>), dim3(g), dim3(kThreads), 0, st, (const uint8_t*)x, packed, scales,
                     nchunks, (const uint32_t*)slot);
}

template <int DT>
static hipError_t launch_quantize_nvfp4_t(const void* x, int64_t rows, int64_t k, uint8_t* packed, uint8_t* scales,
                                          float* gscale, hipStream_t st) {
  const int64_t n = rows * k;
  uint32_t* slot = reinterpret_cast<uint32_t*>(gscale);
  hipLaunchKernelGGL(k_nvfp4_amax_init, dim3(1), dim3(1), 0, st, slot);
  if (aligned(x, 16) && aligned(packed, 4)) {
    const int64_t nchunks = n / 8, bytes = n * (DT == DT_F32 ? 4 : 2);
    if (bytes >= kBigStreamBytes) launch_nvfp4_fast<DT, StreamBig>(x, nchunks, (uint32_t*)packed, scales, slot, st);
    else if (bytes >= kTinyStreamBytes) launch_nvfp4_fast<DT, StreamSmall>(x, nchunks, (uint32_t*)packed, scales, slot, st);
    else launch_nvfp4_fast<DT, StreamTiny>(x, nchunks, (uint32_t*)packed, scales, slot, st);
  } else {
    hipLaunchKernelGGL(k_nvfp4_amax_general<DT>, dim3(std::min(grid_for(n, kThreads * 16), kAmaxGridCap)), dim3(kThreads), 0, st,
                       (const uint8_t*)x, n, slot);
    hipLaunchKernelGGL(k_quantize_nvfp4_general<DT>, dim3(grid_for(n / 16, kThreads)), dim3(kThreads), 0, st,
                       (const uint8_t*)x, packed, scales, n / 16, (const uint32_t*)slot);
  }
  hipLaunchKernelGGL(k_nvfp4_finalize, dim3(1), dim3(1), 0, st, slot);
  return hipGetLastError();
}

hipError_t launch_quantize_nvfp4(const void* x, int dt, int64_t rows, int64_t k, uint8_t* packed, uint8_t* scales,
                                 float* global_scale, hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_quantize_nvfp4_t<DT_F32>(x, rows, k, packed, scales, global_scale, st);
    case DT_BF16: return launch_quantize_nvfp4_t<DT_BF16>(x, rows, k, packed, scales, global_scale, st);
    default: return launch_quantize_nvfp4_t<DT_F16>(x, rows, k, packed, scales, global_scale, st);
  }
}

template <int DT>
static hipError_t launch_quantize_nvfp4_mse_t(const void* x, int64_t rows, int64_t k, uint8_t* packed,
                                              uint8_t* scales, float* gscale, hipStream_t st) {
  const int64_t n = rows * k;
  uint32_t* slot = reinterpret_cast<uint32_t*>(gscale);
  hipLaunchKernelGGL(k_nvfp4_amax_init, dim3(1), dim3(1), 0, st, slot);
  if (aligned(x, 16)) {
    const int64_t nchunks = n / 8, bytes = n * (DT == DT_F32 ? 4 : 2);
    if (bytes >= kBigStreamBytes)
      hipLaunchKernelGGL((k_nvfp4_amax<DT, StreamBig>),
                         dim3(std::min(grid_for(nchunks, kThreads * StreamBig::kUnroll), kAmaxGridCap)), dim3(kThreads),
                         0, st, (const uint8_t*)x, nchunks, slot);
    else if (bytes >= kTinyStreamBytes)
      hipLaunchKernelGGL((k_nvfp4_amax<DT, StreamSmall>),
                         dim3(std::min(grid_for(nchunks, kThreads * StreamSmall::kUnroll), kAmaxGridCap)),
                         dim3(kThreads), 0, st, (const uint8_t*)x, nchunks, slot);
    else
      hipLaunchKernelGGL((k_nvfp4_amax<DT, StreamTiny>),
                         dim3(std::min(grid_for(nchunks, kThreads * StreamTiny::kUnroll), kAmaxGridCap)),
                         dim3(kThreads), 0, st, (const uint8_t*)x, nchunks, slot);
  } else {
    hipLaunchKernelGGL(k_nvfp4_amax_general<DT>, dim3(std::min(grid_for(n, kThreads * 16), kAmaxGridCap)),
                       dim3(kThreads), 0, st, (const uint8_t*)x, n, slot);
  }
  hipLaunchKernelGGL(k_quantize_nvfp4_mse<DT>, dim3(grid_for(n / 16, kThreads)), dim3(kThreads), 0, st,
                     (const uint8_t*)x, packed, scales, n / 16, (const uint32_t*)slot);
  hipLaunchKernelGGL(k_nvfp4_finalize, dim3(1), dim3(1), 0, st, slot);
  return hipGetLastError();
}

hipError_t launch_quantize_nvfp4_mse(const void* x, int dt, int64_t rows, int64_t k, uint8_t* packed,
                                     uint8_t* scales, float* global_scale, hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_quantize_nvfp4_mse_t<DT_F32>(x, rows, k, packed, scales, global_scale, st);
    case DT_BF16: return launch_quantize_nvfp4_mse_t<DT_BF16>(x, rows, k, packed, scales, global_scale, st);
    default: return launch_quantize_nvfp4_mse_t<DT_F16>(x, rows, k, packed, scales, global_scale, st);
  }
}

template <int DT>
static hipError_t launch_dequantize_nvfp4_t(const uint8_t* packed, const uint8_t* scales, const float* gscale,
                                            int64_t rows, int64_t k, void* out, hipStream_t st) {
  const int64_t n = rows * k;
  if (aligned(packed, 4) && aligned(out, 16)) {
    const int64_t nchunks = n / 8;
    hipLaunchKernelGGL((k_dequantize_nvfp4<DT, StreamDequant>), dim3(grid_for(nchunks, kThreads * StreamDequant::kUnroll, kDequantGridCap)),
                       dim3(kThreads), 0, st, (const uint32_t*)packed, scales, gscale, (uint8_t*)out, nchunks);
  } else {
    hipLaunchKernelGGL(k_dequantize_nvfp4_general<DT>, dim3(grid_for(n / 16, kThreads)), dim3(kThreads), 0, st,
                       packed, scales, gscale, (uint8_t*)out, n / 16);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize_nvfp4(const uint8_t* packed, const uint8_t* scales, const float* global_scale,
                                   int64_t rows, int64_t k, void* out, int dt, hipStream_t st) {
  switch (dt) {
    case DT_F32: return launch_dequantize_nvfp4_t<DT_F32>(packed, scales, global_scale, rows, k, out, st);
    case DT_BF16: return launch_dequantize_nvfp4_t<DT_BF16>(packed, scales, global_scale, rows, k, out, st);
    default: return launch_dequantize_nvfp4_t<DT_F16>(packed, scales, global_scale, rows, k, out, st);
  }
}

}  // namespace mxq
