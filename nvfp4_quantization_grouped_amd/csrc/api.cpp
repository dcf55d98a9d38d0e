// C ABI of libmxq (declared in include/mxq.h): host-side validation, then
// one asynchronous launch on the caller's stream.  No allocation, no sync.
#include <vector>
#include "../../include/mxq.h"
#include "launch.hpp"

namespace {

bool dtype_ok(int t) { return t == MXQ_F32 || t == MXQ_BF16 || t == MXQ_F16; }
int64_t dtype_bytes(int t) { return t == MXQ_F32 ? 4 : 2; }

// Do [a, a + na) and [b, b + nb) overlap?
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return na > 0 && nb > 0 && pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

int from_hip(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP; }

}  // namespace

extern "C" {

int quantize_mxfp4(const void* x, int xt, int64_t rows, int64_t k, int8_t* packed, uint8_t* scales, void* stream) {
  if (rows < 0 || k < 0 || k % 32 != 0) return MXQ_ERR_SHAPE;
  if (!dtype_ok(xt)) return MXQ_ERR_DTYPE;
  if (rows == 0 || k == 0) return MXQ_OK;
  if (!x || !packed || !scales) return MXQ_ERR_NULL;
  const int64_t n = rows * k;
  if (overlap(x, n * dtype_bytes(xt), packed, n / 2) || overlap(x, n * dtype_bytes(xt), scales, n / 32) ||
      overlap(packed, n / 2, scales, n / 32))
    return MXQ_ERR_ALIAS;
  return from_hip(mxq::launch_quantize_mxfp4(x, xt, rows, k, packed, scales, (hipStream_t)stream));
}

int dequantize_mxfp4(const int8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, void* out, int ot,
                     void* stream) {
  if (rows < 0 || k < 0 || k % 32 != 0) return MXQ_ERR_SHAPE;
  if (!dtype_ok(ot)) return MXQ_ERR_DTYPE;
  if (rows == 0 || k == 0) return MXQ_OK;
  if (!packed || !scales || !out) return MXQ_ERR_NULL;
  const int64_t n = rows * k;
  if (overlap(out, n * dtype_bytes(ot), packed, n / 2) || overlap(out, n * dtype_bytes(ot), scales, n / 32))
    return MXQ_ERR_ALIAS;
  return from_hip(mxq::launch_dequantize_mxfp4(packed, scales, rows, k, out, ot, (hipStream_t)stream));
}

int quantize_cache(const void* x, void* out, int t, int64_t rows, int64_t channels, int fmt, int32_t block_size,
                   void* stream) {
  if (rows < 0 || channels < 0) return MXQ_ERR_SHAPE;
  if (!dtype_ok(t)) return MXQ_ERR_DTYPE;
  if (fmt != MXQ_FMT_FP8 && fmt != MXQ_FMT_MXFP4 && fmt != MXQ_FMT_NVFP4) return MXQ_ERR_FORMAT;
  if (block_size <= 0) return MXQ_ERR_BLOCK;
  if (rows == 0 || channels == 0) return MXQ_OK;
  if (!x || !out) return MXQ_ERR_NULL;
  const int64_t bytes = rows * channels * dtype_bytes(t);
  if (overlap(x, bytes, out, bytes)) return MXQ_ERR_ALIAS;
  return from_hip(mxq::launch_quantize_cache(x, out, t, rows, channels, fmt, block_size, (hipStream_t)stream));
}

int quantize_cache_bwd(const void* grad_out, void* grad_in, int t, int64_t numel, void* stream) {
  if (numel < 0) return MXQ_ERR_SHAPE;
  if (!dtype_ok(t)) return MXQ_ERR_DTYPE;
  if (numel == 0) return MXQ_OK;
  if (!grad_out || !grad_in) return MXQ_ERR_NULL;
  if (grad_out == grad_in) return MXQ_OK;   // already the identity
  const int64_t bytes = numel * dtype_bytes(t);
  if (overlap(grad_out, bytes, grad_in, bytes)) return MXQ_ERR_ALIAS;
  return from_hip(mxq::launch_copy(grad_out, grad_in, bytes, (hipStream_t)stream));
}

// Shared argument checks of the packed cache entries; sets the code and scale byte counts.
static int cache_packed_check(int t, int64_t rows, int64_t channels, int fmt, int32_t block, int64_t* ncode,
                              int64_t* nscale) {
  if (rows < 0 || channels < 0) return MXQ_ERR_SHAPE;
  if (!dtype_ok(t)) return MXQ_ERR_DTYPE;
  if (fmt != MXQ_FMT_FP8 && fmt != MXQ_FMT_MXFP4 && fmt != MXQ_FMT_NVFP4) return MXQ_ERR_FORMAT;
  if (block <= 0 || (fmt != MXQ_FMT_FP8 && block % 2 != 0)) return MXQ_ERR_BLOCK;
  if (channels % block != 0) return MXQ_ERR_SHAPE;
  const int64_t n = rows * channels;
  *ncode = fmt == MXQ_FMT_FP8 ? n : n / 2;
  *nscale = n / block;
  return MXQ_OK;
}

int quantize_cache_packed(const void* x, int t, int64_t rows, int64_t channels, int fmt, int32_t block_size,
                          uint8_t* codes, uint8_t* scales, void* stream) {
  int64_t nc = 0, ns = 0;
  const int st = cache_packed_check(t, rows, channels, fmt, block_size, &nc, &ns);
  if (st != MXQ_OK) return st;
  if (rows == 0 || channels == 0) return MXQ_OK;
  if (!x || !codes || !scales) return MXQ_ERR_NULL;
  const int64_t xb = rows * channels * dtype_bytes(t);
  if (overlap(x, xb, codes, nc) || overlap(x, xb, scales, ns) || overlap(codes, nc, scales, ns)) return MXQ_ERR_ALIAS;
  return from_hip(
      mxq::launch_quantize_cache_packed(x, t, rows, channels, fmt, block_size, codes, scales, (hipStream_t)stream));
}

int dequantize_cache_packed(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t channels, int fmt,
                            int32_t block_size, void* out, int t, void* stream) {
  int64_t nc = 0, ns = 0;
  const int st = cache_packed_check(t, rows, channels, fmt, block_size, &nc, &ns);
  if (st != MXQ_OK) return st;
  if (rows == 0 || channels == 0) return MXQ_OK;
  if (!codes || !scales || !out) return MXQ_ERR_NULL;
  const int64_t ob = rows * channels * dtype_bytes(t);
  if (overlap(out, ob, codes, nc) || overlap(out, ob, scales, ns)) return MXQ_ERR_ALIAS;
  return from_hip(mxq::launch_dequantize_cache_packed(codes, scales, rows, channels, fmt, block_size, out, t,
                                                      (hipStream_t)stream));
}

// Checks shared by the two NVFP4 quantizers; MXQ_OK with *launch = false means nothing to do.
static int nvfp4_quantize_check(const void* x, int xt, int64_t rows, int64_t k, const uint8_t* packed,
                                const uint8_t* block_scales, const float* global_scale, bool* launch) {
  *launch = false;
  if (rows < 0 || k < 0 || k % 16 != 0) return MXQ_ERR_SHAPE;
  if (!dtype_ok(xt)) return MXQ_ERR_DTYPE;
  if (rows == 0 || k == 0) return MXQ_OK;
  if (!x || !packed || !block_scales || !global_scale) return MXQ_ERR_NULL;
  if ((uintptr_t)global_scale & 3) return MXQ_ERR_ALIGN;
  const int64_t n = rows * k, xb = n * dtype_bytes(xt);
  if (overlap(x, xb, packed, n / 2) || overlap(x, xb, block_scales, n / 16) || overlap(x, xb, global_scale, 4) ||
      overlap(packed, n / 2, block_scales, n / 16) || overlap(packed, n / 2, global_scale, 4) ||
      overlap(block_scales, n / 16, global_scale, 4))
    return MXQ_ERR_ALIAS;
  *launch = true;
  return MXQ_OK;
}

int quantize_nvfp4(const void* x, int xt, int64_t rows, int64_t k, uint8_t* packed, uint8_t* block_scales,
                   float* global_scale, void* stream) {
  bool launch = false;
  const int st = nvfp4_quantize_check(x, xt, rows, k, packed, block_scales, global_scale, &launch);
  if (st != MXQ_OK || !launch) return st;
  return from_hip(mxq::launch_quantize_nvfp4(x, xt, rows, k, packed, block_scales, global_scale, (hipStream_t)stream));
}

int quantize_nvfp4_mse(const void* x, int xt, int64_t rows, int64_t k, uint8_t* packed, uint8_t* block_scales,
                       float* global_scale, void* stream) {
  bool launch = false;
  const int st = nvfp4_quantize_check(x, xt, rows, k, packed, block_scales, global_scale, &launch);
  if (st != MXQ_OK || !launch) return st;
  return from_hip(
      mxq::launch_quantize_nvfp4_mse(x, xt, rows, k, packed, block_scales, global_scale, (hipStream_t)stream));
}

int dequantize_nvfp4(const uint8_t* packed, const uint8_t* block_scales, const float* global_scale, int64_t rows,
                     int64_t k, void* out, int ot, void* stream) {
  if (rows < 0 || k < 0 || k % 16 != 0) return MXQ_ERR_SHAPE;
  if (!dtype_ok(ot)) return MXQ_ERR_DTYPE;
  if (rows == 0 || k == 0) return MXQ_OK;
  if (!packed || !block_scales || !global_scale || !out) return MXQ_ERR_NULL;
  if ((uintptr_t)global_scale & 3) return MXQ_ERR_ALIGN;
  const int64_t n = rows * k, ob = n * dtype_bytes(ot);
  if (overlap(out, ob, packed, n / 2) || overlap(out, ob, block_scales, n / 16) || overlap(out, ob, global_scale, 4))
    return MXQ_ERR_ALIAS;
  return from_hip(
      mxq::launch_dequantize_nvfp4(packed, block_scales, global_scale, rows, k, out, ot, (hipStream_t)stream));
}

static int grouped_mm_check(const void* a, int64_t tokens, int64_t red, const int8_t* packed, const uint8_t* scales,
                            int64_t experts, int64_t other, const int32_t* offs, void* out, int64_t k, int64_t n) {
  if (tokens < 0 || red < 0 || other < 0 || experts < 0) return MXQ_ERR_SHAPE;
  if (k % 32 != 0 || n % 8 != 0) return MXQ_ERR_SHAPE;
  if (tokens > 0 && other > 0 && (!a || !out || (experts > 0 && (!packed || !scales || !offs)))) return MXQ_ERR_NULL;
  if (((uintptr_t)a & 15) || ((uintptr_t)packed & 15) || ((uintptr_t)out & 15)) return MXQ_ERR_ALIGN;
  if (overlap(a, tokens * red * 2, out, tokens * other * 2)) return MXQ_ERR_ALIAS;
  return MXQ_OK;
}

int mxfp4_grouped_mm_fwd(const void* x, int64_t tokens, int64_t k, const int8_t* packed, const uint8_t* scales,
                         int64_t experts, int64_t n, const int32_t* offs, void* y, void* stream) {
  const int st = grouped_mm_check(x, tokens, k, packed, scales, experts, n, offs, y, k, n);
  if (st != MXQ_OK) return st;
  if (tokens == 0 || n == 0) return MXQ_OK;
  if (k == 0 || experts == 0) {   // nothing to reduce / no expert owns any row: y = 0
    return from_hip(mxq::launch_zero(y, tokens * n * 2, (hipStream_t)stream));
  }
  return from_hip(mxq::launch_grouped_mm(false, x, tokens, packed, scales, experts, n, k, offs, y, (hipStream_t)stream));
}

int mxfp4_grouped_mm_bwd_x(const void* grad_out, int64_t tokens, int64_t n, const int8_t* packed,
                           const uint8_t* scales, int64_t experts, int64_t k, const int32_t* offs, void* grad_x,
                           void* stream) {
  const int st = grouped_mm_check(grad_out, tokens, n, packed, scales, experts, k, offs, grad_x, k, n);
  if (st != MXQ_OK) return st;
  // the kernel addresses a row tile of grad_out and one expert's weights with 32-bit offsets
  if (n > (int64_t(1) << 22) || n * (k / 2) >= (int64_t(1) << 31)) return MXQ_ERR_SHAPE;
  if (tokens == 0 || k == 0) return MXQ_OK;
  if (n == 0 || experts == 0) {
    return from_hip(mxq::launch_zero(grad_x, tokens * k * 2, (hipStream_t)stream));
  }
  return from_hip(
      mxq::launch_grouped_mm(true, grad_out, tokens, packed, scales, experts, n, k, offs, grad_x, (hipStream_t)stream));
}

int mxq_validate_offs(const int32_t* offs, int64_t experts, int64_t tokens, int64_t* first_bad, void* stream) {
  if (first_bad) *first_bad = -1;
  if (experts < 0 || tokens < 0 || experts > (int64_t(1) << 26)) return MXQ_ERR_SHAPE;
  if (experts == 0) return MXQ_OK;
  if (!offs) return MXQ_ERR_NULL;
  std::vector<int32_t> h((size_t)experts);
  if (mxq::copy_to_host_sync(offs, h.data(), experts * 4, (hipStream_t)stream) != hipSuccess) return MXQ_ERR_HIP;
  int64_t prev = 0;
  for (int64_t e = 0; e < experts; ++e) {
    if (h[(size_t)e] < prev || h[(size_t)e] > tokens) {
      if (first_bad) *first_bad = e;
      return MXQ_ERR_OFFS;
    }
    prev = h[(size_t)e];
  }
  return MXQ_OK;
}

int mxfp4_grouped_mm_fwd_w4a4(const int8_t* xq, const uint8_t* xs, int64_t tokens, int64_t k, const int8_t* packed,
                              const uint8_t* scales, int64_t experts, int64_t n, const int32_t* offs, void* y,
                              void* stream) {
  if (tokens < 0 || k < 0 || n < 0 || experts < 0) return MXQ_ERR_SHAPE;
  // whole 16-byte scale chunks per row; 32-bit buffer offsets into one expert's weights
  if (k % 512 != 0 || n % 8 != 0 || k >= (int64_t(1) << 22) || n * (k / 2) >= (int64_t(1) << 31)) return MXQ_ERR_SHAPE;
  if (tokens > 0 && n > 0 && (!y || (k > 0 && (!xq || !xs)) || (k > 0 && experts > 0 && (!packed || !scales || !offs))))
    return MXQ_ERR_NULL;
  if (((uintptr_t)xq & 15) || ((uintptr_t)xs & 15) || ((uintptr_t)packed & 15) || ((uintptr_t)scales & 15) ||
      ((uintptr_t)y & 15))
    return MXQ_ERR_ALIGN;
  const int64_t ybytes = tokens * n * 2;
  if (overlap(xq, tokens * (k / 2), y, ybytes) || overlap(xs, tokens * (k / 32), y, ybytes)) return MXQ_ERR_ALIAS;
  if (tokens == 0 || n == 0) return MXQ_OK;
  if (k == 0 || experts == 0) return from_hip(mxq::launch_zero(y, ybytes, (hipStream_t)stream));
  return from_hip(
      mxq::launch_grouped_mm_w4a4(xq, xs, tokens, packed, scales, experts, n, k, offs, y, (hipStream_t)stream));
}

int mxfp4_grouped_mm_fwd_w4a8(const uint8_t* xq, const uint8_t* xs, int64_t tokens, int64_t k, const int8_t* packed,
                              const uint8_t* scales, int64_t experts, int64_t n, const int32_t* offs, void* y,
                              void* stream) {
  if (tokens < 0 || k < 0 || n < 0 || experts < 0) return MXQ_ERR_SHAPE;
  // whole 16-byte scale chunks per row; 32-bit buffer offsets into one expert's weights
  if (k % 512 != 0 || n % 8 != 0 || k >= (int64_t(1) << 22) || n * (k / 2) >= (int64_t(1) << 31)) return MXQ_ERR_SHAPE;
  if (tokens > 0 && n > 0 && (!y || (k > 0 && (!xq || !xs)) || (k > 0 && experts > 0 && (!packed || !scales || !offs))))
    return MXQ_ERR_NULL;
  if (((uintptr_t)xq & 15) || ((uintptr_t)xs & 15) || ((uintptr_t)packed & 15) || ((uintptr_t)scales & 15) ||
      ((uintptr_t)y & 15))
    return MXQ_ERR_ALIGN;
  const int64_t ybytes = tokens * n * 2;
  if (overlap(xq, tokens * k, y, ybytes) || overlap(xs, tokens * (k / 32), y, ybytes)) return MXQ_ERR_ALIAS;
  if (tokens == 0 || n == 0) return MXQ_OK;
  if (k == 0 || experts == 0) return from_hip(mxq::launch_zero(y, ybytes, (hipStream_t)stream));
  return from_hip(
      mxq::launch_grouped_mm_w4a8(xq, xs, tokens, packed, scales, experts, n, k, offs, y, (hipStream_t)stream));
}

const char* mxq_status_string(int s) {
  switch (s) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "null pointer";
    case MXQ_ERR_SHAPE: return "bad shape (negative size, k not a multiple of the block (32 mxfp4, 16 nvfp4, 512 W4A4 and W4A8), n not a multiple of 8, or past a size limit)";
    case MXQ_ERR_DTYPE: return "unsupported dtype";
    case MXQ_ERR_FORMAT: return "unknown format (fp8, mxfp4 or nvfp4)";
    case MXQ_ERR_BLOCK: return "block_size must be positive";
    case MXQ_ERR_ALIGN: return "misaligned pointer (grouped GEMM activations, packed weights and output need 16-byte alignment)";
    case MXQ_ERR_ALIAS: return "output overlaps an input";
    case MXQ_ERR_HIP: return "HIP launch error";
    case MXQ_ERR_OFFS: return "offs is not non-decreasing within [0, tokens]";
    default: return "unknown status";
  }
}

}  // extern "C"
