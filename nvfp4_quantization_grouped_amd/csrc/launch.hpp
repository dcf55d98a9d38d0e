// Host-side launchers of the libmxq kernels (internal; the public ABI is
// include/mxq.h).  Each launcher enqueues on `st` and returns the HIP error
// of the launch.  Arguments are validated by the ABI layer before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

hipError_t launch_quantize_mxfp4(const void* x, int dt, int64_t rows, int64_t k, int8_t* packed, uint8_t* scales,
                                 hipStream_t st);
hipError_t launch_dequantize_mxfp4(const int8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, void* out,
                                   int dt, hipStream_t st);
hipError_t launch_quantize_cache(const void* x, void* out, int dt, int64_t rows, int64_t channels, int fmt,
                                 int32_t block, hipStream_t st);
// Two-level NVFP4: packed e2m1 [n/2], E4M3 block-16 scales [n/16], FP32 global scale (1 float, device).
hipError_t launch_quantize_nvfp4(const void* x, int dt, int64_t rows, int64_t k, uint8_t* packed, uint8_t* scales,
                                 float* global_scale, hipStream_t st);
// Same outputs with the block scales chosen by the MSE sweep over the 126 positive finite E4M3 values.
hipError_t launch_quantize_nvfp4_mse(const void* x, int dt, int64_t rows, int64_t k, uint8_t* packed, uint8_t* scales,
                                     float* global_scale, hipStream_t st);
hipError_t launch_dequantize_nvfp4(const uint8_t* packed, const uint8_t* scales, const float* global_scale,
                                   int64_t rows, int64_t k, void* out, int dt, hipStream_t st);
// Packed cache storage: codes [n] (fp8) or [n/2] (e2m1), one scale byte per group; whole groups only.
hipError_t launch_quantize_cache_packed(const void* x, int dt, int64_t rows, int64_t channels, int fmt, int32_t block,
                                        uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_dequantize_cache_packed(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t channels,
                                          int fmt, int32_t block, void* out, int dt, hipStream_t st);
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t st);
hipError_t launch_zero(void* dst, int64_t bytes, hipStream_t st);
// device -> host copy on st, then wait for st (used only by the offs debug check)
hipError_t copy_to_host_sync(const void* src, void* dst, int64_t bytes, hipStream_t st);
// bwd = false: out[T, N] = a[T, K] W_e^T;  bwd = true: out[T, K] = a[T, N] W_e.
hipError_t launch_grouped_mm(bool bwd, const void* a, int64_t tokens, const int8_t* packed, const uint8_t* scales,
                             int64_t experts, int64_t wn_dim, int64_t wk_dim, const int32_t* offs, void* out,
                             hipStream_t st);
// out[T, N] = dq(xq)[T, K] dq(W_e)^T, both operands MXFP4 (K % 512 == 0).
hipError_t launch_grouped_mm_w4a4(const void* xq, const uint8_t* xs, int64_t tokens, const int8_t* packed,
                                  const uint8_t* scales, int64_t experts, int64_t n, int64_t k, const int32_t* offs,
                                  void* out, hipStream_t st);

// out[T, N] = dq(xq)[T, K] dq(W_e)^T, activations E4M3 with E8M0 block-32 scales (K % 512 == 0).
hipError_t launch_grouped_mm_w4a8(const void* xq, const uint8_t* xs, int64_t tokens, const int8_t* packed,
                                  const uint8_t* scales, int64_t experts, int64_t n, int64_t k, const int32_t* offs,
                                  void* out, hipStream_t st);

}  // namespace mxq
