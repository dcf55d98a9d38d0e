// Stand-ins for the kernel launchers of libmxq (csrc/launch.hpp) in the host
// AddressSanitizer build of the C ABI layer (csrc/api.cpp).  The ABI tests
// only make calls that must be answered on the host (a rejected argument or
// an empty problem); a call that gets past validation reaches one of these,
// which returns an error instead of launching, so the ABI reports
// MXQ_ERR_HIP and the test that made it fails.
#include "../../nvfp4_quantization_grouped_amd/csrc/launch.hpp"

namespace mxq {

static hipError_t reached() { return hipErrorNotSupported; }

hipError_t launch_quantize_mxfp4(const void*, int, int64_t, int64_t, int8_t*, uint8_t*, hipStream_t) { return reached(); }
hipError_t launch_dequantize_mxfp4(const int8_t*, const uint8_t*, int64_t, int64_t, void*, int, hipStream_t) {
  return reached();
}
hipError_t launch_quantize_cache(const void*, void*, int, int64_t, int64_t, int, int32_t, hipStream_t) { return reached(); }
hipError_t launch_quantize_nvfp4(const void*, int, int64_t, int64_t, uint8_t*, uint8_t*, float*, hipStream_t) {
  return reached();
}
hipError_t launch_quantize_nvfp4_mse(const void*, int, int64_t, int64_t, uint8_t*, uint8_t*, float*, hipStream_t) {
  return reached();
}
hipError_t launch_dequantize_nvfp4(const uint8_t*, const uint8_t*, const float*, int64_t, int64_t, void*, int,
                                   hipStream_t) {
  return reached();
}
hipError_t launch_quantize_cache_packed(const void*, int, int64_t, int64_t, int, int32_t, uint8_t*, uint8_t*,
                                        hipStream_t) {
  return reached();
}
hipError_t launch_dequantize_cache_packed(const uint8_t*, const uint8_t*, int64_t, int64_t, int, int32_t, void*, int,
                                          hipStream_t) {
  return reached();
}
hipError_t launch_copy(const void*, void*, int64_t, hipStream_t) { return reached(); }
hipError_t launch_zero(void*, int64_t, hipStream_t) { return reached(); }
hipError_t copy_to_host_sync(const void*, void*, int64_t, hipStream_t) { return reached(); }
hipError_t launch_grouped_mm(bool, const void*, int64_t, const int8_t*, const uint8_t*, int64_t, int64_t, int64_t,
                             const int32_t*, void*, hipStream_t) {
  return reached();
}
hipError_t launch_grouped_mm_w4a4(const void*, const uint8_t*, int64_t, const int8_t*, const uint8_t*, int64_t, int64_t,
                                  int64_t, const int32_t*, void*, hipStream_t) {
  return reached();
}

hipError_t launch_grouped_mm_w4a8(const void*, const uint8_t*, int64_t, const int8_t*, const uint8_t*, int64_t, int64_t,
                                  int64_t, const int32_t*, void*, hipStream_t) {
  return reached();
}

}  // namespace mxq
