// launch.h -- internal launchers, one per entry point.  Each returns 0 or
// the hipError_t of the launch; arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skinny {

hipError_t launch_quantize_q8_1(const float *x, int M, int K, int8_t *qs,
                                uint16_t *d, uint16_t *s, hipStream_t stream);

hipError_t launch_mmvq_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                            const int8_t *a_qs, const uint16_t *a_d,
                            const uint16_t *a_s, int M, float *y, hipStream_t stream);

hipError_t launch_gemv_nvfp4(const uint8_t *w_codes, const uint8_t *w_scales,
                             float g, int N, int K, const uint16_t *x, int M,
                             uint16_t *y, hipStream_t stream);

hipError_t launch_gemv_fp8(const uint8_t *w, const float *cs, int N, int K,
                           const uint16_t *x, int M, uint16_t *y, hipStream_t stream);

}  // namespace skinny
