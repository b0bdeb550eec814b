// launch.h -- internal launchers, one per entry point.  Each returns 0 or
// the hipError_t of the launch; arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

namespace skinny {

hipError_t launch_quantize_q8_1(const float *x, int M, int K, int8_t *qs,
                                uint16_t *d, uint16_t *s, hipStream_t stream);

hipError_t launch_mmvq_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                            const int8_t *a_qs, const uint16_t *a_d,
                            const uint16_t *a_s, int M, float *y, hipStream_t stream);

hipError_t launch_mmvq_q4_0_f32act(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                                   const float *x, int M, float *y, hipStream_t stream);

hipError_t launch_mmvq_q4_k(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                            const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s, int M,
                            float *y, hipStream_t stream);

// Q4_K on the Q4_0 matrix-core kernel (3 <= M <= 8), defined with it.
hipError_t launch_mmvq_q4_k_mfma(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                 const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                 int M, float *y, hipStream_t stream);

// IQ4_XS on the Q4_0 matrix-core kernel (3 <= M <= 8, K % 256 == 0).
hipError_t launch_mmvq_iq4_xs_mfma(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                   const int8_t *a_qs, const uint16_t *a_d, int M, float *y,
                                   hipStream_t stream);

hipError_t launch_mmvq_q6_k(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                            const uint16_t *w_d, int N, int K, const int8_t *a_qs,
                            const uint16_t *a_d, int M, float *y, hipStream_t stream);

hipError_t launch_mmvq_iq4_xs(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                              const int8_t *a_qs, const uint16_t *a_d, int M, float *y,
                              hipStream_t stream);

hipError_t launch_gemv_nvfp4(const uint8_t *w_codes, const uint8_t *w_scales,
                             float g, int N, int K, const uint16_t *x, int M,
                             uint16_t *y, hipStream_t stream);

// Pre-permuted Q4_0, Q4_K and IQ4_XS (mmvq_q4_0_packed.hip).
hipError_t launch_prepack_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                               uint8_t *w_packed, hipStream_t stream);

hipError_t launch_mmvq_q4_0_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                                   const uint16_t *a_d, const uint16_t *a_s, int M, float *y,
                                   hipStream_t stream);

hipError_t launch_prepack_q4_k(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                               uint8_t *w_packed, hipStream_t stream);

hipError_t launch_mmvq_q4_k_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                                   const uint16_t *a_d, const uint16_t *a_s, int M, float *y,
                                   hipStream_t stream);

hipError_t launch_prepack_iq4_xs(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                 uint8_t *w_packed, hipStream_t stream);

hipError_t launch_mmvq_iq4_xs_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                                     const uint16_t *a_d, int M, float *y, hipStream_t stream);

// Pre-permuted Q6_K (mmvq_q6_k_packed.hip).
hipError_t launch_prepack_q6_k(const uint8_t *ql, const uint8_t *qh, const int8_t *sc,
                               const uint16_t *d, int N, int K, uint8_t *w_packed,
                               hipStream_t stream);

hipError_t launch_mmvq_q6_k_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                                   const uint16_t *a_d, int M, float *y, hipStream_t stream);

// Pre-permuted NVFP4 (gemv_nvfp4_packed.hip).
hipError_t launch_prepack_nvfp4(const uint8_t *codes, const uint8_t *scales, int N, int K,
                                uint8_t *w_packed, hipStream_t stream);

hipError_t launch_gemv_nvfp4_packed(const uint8_t *w_packed, float g, int N, int K,
                                    const uint16_t *x, int M, uint16_t *y, hipStream_t stream);

// Pre-permuted FP8 (gemv_fp8_packed.hip).
hipError_t launch_prepack_fp8(const uint8_t *w, int N, int K, uint8_t *w_packed,
                              hipStream_t stream);

hipError_t launch_gemv_fp8_packed(const uint8_t *w_packed, const float *cs, int N, int K,
                                  const uint16_t *x, int M, uint16_t *y, hipStream_t stream);

hipError_t launch_gemv_fp8(const uint8_t *w, const float *cs, int N, int K,
                           const uint16_t *x, int M, uint16_t *y, hipStream_t stream);

// Let a kernel use more than 64 KB of LDS per workgroup (gfx950 has 160 KB
// per compute unit); a no-op at or below 64 KB.  The limit is raised once
// per (device, kernel) and never lowered, so calls of any size, from any
// thread, on any device, see a limit at least as large as they asked for.
inline hipError_t allow_lds(const void *kernel, int bytes) {
  if (bytes <= 65536) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, int> granted;
  std::lock_guard<std::mutex> lock(mu);
  int &have = granted[{dev, kernel}];
  if (bytes <= have) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

}  // namespace skinny
