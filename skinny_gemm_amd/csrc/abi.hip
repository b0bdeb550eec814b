// abi.hip -- the exported C entry points: host-side argument validation,
// then the kernel launch(es) on the caller's stream.  Validation makes no HIP
// call, so it runs (and is tested) on machines without a GPU.  An invalid
// call returns its status code and enqueues nothing; a valid call never
// switches to another kernel.
#include <stdint.h>

#include "launch.h"
#include "skinny_gemm.h"

namespace {

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int shape_status(int N, int K, int kmult) {
  if (K <= 0 || K > SKINNY_MAX_K || (K % kmult) != 0) return SKINNY_ERR_SHAPE;
  if (N < 0 || N > SKINNY_MAX_N) return SKINNY_ERR_SHAPE;
  return SKINNY_OK;
}

inline int gemv_m_status(int M, int max_m) {
  if (M < 0 || M > max_m) return SKINNY_ERR_M;
  return SKINNY_OK;
}

inline int launched(hipError_t e) { return e == hipSuccess ? SKINNY_OK : SKINNY_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char *skinny_status_string(int status) {
  switch (status) {
    case SKINNY_OK: return "ok";
    case SKINNY_ERR_NULL: return "null pointer argument";
    case SKINNY_ERR_SHAPE: return "unsupported shape (K or N out of range, or K not a multiple of the block)";
    case SKINNY_ERR_ALIGN: return "misaligned pointer argument";
    case SKINNY_ERR_M: return "unsupported number of activation rows M";
    case SKINNY_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int quantize_act_q8_1(const float *x, int M, int K, int8_t *qs, uint16_t *d, uint16_t *s,
                      void *stream) {
  if (M < 0 || M > SKINNY_MAX_M_QUANT) return SKINNY_ERR_M;
  if (K <= 0 || K > SKINNY_MAX_K || (K % 32) != 0) return SKINNY_ERR_SHAPE;
  if ((long long)M * K > SKINNY_MAX_MK_QUANT) return SKINNY_ERR_SHAPE;
  if (M == 0) return SKINNY_OK;
  if (!x || !qs || !d || !s) return SKINNY_ERR_NULL;
  if (!aligned(x, 16) || !aligned(qs, 16) || !aligned(d, 2) || !aligned(s, 2))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_quantize_q8_1(x, M, K, qs, d, s, (hipStream_t)stream));
}

int mmvq_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K, const int8_t *a_qs,
              const uint16_t *a_d, const uint16_t *a_s, int M, float *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_GEMV);
  if (st) return st;
  if ((st = shape_status(N, K, 32))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_qs || !w_d || !a_qs || !a_d || !a_s || !y) return SKINNY_ERR_NULL;
  // the scale arrays too are read with 128-bit loads on some paths
  if (!aligned(w_qs, 16) || !aligned(a_qs, 16) || !aligned(w_d, 16) || !aligned(a_d, 16) ||
      !aligned(a_s, 16) || !aligned(y, 4))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_mmvq_q4_0(w_qs, w_d, N, K, a_qs, a_d, a_s, M, y,
                                           (hipStream_t)stream));
}

int mmvq_q4_0_f32act(const uint8_t *w_qs, const uint16_t *w_d, int N, int K, const float *x,
                     int M, float *y, void *stream) {
  if (M < 0 || M > SKINNY_MAX_M_F32ACT) return SKINNY_ERR_M;
  int st = shape_status(N, K, 32);
  if (st) return st;
  if (K > SKINNY_MAX_K_F32ACT) return SKINNY_ERR_SHAPE;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_qs || !w_d || !x || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_qs, 16) || !aligned(w_d, 2) || !aligned(x, 16) || !aligned(y, 4))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_mmvq_q4_0_f32act(w_qs, w_d, N, K, x, M, y, (hipStream_t)stream));
}

int mmvq_q4_k(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, const int8_t *a_qs,
              const uint16_t *a_d, const uint16_t *a_s, int M, float *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_GEMV);
  if (st) return st;
  if ((st = shape_status(N, K, 256))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_qs || !w_hdr || !a_qs || !a_d || !a_s || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_qs, 16) || !aligned(w_hdr, 16) || !aligned(a_qs, 16) || !aligned(a_d, 16) ||
      !aligned(a_s, 16) || !aligned(y, 4))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_mmvq_q4_k(w_qs, w_hdr, N, K, a_qs, a_d, a_s, M, y,
                                           (hipStream_t)stream));
}

int mmvq_q6_k(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc, const uint16_t *w_d,
              int N, int K, const int8_t *a_qs, const uint16_t *a_d, int M, float *y,
              void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_GEMV);
  if (st) return st;
  if ((st = shape_status(N, K, 256))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_ql || !w_qh || !w_sc || !w_d || !a_qs || !a_d || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_ql, 16) || !aligned(w_qh, 8) || !aligned(w_sc, 2) || !aligned(w_d, 2) ||
      !aligned(a_qs, 16) || !aligned(a_d, 16) || !aligned(y, 4))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_mmvq_q6_k(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, M, y,
                                           (hipStream_t)stream));
}

int mmvq_iq4_xs(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, const int8_t *a_qs,
                const uint16_t *a_d, int M, float *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_GEMV);
  if (st) return st;
  if ((st = shape_status(N, K, 256))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_qs || !w_hdr || !a_qs || !a_d || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_qs, 16) || !aligned(w_hdr, 16) || !aligned(a_qs, 16) || !aligned(a_d, 16) ||
      !aligned(y, 4))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_mmvq_iq4_xs(w_qs, w_hdr, N, K, a_qs, a_d, M, y,
                                             (hipStream_t)stream));
}

int gemv_nvfp4_w4a16(const uint8_t *w_codes, const uint8_t *w_scales, float global_scale,
                     int N, int K, const uint16_t *x, int M, uint16_t *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_F16ACT);
  if (st) return st;
  if ((st = shape_status(N, K, 32))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_codes || !w_scales || !x || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_codes, 16) || !aligned(w_scales, 16) || !aligned(x, 16) || !aligned(y, 2))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_gemv_nvfp4(w_codes, w_scales, global_scale, N, K, x, M, y,
                                            (hipStream_t)stream));
}

int prepack_q4_0_size(int N, int K, size_t *bytes) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (!bytes) return SKINNY_ERR_NULL;
  const size_t U = ((size_t)N + 15) / 16, P = (size_t)K / 128, V = ((size_t)K + 511) / 512;
  *bytes = 1024 * U * P + 512 * U * V;
  return SKINNY_OK;
}

int prepack_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K, uint8_t *w_packed,
                 void *stream) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (N == 0) return SKINNY_OK;
  if (!w_qs || !w_d || !w_packed) return SKINNY_ERR_NULL;
  if (!aligned(w_qs, 16) || !aligned(w_d, 2) || !aligned(w_packed, 16)) return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_prepack_q4_0(w_qs, w_d, N, K, w_packed, (hipStream_t)stream));
}

int mmvq_q4_0_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                     const uint16_t *a_d, const uint16_t *a_s, int M, float *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_GEMV);
  if (st) return st;
  if ((st = shape_status(N, K, 256))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_packed || !a_qs || !a_d || !a_s || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_packed, 16) || !aligned(a_qs, 16) || !aligned(a_d, 16) || !aligned(a_s, 16) ||
      !aligned(y, 4))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_mmvq_q4_0_packed(w_packed, N, K, a_qs, a_d, a_s, M, y,
                                                  (hipStream_t)stream));
}

int prepack_q4_k_size(int N, int K, size_t *bytes) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (!bytes) return SKINNY_ERR_NULL;
  const size_t U = ((size_t)N + 15) / 16;
  *bytes = 1024 * U * ((size_t)K / 128) + U * (size_t)K;
  return SKINNY_OK;
}

int prepack_q4_k(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, uint8_t *w_packed,
                 void *stream) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (N == 0) return SKINNY_OK;
  if (!w_qs || !w_hdr || !w_packed) return SKINNY_ERR_NULL;
  if (!aligned(w_qs, 16) || !aligned(w_hdr, 16) || !aligned(w_packed, 16))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_prepack_q4_k(w_qs, w_hdr, N, K, w_packed, (hipStream_t)stream));
}

int prepack_iq4_xs_size(int N, int K, size_t *bytes) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (!bytes) return SKINNY_ERR_NULL;
  const size_t U = ((size_t)N + 15) / 16;
  *bytes = 1024 * U * ((size_t)K / 128) + U * (size_t)K / 2;
  return SKINNY_OK;
}

int prepack_iq4_xs(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, uint8_t *w_packed,
                   void *stream) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (N == 0) return SKINNY_OK;
  if (!w_qs || !w_hdr || !w_packed) return SKINNY_ERR_NULL;
  if (!aligned(w_qs, 16) || !aligned(w_hdr, 16) || !aligned(w_packed, 16))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_prepack_iq4_xs(w_qs, w_hdr, N, K, w_packed,
                                                (hipStream_t)stream));
}

int mmvq_iq4_xs_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                       const uint16_t *a_d, int M, float *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_GEMV);
  if (st) return st;
  if ((st = shape_status(N, K, 256))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_packed || !a_qs || !a_d || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_packed, 16) || !aligned(a_qs, 16) || !aligned(a_d, 16) || !aligned(y, 4))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_mmvq_iq4_xs_packed(w_packed, N, K, a_qs, a_d, M, y,
                                                    (hipStream_t)stream));
}

int mmvq_q4_k_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                     const uint16_t *a_d, const uint16_t *a_s, int M, float *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_GEMV);
  if (st) return st;
  if ((st = shape_status(N, K, 256))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_packed || !a_qs || !a_d || !a_s || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_packed, 16) || !aligned(a_qs, 16) || !aligned(a_d, 16) || !aligned(a_s, 16) ||
      !aligned(y, 4))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_mmvq_q4_k_packed(w_packed, N, K, a_qs, a_d, a_s, M, y,
                                                  (hipStream_t)stream));
}

int prepack_q6_k_size(int N, int K, size_t *bytes) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (!bytes) return SKINNY_ERR_NULL;
  const size_t U = ((size_t)N + 15) / 16;
  *bytes = 1024 * U * ((size_t)K / 128) + 1312 * U * ((size_t)K / 256);
  return SKINNY_OK;
}

int prepack_q6_k(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                 const uint16_t *w_d, int N, int K, uint8_t *w_packed, void *stream) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (N == 0) return SKINNY_OK;
  if (!w_ql || !w_qh || !w_sc || !w_d || !w_packed) return SKINNY_ERR_NULL;
  if (!aligned(w_ql, 16) || !aligned(w_qh, 8) || !aligned(w_sc, 2) || !aligned(w_d, 2) ||
      !aligned(w_packed, 16))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_prepack_q6_k(w_ql, w_qh, w_sc, w_d, N, K, w_packed,
                                              (hipStream_t)stream));
}

int mmvq_q6_k_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                     const uint16_t *a_d, int M, float *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_GEMV);
  if (st) return st;
  if ((st = shape_status(N, K, 256))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_packed || !a_qs || !a_d || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_packed, 16) || !aligned(a_qs, 16) || !aligned(a_d, 16) || !aligned(y, 4))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_mmvq_q6_k_packed(w_packed, N, K, a_qs, a_d, M, y,
                                                  (hipStream_t)stream));
}

int prepack_nvfp4_size(int N, int K, size_t *bytes) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (!bytes) return SKINNY_ERR_NULL;
  const size_t U = ((size_t)N + 15) / 16, S = (size_t)K / 128, V = (S + 7) / 8;
  *bytes = 1024 * U * (S + V);
  return SKINNY_OK;
}

int prepack_nvfp4(const uint8_t *w_codes, const uint8_t *w_scales, int N, int K,
                  uint8_t *w_packed, void *stream) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (N == 0) return SKINNY_OK;
  if (!w_codes || !w_scales || !w_packed) return SKINNY_ERR_NULL;
  if (!aligned(w_codes, 16) || !aligned(w_scales, 2) || !aligned(w_packed, 16))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_prepack_nvfp4(w_codes, w_scales, N, K, w_packed,
                                               (hipStream_t)stream));
}

int gemv_nvfp4_w4a16_packed(const uint8_t *w_packed, float global_scale, int N, int K,
                            const uint16_t *x, int M, uint16_t *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_F16ACT);
  if (st) return st;
  if ((st = shape_status(N, K, 256))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_packed || !x || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_packed, 16) || !aligned(x, 16) || !aligned(y, 2)) return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_gemv_nvfp4_packed(w_packed, global_scale, N, K, x, M, y,
                                                   (hipStream_t)stream));
}

int gemv_fp8_w8a16(const uint8_t *w, const float *channel_scale, int N, int K,
                   const uint16_t *x, int M, uint16_t *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_FP8);
  if (st) return st;
  if ((st = shape_status(N, K, 16))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w || !channel_scale || !x || !y) return SKINNY_ERR_NULL;
  if (!aligned(w, 16) || !aligned(channel_scale, 4) || !aligned(x, 16) || !aligned(y, 2))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_gemv_fp8(w, channel_scale, N, K, x, M, y, (hipStream_t)stream));
}

int prepack_fp8_size(int N, int K, size_t *bytes) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (!bytes) return SKINNY_ERR_NULL;
  *bytes = 16 * (((size_t)N + 15) / 16) * (size_t)K;
  return SKINNY_OK;
}

int prepack_fp8(const uint8_t *w, int N, int K, uint8_t *w_packed, void *stream) {
  const int st = shape_status(N, K, 256);
  if (st) return st;
  if (N == 0) return SKINNY_OK;
  if (!w || !w_packed) return SKINNY_ERR_NULL;
  if (!aligned(w, 16) || !aligned(w_packed, 16)) return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_prepack_fp8(w, N, K, w_packed, (hipStream_t)stream));
}

int gemv_fp8_w8a16_packed(const uint8_t *w_packed, const float *channel_scale, int N, int K,
                          const uint16_t *x, int M, uint16_t *y, void *stream) {
  int st = gemv_m_status(M, SKINNY_MAX_M_FP8);
  if (st) return st;
  if ((st = shape_status(N, K, 256))) return st;
  if (M == 0 || N == 0) return SKINNY_OK;
  if (!w_packed || !channel_scale || !x || !y) return SKINNY_ERR_NULL;
  if (!aligned(w_packed, 16) || !aligned(channel_scale, 4) || !aligned(x, 16) || !aligned(y, 2))
    return SKINNY_ERR_ALIGN;
  return launched(skinny::launch_gemv_fp8_packed(w_packed, channel_scale, N, K, x, M, y,
                                                 (hipStream_t)stream));
}

}  // extern "C"
