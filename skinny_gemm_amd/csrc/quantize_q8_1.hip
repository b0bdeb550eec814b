// quantize_q8_1.hip -- activation rows -> Q8_1 (int8 codes, binary16 scale
// and binary16 scaled code sum per 32-element block).
//
// The quantized mat x vec kernel of "Machine Learning on NVIDIA CMP"
// ("TL;DR", "The DP2A patch") consumes int8 activation codes; the pages do
// not define the activation format.  Per block: amax, d32 = amax / 127
// (correctly rounded binary32 division), q = round-half-away(x / d32)
// clamped to +-127, d = binary16(d32), s = binary16(d32 * sum q).
//
// Mapping: one lane per 8 consecutive elements, so a 32-element block is
// one aligned quad of lanes; the block's amax and code sum are reduced
// with quad DPP moves.  Reads 32 B and writes 8 B per lane (coalesced);
// lane 0 of each quad writes d and s.  The input is treated as one flat
// array of M*K elements, which is valid because K % 32 == 0.
#include "device.h"
#include "launch.h"

namespace skinny {

__device__ __forceinline__ float quad_max(float v) {
  int x = __builtin_bit_cast(int, v);
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false)));
  x = __builtin_bit_cast(int, v);
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false)));
  return v;
}

__device__ __forceinline__ int quad_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  return v;
}

__device__ __forceinline__ int q8_code(float x, float d32) {
  float v = roundf(x / d32);
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return (int)v;
}

__global__ __launch_bounds__(256) void quantize_q8_1_kernel(
    const float *__restrict__ x, int64_t groups, int8_t *__restrict__ qs,
    uint16_t *__restrict__ d, uint16_t *__restrict__ s) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;   // group of 8 elements
  const bool active = t < groups;                                // quads are all-or-nothing
  float4_t v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    const float4_t *p = reinterpret_cast<const float4_t *>(x + t * 8);
    v0 = p[0];
    v1 = p[1];
  }
  float amax = fmaxf(fmaxf(fmaxf(fabsf(v0[0]), fabsf(v0[1])), fmaxf(fabsf(v0[2]), fabsf(v0[3]))),
                     fmaxf(fmaxf(fabsf(v1[0]), fabsf(v1[1])), fmaxf(fabsf(v1[2]), fabsf(v1[3]))));
  amax = quad_max(amax);

  uint32_t lo = 0, hi = 0;
  int sq = 0;
  float d32 = 0.0f;
  if (amax != 0.0f) {
    d32 = amax / 127.0f;
    int q[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = q8_code(v0[i], d32);
      q[4 + i] = q8_code(v1[i], d32);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= (uint32_t)(q[i] & 0xFF) << (8 * i);
      hi |= (uint32_t)(q[4 + i] & 0xFF) << (8 * i);
      sq += q[i] + q[4 + i];
    }
  }
  sq = quad_sum(sq);
  if (active) {
    uint32_t *out = reinterpret_cast<uint32_t *>(qs + t * 8);
    out[0] = lo;
    out[1] = hi;
    if ((threadIdx.x & 3) == 0) {
      const int64_t b = t >> 2;
      const float scaled = d32 * (float)sq;
      d[b] = amax != 0.0f ? f32_to_f16_bits(d32) : (uint16_t)0;
      s[b] = amax != 0.0f ? f32_to_f16_bits(scaled) : (uint16_t)0;
    }
  }
}

hipError_t launch_quantize_q8_1(const float *x, int M, int K, int8_t *qs,
                                uint16_t *d, uint16_t *s, hipStream_t stream) {
  const int64_t groups = (int64_t)M * K / 8;
  const int64_t blocks = (groups + 255) / 256;
  hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     x, groups, qs, d, s);
  return hipGetLastError();
}

}  // namespace skinny
