// q8_1.h -- the Q8_1 block quantizer, shared by the stand-alone quantize
// kernel and the kernels that quantize activations in LDS, so that every
// path produces the same bytes.
//
// Per 32-element block: amax, d32 = amax / 127 (correctly rounded binary32
// division), q = round-half-away(x / d32) clamped to +-127, d = binary16(d32),
// s = binary16(d32 * sum q); an all-zero block gives q = 0, d = s = 0.
// A block is one aligned quad of lanes, 8 consecutive elements per lane; the
// block's amax and code sum are reduced with quad DPP moves, so all four
// lanes of a quad must call quantize_q8_1_group together.
#pragma once

#include "device.h"

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

// One lane's 8 elements (v0, v1) -> 8 codes packed in lo, hi; the block's
// binary16 d and s bits (the same in all four lanes of the quad).
__device__ __forceinline__ void quantize_q8_1_group(const float4_t &v0, const float4_t &v1,
                                                    uint32_t &lo, uint32_t &hi, uint16_t &dbits,
                                                    uint16_t &sbits) {
  float amax = fmaxf(fmaxf(fmaxf(fabsf(v0[0]), fabsf(v0[1])), fmaxf(fabsf(v0[2]), fabsf(v0[3]))),
                     fmaxf(fmaxf(fabsf(v1[0]), fabsf(v1[1])), fmaxf(fabsf(v1[2]), fabsf(v1[3]))));
  amax = quad_max(amax);
  lo = 0;
  hi = 0;
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
  dbits = amax != 0.0f ? f32_to_f16_bits(d32) : (uint16_t)0;
  sbits = amax != 0.0f ? f32_to_f16_bits(d32 * (float)sq) : (uint16_t)0;
}

}  // namespace skinny
