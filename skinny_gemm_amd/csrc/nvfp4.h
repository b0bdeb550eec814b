// nvfp4.h -- the NVFP4 matrix-core step shared by the kernels that stream
// canonical and pre-permuted NVFP4 weights.
#pragma once

#include "device.h"

namespace skinny {

// One 128-K step of a 16-row tile: decode the lane's 16 code bytes with its
// two group scales into four A operands and accumulate against the four B
// operands xv.
__device__ __forceinline__ void nvfp4_step(const uint4_t &wq, uint32_t sc, const uint4_t (&xv)[4],
                                           float4_t &acc) {
  const half2_t s0 = h2_bcast(e4m3_to_f32<0>(sc));
  const half2_t s1 = h2_bcast(e4m3_to_f32<1>(sc));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const half2_t st = t < 2 ? s0 : s1;
    const half2_t h0 = e2m1x2_to_h2<0>(wq[t]) * st;
    const half2_t h1 = e2m1x2_to_h2<1>(wq[t]) * st;
    const half2_t h2 = e2m1x2_to_h2<2>(wq[t]) * st;
    const half2_t h3 = e2m1x2_to_h2<3>(wq[t]) * st;
    const half8_t a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
    acc = mfma_16x16x32_f16(a, __builtin_bit_cast(half8_t, xv[t]), acc);
  }
}

}  // namespace skinny
