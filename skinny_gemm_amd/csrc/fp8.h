// fp8.h -- the FP8 E4M3 operand decode shared by the matrix-core kernels
// that stream canonical and pre-permuted FP8 weights.
#pragma once

#include "device.h"

namespace skinny {

// A lane's 32 weight bytes (two 16-byte pieces, elements 0..15 and 16..31
// of its K slot group) -> the four binary16 A operands of one 128-K step,
// operand u taking elements 8u .. 8u + 7; exact, as every E4M3 value is a
// binary16 value.
__device__ __forceinline__ void fp8_decode(const uint4_t (&wq)[2], half8_t (&a)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t w0 = wq[u >> 1][2 * (u & 1)];
    const uint32_t w1 = wq[u >> 1][2 * (u & 1) + 1];
    const half2_t h0 = e4m3x2_to_h2<false>(w0);
    const half2_t h1 = e4m3x2_to_h2<true>(w0);
    const half2_t h2 = e4m3x2_to_h2<false>(w1);
    const half2_t h3 = e4m3x2_to_h2<true>(w1);
    a[u] = half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
  }
}

}  // namespace skinny
