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
// array of M*K elements, which is valid because K % 32 == 0.  The block
// arithmetic lives in q8_1.h.
#include "launch.h"
#include "q8_1.h"

namespace skinny {

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
  uint32_t lo, hi;
  uint16_t db, sb;
  quantize_q8_1_group(v0, v1, lo, hi, db, sb);
  if (active) {
    uint32_t *out = reinterpret_cast<uint32_t *>(qs + t * 8);
    out[0] = lo;
    out[1] = hi;
    if ((threadIdx.x & 3) == 0) {
      const int64_t b = t >> 2;
      d[b] = db;
      s[b] = sb;
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
