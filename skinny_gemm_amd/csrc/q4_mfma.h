// q4_mfma.h -- the Q4_0 / Q4_K / IQ4_XS matrix-core step shared by the
// kernels that stream canonical and pre-permuted weights: exact int32 block
// sums from v_mfma_i32_16x16x64_i8 and the float32 block epilogues.
#pragma once

#include "device.h"
#include "iq4.h"

namespace skinny {

// The exact int32 block sums of one 64-K step: the lane's 8 code bytes split
// into 16 codes (low nibbles, then high nibbles) against the activation
// operand.
__device__ __forceinline__ int4_t q4_mfma_isum(const uint2_t &wq, const int4_t &aop) {
  int4_t bop;
  bop[0] = (int)(wq.x & 0x0F0F0F0Fu);
  bop[1] = (int)(wq.y & 0x0F0F0F0Fu);
  bop[2] = (int)((wq.x >> 4) & 0x0F0F0F0Fu);
  bop[3] = (int)((wq.y >> 4) & 0x0F0F0F0Fu);
  const int4_t zero = {0, 0, 0, 0};
  return mfma_16x16x64_i8(aop, bop, zero);
}

// IQ4_XS: the same 16 indices through the table, as signed int8 values.
__device__ __forceinline__ int4_t iq4_mfma_isum(const uint2_t &wq, const int4_t &aop,
                                                const Iq4Regs &k) {
  uint32_t xl, xh, yl, yh;
  iq4_decode(wq.x, xl, xh, k);
  iq4_decode(wq.y, yl, yh, k);
  const int4_t bop = {(int)xl, (int)yl, (int)xh, (int)yh};
  const int4_t zero = {0, 0, 0, 0};
  return mfma_16x16x64_i8(aop, bop, zero);
}

// Float32 block epilogue of one step: acc += d4 * (d8 * isum - 8 s8) for the
// lane's four activation rows, (d8, 8 s8) pairs in sa (rows 0, 1) and sb
// (rows 2, 3).
__device__ __forceinline__ void q4_mfma_epilogue(const int4_t &isum, float d4,
                                                 const float4_t &sa, const float4_t &sb,
                                                 float4_t &acc) {
  acc[0] = fmaf(d4, fmaf(sa[0], (float)isum[0], -sa[1]), acc[0]);
  acc[1] = fmaf(d4, fmaf(sa[2], (float)isum[1], -sa[3]), acc[1]);
  acc[2] = fmaf(d4, fmaf(sb[0], (float)isum[2], -sb[1]), acc[2]);
  acc[3] = fmaf(d4, fmaf(sb[2], (float)isum[3], -sb[3]), acc[3]);
}

// Q4_K epilogue of one step (KQ): the lane's sub-block scale and min come
// from its super-block header, acc += d sc d8 isum - dmin m s8, with the
// staged activation pairs (d8, 8 s8) and dmm8 = dmin m / 8 (exact).
__device__ __forceinline__ void q4k_mfma_epilogue(const int4_t &isum, float dsc, float dmm8,
                                                  const float4_t &sa, const float4_t &sb,
                                                  float4_t &acc) {
  acc[0] = fmaf(dsc, sa[0] * (float)isum[0], fmaf(-dmm8, sa[1], acc[0]));
  acc[1] = fmaf(dsc, sa[2] * (float)isum[1], fmaf(-dmm8, sa[3], acc[1]));
  acc[2] = fmaf(dsc, sb[0] * (float)isum[2], fmaf(-dmm8, sb[1], acc[2]));
  acc[3] = fmaf(dsc, sb[2] * (float)isum[3], fmaf(-dmm8, sb[3], acc[3]));
}

// IQ4_XS epilogue of one step: acc += d (ls - 32) d8 isum, dls = d (ls - 32)
// of the lane's sub-block (the table values are signed: no sum term).
__device__ __forceinline__ void iq4_mfma_epilogue(const int4_t &isum, float dls,
                                                  const float4_t &sa, const float4_t &sb,
                                                  float4_t &acc) {
  acc[0] = fmaf(dls, sa[0] * (float)isum[0], acc[0]);
  acc[1] = fmaf(dls, sa[2] * (float)isum[1], acc[1]);
  acc[2] = fmaf(dls, sb[0] * (float)isum[2], acc[2]);
  acc[3] = fmaf(dls, sb[2] * (float)isum[3], acc[3]);
}

}  // namespace skinny
