// iq4.h -- decode of IQ4_XS table indices into int8 values, shared by the
// IQ4_XS vector kernels and the matrix-core kernel.
//
// IQ4_XS (named by "Machine Learning on NVIDIA CMP", "llama.cpp results",
// model table; the format is the published GGUF one): each weight is a 4-bit
// index into a fixed 16-entry table of signed integers (the IQ4_NL table
// below), scaled per sub-block of 32.  A word of four indices (one per byte)
// becomes four int8 table values with three byte permutes: the low three
// bits of each index select among entries 0-7 and, separately, among
// entries 8-15 (the table lives in four registers, eight entries per
// permute); the fourth bit then picks, per byte, which of the two to keep.
#pragma once

#include "device.h"

namespace skinny {

constexpr int8_t kIq4Table[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                  1,    13,   25,  38,  53,  69,  89,  113};

// Entries 4i..4i+3 of the table as one little-endian word of int8 bytes.
constexpr uint32_t iq4_word(int i) {
  return (uint32_t)(uint8_t)kIq4Table[4 * i] | ((uint32_t)(uint8_t)kIq4Table[4 * i + 1] << 8) |
         ((uint32_t)(uint8_t)kIq4Table[4 * i + 2] << 16) |
         ((uint32_t)(uint8_t)kIq4Table[4 * i + 3] << 24);
}

// The table words and the two byte masks the decode uses, held in vector
// registers for the kernel's lifetime (the empty asm hides their values from
// the compiler): as register operands they let each selector be formed with
// one and-or, where a literal mask would take a separate and and or.
struct Iq4Regs {
  uint32_t m7, m4, t0, t1, t2, t3;
  __device__ __forceinline__ Iq4Regs()
      : m7(0x07070707u), m4(0x04040404u), t0(iq4_word(0)), t1(iq4_word(1)), t2(iq4_word(2)),
        t3(iq4_word(3)) {
    asm volatile("" : "+v"(m7), "+v"(m4), "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t3));
  }
};

// low3: the low three bits of four indices, one per byte; sel: each byte k
// set to k + 4 * (the index's fourth bit).  A byte permute selector s < 4
// takes byte s of its second operand, 4 <= s < 8 byte s - 4 of its first.
__device__ __forceinline__ uint32_t iq4_lookup(uint32_t low3, uint32_t sel, const Iq4Regs &k) {
  const uint32_t e0 = __builtin_amdgcn_perm(k.t1, k.t0, low3);   // entries 0-7
  const uint32_t e8 = __builtin_amdgcn_perm(k.t3, k.t2, low3);   // entries 8-15
  return __builtin_amdgcn_perm(e8, e0, sel);
}

// One word of index bytes -> the int8 table values of its low nibbles and
// of its high nibbles.
__device__ __forceinline__ void iq4_decode(uint32_t w, uint32_t &lo, uint32_t &hi,
                                           const Iq4Regs &k) {
  lo = iq4_lookup(w & k.m7, ((w >> 1) & k.m4) | 0x03020100u, k);
  hi = iq4_lookup((w >> 4) & k.m7, ((w >> 5) & k.m4) | 0x03020100u, k);
}

// d * (ls_j - 32) of sub-block j from the two words of an 8-byte super-block
// header (x: binary16 d | H << 16, y: L; ls_j = ((L >> 4j) & 15) |
// (((H >> 2j) & 3) << 4)).
__device__ __forceinline__ float iq4_scale(uint2_t h, int j) {
  const int ls = (int)((h.y >> (4 * j)) & 15u) | (int)(((h.x >> (16 + 2 * j)) & 3u) << 4);
  return f16_bits_to_f32((uint16_t)(h.x & 0xFFFFu)) * (float)(ls - 32);
}

}  // namespace skinny
