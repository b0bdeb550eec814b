// device.h -- small device-side helpers shared by the gfx950 kernels:
// vector types, binary16 and FP8 conversions through the hardware
// converters, and the wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skinny {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));
typedef int32_t int4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// float32 -> binary16 bits, round to nearest even (v_cvt_f16_f32 under the
// default rounding mode; overflow gives infinity).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// 128-bit global load through the vector memory path.
template <typename T>
__device__ __forceinline__ uint4_t load16(const T *p) {
  return *reinterpret_cast<const uint4_t *>(p);
}

// 128-bit non-temporal load, for the weight stream: every weight byte is
// read exactly once per call, so it should not displace reusable lines.
template <typename T>
__device__ __forceinline__ uint4_t load16_nt(const T *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint4_t *>(p));
}

template <typename T>
__device__ __forceinline__ uint2_t load8_nt(const T *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint2_t *>(p));
}

template <typename T>
__device__ __forceinline__ uint2_t load8(const T *p) {
  return *reinterpret_cast<const uint2_t *>(p);
}

__device__ __forceinline__ uint16_t load_u16_nt(const uint16_t *p) {
  return __builtin_nontemporal_load(p);
}

// Value held by lane (lane ^ D), D in {1, 2, 4, 8}.
template <int D>
__device__ __forceinline__ float xor_lane(float v) {
  static_assert(D == 1 || D == 2 || D == 4 || D == 8, "distance");
  int x = __builtin_bit_cast(int, v);
  if constexpr (D == 1) {
    x = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (D == 2) {
    x = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else {
    x = __builtin_amdgcn_ds_swizzle(x, 0x1F | (D << 10));           // xor within 32 lanes
  }
  return __builtin_bit_cast(float, x);
}

// One butterfly step at lane distance D: lanes whose D-bit is clear end up
// holding a(lane) + a(lane ^ D), the others b(lane) + b(lane ^ D).
template <int D>
__device__ __forceinline__ float bfly(float a, float b, int lane) {
  if constexpr (D == 32) {
    // v_permlane32_swap: lanes 32..63 of the first operand trade places with
    // lanes 0..31 of the second.
    auto r = __builtin_amdgcn_permlane32_swap(as_u32(a), as_u32(b), false, false);
    return as_f32(r[0]) + as_f32(r[1]);
  } else if constexpr (D == 16) {
    // v_permlane16_swap: odd 16-lane rows of the first operand trade places
    // with even rows of the second.
    auto r = __builtin_amdgcn_permlane16_swap(as_u32(a), as_u32(b), false, false);
    return as_f32(r[0]) + as_f32(r[1]);
  } else {
    const bool hi = (lane & D) != 0;
    const float keep = hi ? b : a;
    const float send = hi ? a : b;
    return keep + xor_lane<D>(send);
  }
}

// Sum of v over all lanes whose bits below D*2 differ (D = 32, 16, ..., 1).
template <int D>
__device__ __forceinline__ float allsum_from(float v) {
  if constexpr (D == 0) {
    return v;
  } else {
    float s;
    if constexpr (D == 32) {
      auto r = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
      s = as_f32(r[0]) + as_f32(r[1]);
    } else if constexpr (D == 16) {
      auto r = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
      s = as_f32(r[0]) + as_f32(r[1]);
    } else {
      s = v + xor_lane<D>(v);
    }
    return allsum_from<D / 2>(s);
  }
}

template <int V>
struct Log2 { static constexpr int value = 1 + Log2<V / 2>::value; };
template <>
struct Log2<1> { static constexpr int value = 0; };

template <int V, int D>
__device__ __forceinline__ void bfly_stages(float (&v)[V], int lane) {
  if constexpr (V > 1 && D >= 1) {
    constexpr int H = V / 2;
#pragma unroll
    for (int i = 0; i < H; ++i)
      v[i] = bfly<D>(v[i], v[i + H], lane);
    float (&w)[H] = *reinterpret_cast<float (*)[H]>(&v[0]);
    bfly_stages<H, D / 2>(w, lane);
  }
}

// Transposing wave reduction: V (a power of two <= 64) partial sums per
// lane in, one total per lane out.  Lane l returns the wave-wide total of
// value index (l >> (6 - log2 V)); lanes that share that index hold the
// same total.  Costs about 2-3 VALU ops per value instead of 12 per value
// for V independent reductions.
template <int V>
__device__ __forceinline__ float wave_reduce_transpose(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
  constexpr int P = Log2<V>::value;
  bfly_stages<V, 32>(v, lane);
  return allsum_from<(32 >> P)>(v[0]);
}

// Two OCP E4M3 bytes (HI = 0: bytes 0,1; HI = 1: bytes 2,3 of w) ->
// binary16 pair, exact (every E4M3 value is a binary16 value).
template <bool HI>
__device__ __forceinline__ half2_t e4m3x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Two E2M1 codes from byte `sel` of w (low nibble -> .x) -> binary16 pair.
template <int SEL>
__device__ __forceinline__ half2_t e2m1x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// One OCP E4M3 byte (byte `SEL` of w) -> float32, exact.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

__device__ __forceinline__ int32_t dot4_i8(uint32_t a, uint32_t b, int32_t c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// 16x16 matrix-core products.  Operand layout (wave64): lane l supplies
// row (l % 16) of A and column (l % 16) of B for k-slot (l / 16); both
// operands use the same slot and element positions, so any consistent
// assignment of K indices to (slot, position) gives
//   C[i][j] = sum over lanes l = i + 16g, j + 16g and positions p of
//             A_l[p] * B_l[p].
// Lane l receives C[4 * (l / 16) + r][l % 16] in element r of the result.
__device__ __forceinline__ float4_t mfma_16x16x32_f16(const half8_t &a, const half8_t &b,
                                                      const float4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int4_t mfma_16x16x64_i8(const int4_t &a, const int4_t &b,
                                                   const int4_t &c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// x + (value of x in lane l ^ 32): one v_permlane32_swap and one add.
__device__ __forceinline__ float add_swap32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}

// Compiler-only fence: memory operations are not moved across it, so the
// hardware sees loads in program order (what vmcnt counts).
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Fence plus scheduling barrier: no instruction (arithmetic included) is
// moved across it, so all loads above it are in flight before any of their
// results is waited for.
__device__ __forceinline__ void issue_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier with no implied memory wait (in-flight loads stay in
// flight); LDS accesses are not moved across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Binary16 activation rows staged in LDS for the vector kernels: rows [M][K]
// as 16-byte pieces, P pieces per lane chunk; piece q of chunk c sits at
// slot P c + (q ^ ((c / (16 / P)) % P)) of its row, so the 16 lanes of one
// LDS read pass (consecutive chunks, same q) hit 16 distinct 16-byte bank
// groups, and 16 consecutive pieces (one store pass) stay distinct too.
template <int P>
__device__ __forceinline__ int act_slot(int c, int q) {
  return P * c + (q ^ ((c / (16 / P)) % P));
}

// First batch of the staging: A pieces per thread (of tot = M K / 8, piece
// p = thread + NT a), issued before the weight loads so that waiting for
// them does not wait for the weights; pieces past the end repeat the last.
template <int A, int NT>
__device__ __forceinline__ void act_issue(const uint16_t *x, int tot, uint4_t (&av)[A]) {
#pragma unroll
  for (int a = 0; a < A; ++a)
    av[a] = load16(x + 8 * (size_t)min((int)threadIdx.x + NT * a, tot - 1));
}

// Stores the first batch into LDS (straight-line, so its wait covers only
// the activation loads), then loads and stores any remaining pieces in
// batches of A; np = K / 8 pieces per row.
template <int P, int A, int NT>
__device__ __forceinline__ void act_store_batch(int p0, int tot, int np, uint4_t *xs,
                                                const uint4_t (&av)[A]) {
#pragma unroll
  for (int a = 0; a < A; ++a) {
    const int p = p0 + (int)threadIdx.x + NT * a;
    if (p < tot) {
      const int m = p / np, pr = p - m * np;
      xs[m * np + act_slot<P>(pr / P, pr % P)] = av[a];
    }
  }
}

template <int P, int A, int NT>
__device__ __forceinline__ void act_stage(const uint16_t *x, int tot, int np, uint4_t *xs,
                                          uint4_t (&av)[A]) {
  act_store_batch<P, A, NT>(0, tot, np, xs, av);
  for (int p0 = NT * A; p0 < tot; p0 += NT * A) {
#pragma unroll
    for (int a = 0; a < A; ++a)
      av[a] = load16(x + 8 * (size_t)min(p0 + (int)threadIdx.x + NT * a, tot - 1));
    act_store_batch<P, A, NT>(p0, tot, np, xs, av);
  }
}

__device__ __forceinline__ half2_t h2_bcast(float f) {
  const _Float16 h = (_Float16)f;
  return half2_t{h, h};
}

}  // namespace skinny
