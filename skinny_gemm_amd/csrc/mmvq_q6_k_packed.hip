// mmvq_q6_k_packed.hip -- Q6_K weights permuted once, when they are loaded,
// into the matrix cores' operand order, and the MMVQ that streams them
// (M = 1..8 rows of Q8_1 activations).
//
// "v100-skinny README", "How QPN works": weights rearranged at load time into
// the order in which the matrix instructions consume them.  The arithmetic
// is Q6_K's ("Machine Learning on NVIDIA CMP", "llama.cpp results": K-quant
// models decode through the same int8 dot): 6-bit codes q, weight
// d * sc * (q - 32) with an int8 scale per 16-element sub-block and a
// binary16 d per 256 elements, exact int32 sums of (q - 32) * q8 per
// sub-block, then acc += d sc d8 isum in float32.
//
// Matrix-core mapping (v_mfma_i32_16x16x64_i8, one 64-element step = four
// sub-blocks): K slot g of the step is sub-block g.  B operand: lane
// l = 16 g + j supplies the 16 codes q - 32 of sub-block g of weight row j
// of a 16-row tile.  A operand: block-diagonal in sub-blocks, rows
// a = 4 g' + m: lane (a, g) supplies the 16 Q8_1 codes of activation row m
// for sub-block g when g == a / 4, zeros otherwise.  So lane (j, g) receives
// the exact sums of weight row j, sub-block g and activation rows m = 0..3
// (a second instruction takes rows 4..7), and scales them by its own
// sub-block's d sc and the rows' d8; the four sub-blocks of a row are summed
// across lanes at the end.
//
// Packed layout (K % 256 == 0; U = ceil(N / 16) tiles of 16 rows, P = K / 128,
// Q = K / 256 super-blocks; lane l = 16 g + j, g < 4, j < 16), four planes:
//   L, low 4 bits: U P blocks of 1024 bytes, block (u, p) at byte 1024 (u P + p);
//     bytes 16 l + 8 e + c (e < 2, c < 8) = low(c) | low(8 + c) << 4, where
//     low(x) is the low 4 bits of element x of sub-block g of step 2 p + e
//     of row 16 u + j;
//   H, high 2 bits, from 1024 U P: U Q blocks of 1024 bytes, block (u, q);
//     bytes 16 l + 4 t .. + 3 (t < 4) = the four w_qh bytes that hold the high
//     bits of sub-block g of step 4 q + t (byte t', bits 2 c .. 2 c + 1 =
//     element 4 c + t' of the sub-block);
//   C, scales, from 1024 U (P + Q): U Q blocks of 256 bytes, block (u, q);
//     byte 4 l + t = w_sc of sub-block g of step 4 q + t;
//   D, from 1024 U (P + Q) + 256 U Q: U Q blocks of 32 bytes, block (u, q);
//     bytes 2 j, 2 j + 1 = w_d[16 u + j][q].
//   Rows at or past N are zero.  Size 1024 U P + 1312 U Q bytes: exactly the
//   canonical bytes of 16 U rows.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace skinny {

// Workgroup: WR x KS waves; WR waves own different tiles (T each) and share
// one K slice's activation chunks, KS slices split K.  A chunk is S steps
// (S / 4 super-blocks).  Activations are staged as in the Q4_0 matrix-core
// kernels: MP rows of Q8_1 codes in 1 KB pieces (rows past M repeat row
// M - 1) and the scales d8 as floats (no scaled sums: the -32 is in the
// codes), read back as the block-diagonal A operand; off-diagonal lanes read
// a zero area.
namespace q6p {
template <int T, int WR, int KS, int S, int MP>
struct Cfg {
  static constexpr int kWaves = WR * KS;
  static constexpr int kMH = MP > 4 ? 2 : 1;        // instructions per step (4 rows each)
  static constexpr int kRpa = 16 / S;               // activation rows per 1 KB piece
  static constexpr int kAi = MP >= kRpa ? MP / kRpa : 1;
  static constexpr int kAp = kAi + 1;               // ... plus one scale piece
  static constexpr int kApw = (kAp + WR - 1) / WR;  // activation loads per wave
  static constexpr int kNd = S * MP / 4;            // lanes loading d8
  static constexpr int kNab = WR > 1 ? 2 : 1;
  static constexpr int kAsOff = kAi * 1024;         // float d8 [2S][8][2] (slot 1 unused)
  static constexpr int kAst = kAsOff + 2 * S * 8 * 8;
  static constexpr int kZeroOff = KS * kNab * kAst;   // 1 KB of zeros
  static constexpr int kRed = KS > 1 ? kWaves * T * kMH * kWave * 16 : 0;
  static constexpr int kLds = kZeroOff + 1024 > kRed ? kZeroOff + 1024 : kRed;
  static_assert(S == 4 || S == 8, "chunk steps");
  static_assert(MP == 1 || MP == 2 || MP == 4 || MP == 8, "padded activation rows");
  static_assert(kNd <= 64, "one scale load per chunk");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};
}  // namespace q6p

template <int T, int S>
struct Q6pWeights {
  uint4_t l[T][S / 2];      // low bits, two steps per load
  uint4_t h[T][S / 4];      // high bits, four steps per load
  uint32_t sc[T][S / 4];    // sub-block scales, four steps
  uint32_t d[T][S / 4];     // binary16 d (low half), one per super-block
};

// The 16 codes q - 32 of one sub-block from its low-bit half (lo0, lo1: byte
// c = low(c) | low(8 + c) << 4) and its high-bit word, elements in order.
__device__ __forceinline__ int4_t q6_codes(uint32_t lo0, uint32_t lo1, uint32_t hw) {
  const uint32_t m = 0x0F0F0F0Fu;
  const uint32_t lo[4] = {lo0 & m, lo1 & m, (lo0 >> 4) & m, (lo1 >> 4) & m};
  int4_t q;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t v = lo[c] | (((hw >> (2 * c)) & 0x03030303u) << 4);   // 0..63 per byte
    q[c] = (int)(((v | 0x80808080u) - 0x20202020u) ^ 0x80808080u);      // q - 32, no borrow
  }
  return q;
}

// (No __restrict__ on the inputs: the issue fences below must be able to
// order their loads.)
template <int T, int WR, int KS, int S, int MP>
__global__ __launch_bounds__(64 * WR * KS) void mmvq_q6_k_packed_kernel(
    const uint8_t *wp, int N, int K, const int8_t *a_qs, const uint16_t *a_d, int M, float *y) {
  using C = q6p::Cfg<T, WR, KS, S, MP>;
  using R = Q6pWeights<T, S>;
  constexpr int MH = C::kMH;
  extern __shared__ uint4_t smem4[];
  uint8_t *smem = reinterpret_cast<uint8_t *>(smem4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wr = wave % WR, ks = wave / WR;
  const int j = lane & 15, grp = lane >> 4;
  const int U = (N + 15) >> 4, P = K >> 7, Q = K >> 8, nb = K >> 5;
  const int u0 = (blockIdx.x * WR + wr) * T;
  uint8_t *abuf = smem + ks * C::kNab * C::kAst;

  const int nct = K / (64 * S);
  const int cps = (nct + KS - 1) / KS;
  const int cb = ks * cps, ce = min(nct, cb + cps);

  // weight sources: tiles past the last repeat it (their rows are not stored)
  const size_t oH = (size_t)U * P * 1024, oC = oH + (size_t)U * Q * 1024,
               oD = oC + (size_t)U * Q * 256;
  const uint8_t *lp[T], *hp[T], *cp[T], *dp[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const size_t u = (size_t)min(u0 + t, U - 1);
    lp[t] = wp + u * P * 1024 + 16 * lane;
    hp[t] = wp + oH + u * Q * 1024 + 16 * lane;
    cp[t] = wp + oC + u * Q * 256 + 4 * lane;
    dp[t] = wp + oD + u * Q * 32 + 2 * j;
  }
  // activation pieces of this wave (as in the Q4_0 matrix-core kernels;
  // the scale piece: lanes [0, kNd) load 16-byte pieces of 8 d8 of row am)
  const int al = lane < C::kNd ? lane : 0;
  const int apc = al % (S / 4), am = al / (S / 4);
  const uint8_t *asrc[C::kApw];
  int apiece[C::kApw];
#pragma unroll
  for (int a = 0; a < C::kApw; ++a) {
    const int p = min(wr + WR * a, C::kAp - 1);
    apiece[a] = p;
    if (p < C::kAi) {
      const int r = min(p * C::kRpa + (lane % C::kRpa), M - 1);
      const int col = (lane / C::kRpa) ^ p;
      asrc[a] = reinterpret_cast<const uint8_t *>(a_qs + (size_t)r * K + 16 * col);
    } else {
      asrc[a] = reinterpret_cast<const uint8_t *>(a_d + (size_t)min(am, M - 1) * nb + 8 * apc);
    }
  }

  // Weights and activations in separate registers: two weight sets
  // alternate, one activation set (it goes to LDS before the next load).
  uint4_t av[C::kApw];
  auto load_w = [&](int c, R &rg) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int e = 0; e < S / 2; ++e)
        rg.l[t][e] = load16_nt(lp[t] + (size_t)(c * (S / 2) + e) * 1024);
#pragma unroll
      for (int q = 0; q < S / 4; ++q) {
        const size_t sb = (size_t)c * (S / 4) + q;
        rg.h[t][q] = load16_nt(hp[t] + sb * 1024);
        rg.sc[t][q] = *reinterpret_cast<const uint32_t *>(cp[t] + sb * 256);
        rg.d[t][q] = *reinterpret_cast<const uint16_t *>(dp[t] + sb * 32);
      }
    }
    issue_fence();   // keep the loads in the order they are waited for
  };
  auto load_a = [&](int c) {
#pragma unroll
    for (int a = 0; a < C::kApw; ++a)
      av[a] = load16(asrc[a] + (size_t)c * (apiece[a] < C::kAi ? 64 * S : 4 * S));
    issue_fence();
  };
  auto store_act = [&](uint8_t *ab) {
#pragma unroll
    for (int a = 0; a < C::kApw; ++a) {
      if (apiece[a] < C::kAi) {
        *reinterpret_cast<uint4_t *>(ab + 1024 * apiece[a] + 16 * lane) = av[a];
      } else if (lane < C::kNd) {
        // 8 blocks of row am: float d8 at slot 0
        float *as = reinterpret_cast<float *>(ab + C::kAsOff) + 2 * am;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          as[16 * (8 * apc + e)] = f16_bits_to_f32((uint16_t)(av[a][e >> 1] >> (16 * (e & 1))));
      }
    }
  };

  float4_t acc[T][MH];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int h = 0; h < MH; ++h) acc[t][h] = float4_t{0.f, 0.f, 0.f, 0.f};

  // A operand sources: lane (a = j, g) is live when a / 4 == g; its
  // activation row is (a % 4) + 4 h for instruction h (rows past MP wrap).
  // Row m's 16-byte column 4 st + g sits at slot (4 st + g) ^ piece.
  const bool live = (j >> 2) == grp;
  int aoff[MH];
#pragma unroll
  for (int h = 0; h < MH; ++h) {
    const int m = (4 * h + (j & 3)) & (MP - 1), ablk = m / C::kRpa;
    aoff[h] = 1024 * ablk + 16 * (m % C::kRpa) + 16 * C::kRpa * (grp ^ ablk);
  }
  const uint8_t *zero = smem + C::kZeroOff;
  constexpr int kAStride = 64 * C::kRpa;                   // bytes per step (4 columns)
  static_assert(kAStride * (S - 1) + 16 <= 1024, "zero area covers the chunk");
  auto consume = [&](const uint8_t *ab, const R &rg) {
    int4_t isum[S][T][MH];
#pragma unroll
    for (int st = 0; st < S; ++st) {
      int4_t aop[MH];
#pragma unroll
      for (int h = 0; h < MH; ++h)
        aop[h] = __builtin_bit_cast(int4_t, *reinterpret_cast<const uint4_t *>(
                                                (live ? ab + aoff[h] : zero) + kAStride * st));
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint4_t &w2 = rg.l[t][st >> 1];
        const int4_t bop = q6_codes(w2[2 * (st & 1)], w2[2 * (st & 1) + 1],
                                    rg.h[t][st >> 2][st & 3]);
        const int4_t z = {0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < MH; ++h) isum[st][t][h] = mfma_16x16x64_i8(aop[h], bop, z);
      }
    }
#pragma unroll
    for (int st = 0; st < S; ++st) {
      // this lane's sub-block grp lies in block 2 st + grp / 2 of the chunk
      const float *asf = reinterpret_cast<const float *>(ab + C::kAsOff + 64 * (2 * st + (grp >> 1)));
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int sc = (int)(int8_t)(rg.sc[t][st >> 2] >> (8 * (st & 3)));
        const float dsc = f16_bits_to_f32((uint16_t)rg.d[t][st >> 2]) * (float)sc;
#pragma unroll
        for (int h = 0; h < MH; ++h) {
          const float4_t d8 = {asf[8 * h], asf[8 * h + 2], asf[8 * h + 4], asf[8 * h + 6]};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[t][h][r] = fmaf(dsc, d8[r] * (float)isum[st][t][h][r], acc[t][h][r]);
        }
      }
    }
  };

  *reinterpret_cast<uint4_t *>(smem + C::kZeroOff + 16 * lane) = uint4_t{0u, 0u, 0u, 0u};
  const int steps = WR > 1 ? cps : ce - cb;
  const int cl = max(ce - 1, 0);
  auto chunk = [&](int k, R &cur, R &nxt, auto load_next) {
    const int c = cb + k;
    if constexpr (decltype(load_next)::value) load_w(min(c + 1, cl), nxt);
    uint8_t *ab = abuf + (k & (C::kNab - 1)) * C::kAst;
    store_act(ab);
    if constexpr (decltype(load_next)::value) load_a(min(c + 1, cl));
    if constexpr (WR > 1) wg_barrier();
    if (c < ce) consume(ab, cur);
  };
  if (steps > 0) {
    R ra, rb;
    load_w(min(cb, cl), ra);
    load_a(min(cb, cl));
    int k = 0;
    for (; k + 2 < steps; k += 2) {
      chunk(k, ra, rb, std::true_type{});
      chunk(k + 1, rb, ra, std::true_type{});
    }
    if (k + 2 == steps) {
      chunk(k, ra, rb, std::true_type{});
      chunk(k + 1, rb, ra, std::false_type{});
    } else {
      chunk(k, ra, rb, std::false_type{});
    }
  }

  if constexpr (KS > 1) {
    wg_barrier();
    float4_t *red = reinterpret_cast<float4_t *>(smem);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int h = 0; h < MH; ++h) red[((wave * T + t) * MH + h) * kWave + lane] = acc[t][h];
    wg_barrier();
    if (ks == 0) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int h = 0; h < MH; ++h)
#pragma unroll
          for (int v = 1; v < KS; ++v)
            acc[t][h] += red[(((v * WR + wr) * T + t) * MH + h) * kWave + lane];
    }
  }
  // lanes j, j + 16, j + 32, j + 48 hold the four sub-blocks of each step
  if (ks == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        float4_t v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = add_swap32(acc[t][h][r]);
          v[r] = s + __shfl_xor(s, 16);
        }
        const int n = 16 * (u0 + t) + j;
        if (lane < 16 && n < N) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int mm = 4 * h + r;
            if (mm < M) y[(size_t)mm * N + n] = v[r];
          }
        }
      }
    }
  }
}

template <int T, int WR, int KS, int S, int MP>
static hipError_t launch_q6p_cfg(const uint8_t *wp, int N, int K, const int8_t *a_qs,
                                 const uint16_t *a_d, int M, float *y, hipStream_t stream) {
  using C = q6p::Cfg<T, WR, KS, S, MP>;
  if (K % (64 * S) != 0) return hipErrorInvalidValue;   // chunks must tile K
  const hipError_t lds_ok =
      allow_lds((const void *)mmvq_q6_k_packed_kernel<T, WR, KS, S, MP>, C::kLds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int tiles = (N + 15) / 16;
  const int blocks = (tiles + T * WR - 1) / (T * WR);
  hipLaunchKernelGGL((mmvq_q6_k_packed_kernel<T, WR, KS, S, MP>), dim3(blocks),
                     dim3(64 * C::kWaves), C::kLds, stream, wp, N, K, a_qs, a_d, M, y);
  return hipGetLastError();
}

// One tile per wave and chunks of 4 steps (one super-block) throughout;
// measured over every configuration on the Qwen3-8B projections and six
// more matrices (K 2560..14336, N 4096..24576) at M = 1, 4, 8: a K split of
// 8 up to 256 tiles, 4 up to 799, 2 up to 1099, and on wider matrices a
// split of 4 at M <= 4, two waves sharing activations with a split of 2 at
// M = 5..8.
template <int MP>
static hipError_t launch_q6p_mp(const uint8_t *wp, int N, int K, const int8_t *a_qs,
                                const uint16_t *a_d, int M, float *y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
#define SKINNY_Q6P(T, WR, KS, S) \
  return launch_q6p_cfg<T, WR, KS, S, MP>(wp, N, K, a_qs, a_d, M, y, stream)
  if (tiles >= 1100) {
    if (MP == 8) SKINNY_Q6P(1, 2, 2, 4);
    SKINNY_Q6P(1, 1, 4, 4);
  }
  if (tiles >= 800) SKINNY_Q6P(1, 1, 2, 4);
  if (tiles > 256) SKINNY_Q6P(1, 1, 4, 4);
  SKINNY_Q6P(1, 1, 8, 4);
#undef SKINNY_Q6P
}

hipError_t launch_mmvq_q6_k_packed(const uint8_t *wp, int N, int K, const int8_t *a_qs,
                                   const uint16_t *a_d, int M, float *y, hipStream_t stream) {
  if (M <= 1) return launch_q6p_mp<1>(wp, N, K, a_qs, a_d, M, y, stream);
  if (M <= 2) return launch_q6p_mp<2>(wp, N, K, a_qs, a_d, M, y, stream);
  if (M <= 4) return launch_q6p_mp<4>(wp, N, K, a_qs, a_d, M, y, stream);
  return launch_q6p_mp<8>(wp, N, K, a_qs, a_d, M, y, stream);
}

// ------------------------------------------------------------------ prepack

// One thread per 16 packed bytes, grid-stride over the four planes in order.
__global__ __launch_bounds__(256) void prepack_q6_k_kernel(
    const uint8_t *__restrict__ ql, const uint8_t *__restrict__ qh,
    const int8_t *__restrict__ sc, const uint16_t *__restrict__ dd, int N, int K,
    uint8_t *__restrict__ wp) {
  const size_t U = (size_t)(N + 15) / 16, P = (size_t)K / 128, Q = (size_t)K / 256;
  const size_t nL = U * P * 64, nH = U * Q * 64, nC = U * Q * 16, nD = U * Q * 2;
  const size_t total = nL + nH + nC + nD;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (size_t)gridDim.x * blockDim.x) {
    uint4_t v = uint4_t{0u, 0u, 0u, 0u};
    if (p < nL) {
      const int l = (int)(p & 63), jj = l & 15, g = l >> 4;
      const size_t blk = p >> 6, u = blk / P, pp = blk - u * P, row = 16 * u + jj;
      if (row < (size_t)N) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          // sub-block g of step 2 pp + e: half g % 2 of 32-element block b
          const size_t b = 4 * pp + 2 * e + (g >> 1);
          const uint4_t src = load16(ql + row * ((size_t)K / 2) + 16 * b);
          const int sh = 4 * (g & 1);
          uint32_t w[2] = {0u, 0u};
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint32_t lo = (src[c >> 2] >> (8 * (c & 3) + sh)) & 15u;
            const uint32_t hi = (src[(c + 8) >> 2] >> (8 * ((c + 8) & 3) + sh)) & 15u;
            w[c >> 2] |= (lo | (hi << 4)) << (8 * (c & 3));
          }
          v[2 * e] = w[0];
          v[2 * e + 1] = w[1];
        }
      }
    } else if (p < nL + nH) {
      const size_t r = p - nL;
      const int l = (int)(r & 63), jj = l & 15, g = l >> 4;
      const size_t blk = r >> 6, u = blk / Q, q = blk - u * Q, row = 16 * u + jj;
      if (row < (size_t)N) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const size_t b = 2 * (4 * q + t) + (g >> 1);
          v[t] = *reinterpret_cast<const uint32_t *>(qh + row * ((size_t)K / 4) + 8 * b +
                                                     4 * (g & 1));
        }
      }
    } else if (p < nL + nH + nC) {
      const size_t r = p - nL - nH;
      const size_t blk = r >> 4, u = blk / Q, q = blk - u * Q;
      const int k = (int)(r & 15);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int l = 4 * k + x, jj = l & 15, g = l >> 4;
        const size_t row = 16 * u + jj;
        if (row >= (size_t)N) continue;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t s = (uint8_t)sc[row * ((size_t)K / 16) + 16 * q + 4 * t + g];
          v[x] |= s << (8 * t);
        }
      }
    } else {
      const size_t r = p - nL - nH - nC;
      const size_t blk = r >> 1, u = blk / Q, q = blk - u * Q;
      const int k = (int)(r & 1);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const size_t row = 16 * u + 8 * k + x;
        if (row < (size_t)N) v[x >> 1] |= (uint32_t)dd[row * Q + q] << (16 * (x & 1));
      }
    }
    *reinterpret_cast<uint4_t *>(wp + 16 * p) = v;
  }
}

hipError_t launch_prepack_q6_k(const uint8_t *ql, const uint8_t *qh, const int8_t *sc,
                               const uint16_t *dd, int N, int K, uint8_t *wp,
                               hipStream_t stream) {
  const size_t U = (size_t)(N + 15) / 16, P = (size_t)K / 128, Q = (size_t)K / 256;
  const size_t total = U * P * 64 + U * Q * (64 + 16 + 2);
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(prepack_q6_k_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ql, qh,
                     sc, dd, N, K, wp);
  return hipGetLastError();
}

}  // namespace skinny
