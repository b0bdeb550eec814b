// gemv_fp8_packed.hip -- FP8 E4M3 weights permuted once, when they are
// loaded, into the matrix cores' operand order, and the skinny GEMM that
// streams them (M = 1..96 binary16 activation rows).
//
// "v100-skinny README", "How QPN works": the weights are rearranged at load
// time into the order in which the matrix instructions consume them, so the
// main loop moves each loaded register straight into an operand with no
// shuffle.  The order is that of the A operand of v_mfma_f32_16x16x32_f16 as
// the FP8 matrix-core kernel feeds it: lane l = 16 g + i of a wave supplies
// row i of a 16-row tile and, for each 128-element step s, the 32
// consecutive elements 128 s + 32 g .. + 31, decoded exactly to binary16.
// The arithmetic is that kernel's: float32 accumulation over all of K, the
// channel scale applied to the finished sum.
//
// Packed layout (K % 256 == 0; U = ceil(N / 16) tiles of 16 rows, S = K / 128
// steps): U S blocks of 2048 bytes, block (u, s) at byte 2048 (u S + s); its
// bytes 1024 e + 16 l .. 1024 e + 16 l + 15 (e < 2) are the weight bytes
// 128 s + 32 g + 16 e .. + 15 of row 16 u + i.  Rows at or past N are zero.
// Size: 16 U K bytes (the canonical bytes of 16 U rows).  The channel scales
// stay the caller's float32 [N] array.
// Bytes per call: 16 U K weights + 4 N scales + 2 M K activations + 2 M N out.
#include <type_traits>

#include "device.h"
#include "fp8.h"
#include "launch.h"

namespace skinny {

// Workgroup: WR x KS waves; WR waves own different tiles (T each) and share
// one K slice's activation chunks, KS slices split K.  A chunk is S steps.
// The activation chunk (MP rows; rows past M repeat row M - 1) is read by
// the WR waves in 1 KB pieces, written to the slice's LDS buffer
// (double-buffered when WR > 1, one barrier per chunk), and read back in the
// B-operand layout; above 16 rows each decoded weight operand feeds MP / 16
// column tiles.  A grid of gridDim.y > 1 takes the rows in groups of MP.
// The KS partial tiles are summed in LDS at the end.
namespace f8p {
template <int T, int WR, int KS, int S, int MP>
struct Cfg {
  static constexpr int kWaves = WR * KS;
  static constexpr int kMT = MP > 16 ? MP / 16 : 1;  // column tiles
  static constexpr int kRpa = 4 / S;                // activation rows per 1 KB piece
  static constexpr int kACols = 16 * S;             // 16-byte columns per activation row
  // activation pieces per chunk (one piece, its rows repeating row 0, when
  // the rows are fewer than a piece holds)
  static constexpr int kAi = MP >= kRpa ? MP / kRpa : 1;
  static constexpr int kApw = (kAi + WR - 1) / WR;  // activation loads per wave
  static constexpr int kNab = WR > 1 ? 2 : 1;       // activation buffers per slice
  static constexpr int kAst = kAi * 1024;
  static constexpr int kAct = KS * kNab * kAst;
  static constexpr int kRed = KS > 1 ? kWaves * T * kMT * kWave * 16 : 0;
  static constexpr int kLds = kAct > kRed ? kAct : kRed;
  static_assert(S == 1 || S == 2 || S == 4, "chunk steps");
  static_assert(MP == 1 || MP == 2 || MP == 4 || MP == 8 || (MP % 16 == 0 && MP <= 96),
                "padded activation rows");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};
}  // namespace f8p

template <int T, int S>
struct F8pWeights {
  uint4_t c[T][S][2];   // [tile][step][half]
};

// (No __restrict__ on the inputs: the issue fences below must be able to
// order their loads.)
template <int T, int WR, int KS, int S, int MP>
__global__ __launch_bounds__(64 * WR * KS) void gemv_fp8_packed_kernel(
    const uint8_t *wp, const float *cs, int N, int K, const uint16_t *x, int M, uint16_t *y) {
  using C = f8p::Cfg<T, WR, KS, S, MP>;
  using R = F8pWeights<T, S>;
  constexpr int MT = C::kMT;
  const int U = (N + 15) >> 4, Ks = K >> 7;
  if ((int)blockIdx.x * (T * WR) >= U) return;        // whole workgroup (grid padding)
  {
    const int m0 = (int)blockIdx.y * MP;
    x += (size_t)m0 * K;
    y += (size_t)m0 * N;
    M = min(MP, M - m0);
  }
  extern __shared__ uint4_t smem4[];
  uint8_t *smem = reinterpret_cast<uint8_t *>(smem4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wr = wave % WR, ks = wave / WR;
  const int i = lane & 15, grp = lane >> 4;
  const int u0 = (blockIdx.x * WR + wr) * T;
  uint8_t *abuf = smem + ks * C::kNab * C::kAst;

  const int nct = Ks / S;
  const int cps = (nct + KS - 1) / KS;
  const int cb = ks * cps, ce = min(nct, cb + cps);

  // per-lane sources: tiles past the last repeat it (their rows are not stored)
  const uint8_t *cp[T];
#pragma unroll
  for (int t = 0; t < T; ++t)
    cp[t] = wp + (size_t)min(u0 + t, U - 1) * Ks * 2048 + 16 * lane;
  const uint16_t *asrc[C::kApw];
  int apiece[C::kApw];
#pragma unroll
  for (int a = 0; a < C::kApw; ++a) {
    const int p = min(wr + WR * a, C::kAi - 1);
    apiece[a] = p;
    const int r = min(p * C::kRpa + (lane % C::kRpa), M - 1);
    const int j = (lane / C::kRpa) ^ (p & (C::kACols - 1));
    asrc[a] = x + (size_t)r * K + 8 * j;
  }
  // Weights and activations are loaded into separate registers: two weight
  // sets alternate (one is consumed while the next is in flight), one
  // activation set suffices (it goes to LDS before the next is loaded).
  uint4_t av[C::kApw];
  auto load_w = [&](int c, R &rg) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int st = 0; st < S; ++st)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          rg.c[t][st][e] = load16_nt(cp[t] + (size_t)(c * S + st) * 2048 + 1024 * e);
    issue_fence();   // keep the loads in the order they are waited for
  };
  auto load_a = [&](int c) {
#pragma unroll
    for (int a = 0; a < C::kApw; ++a) av[a] = load16(asrc[a] + (size_t)c * (128 * S));
    issue_fence();
  };
  auto store_act = [&](uint8_t *ab) {
#pragma unroll
    for (int a = 0; a < C::kApw; ++a)
      *reinterpret_cast<uint4_t *>(ab + 1024 * apiece[a] + 16 * lane) = av[a];
  };

  float4_t acc[T][MT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < MT; ++c) acc[t][c] = float4_t{0.f, 0.f, 0.f, 0.f};

  // B operands: lane (i, grp) of column tile c takes activation row
  // 16 c + i (MP >= 16) or i % MP, elements 128 st + 32 grp + 8 u .. + 7.
  auto act = [&](const uint8_t *ab, int st, int c, uint4_t (&xv)[4]) {
    const int ar = MP >= 16 ? 16 * c + i : (i & (MP - 1)), aa = ar / C::kRpa;
    const uint8_t *ap = ab + 1024 * aa + 16 * (ar % C::kRpa);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 16 * st + 4 * grp + u;
      xv[u] = *reinterpret_cast<const uint4_t *>(ap + 16 * C::kRpa * (j ^ (aa & (C::kACols - 1))));
    }
  };
  auto consume = [&](const uint8_t *ab, const R &rg) {
#pragma unroll
    for (int st = 0; st < S; ++st) {
      if constexpr (MT == 1) {
        uint4_t xv[4];
        act(ab, st, 0, xv);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          half8_t a[4];
          fp8_decode(rg.c[t][st], a);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            acc[t][0] = mfma_16x16x32_f16(a[u], __builtin_bit_cast(half8_t, xv[u]), acc[t][0]);
        }
      } else {
        // several column tiles: decode every weight tile once, reuse it MT times
        half8_t a[T][4];
#pragma unroll
        for (int t = 0; t < T; ++t) fp8_decode(rg.c[t][st], a[t]);
#pragma unroll
        for (int c = 0; c < MT; ++c) {
          uint4_t xv[4];
          act(ab, st, c, xv);
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u)
              acc[t][c] = mfma_16x16x32_f16(a[t][u], __builtin_bit_cast(half8_t, xv[u]), acc[t][c]);
        }
      }
    }
  };

  // One chunk: issue the next chunk's weight loads (LOAD), stage this
  // chunk's activations and issue the next chunk's, then consume this chunk
  // from registers.  Waves that share activations run cps chunks in
  // lockstep (the barrier); chunks past a slice's end re-read its last chunk
  // and compute nothing.  The last chunk issues no loads.
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
      for (int c = 0; c < MT; ++c) red[((wave * T + t) * MT + c) * kWave + lane] = acc[t][c];
    wg_barrier();
    if (ks == 0) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int c = 0; c < MT; ++c)
#pragma unroll
          for (int v = 1; v < KS; ++v)
            acc[t][c] += red[(((v * WR + wr) * T + t) * MT + c) * kWave + lane];
    }
  }
  if (ks == 0) {
#pragma unroll
    for (int c = 0; c < MT; ++c) {
      const int m = MP >= 16 ? 16 * c + i : i;
      if (m < M) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = 16 * (u0 + t) + 4 * grp + r;
            if (n < N) y[(size_t)m * N + n] = f32_to_f16_bits(acc[t][c][r] * cs[n]);
          }
        }
      }
    }
  }
}

// Rows past MP go to further grid rows (groups of MP); the grid's width is
// then rounded up to a multiple of 8, so the groups of one tile land on one
// XCD (workgroups are dealt to the 8 XCDs in turn) and re-read its weights
// from that XCD's L2.
template <int T, int WR, int KS, int S, int MP>
static hipError_t launch_f8p_cfg(const uint8_t *wp, const float *cs, int N, int K,
                                 const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  using C = f8p::Cfg<T, WR, KS, S, MP>;
  if (K % (128 * S) != 0) return hipErrorInvalidValue;   // chunks must tile K
  const hipError_t lds_ok =
      allow_lds((const void *)gemv_fp8_packed_kernel<T, WR, KS, S, MP>, C::kLds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int tiles = (N + 15) / 16;
  const int groups = (M + MP - 1) / MP;
  int blocks = (tiles + T * WR - 1) / (T * WR);
  if (groups > 1) blocks = (blocks + 7) / 8 * 8;
  hipLaunchKernelGGL((gemv_fp8_packed_kernel<T, WR, KS, S, MP>), dim3(blocks, groups),
                     dim3(64 * C::kWaves), C::kLds, stream, wp, cs, N, K, x, M, y);
  return hipGetLastError();
}

// Tiles per wave T, waves sharing activations WR, K slices KS and chunk
// steps S, measured on MI355X over every configuration on 13 matrices (K
// 3072..17408, N 2048..34816; weights rotating over > 2 GiB) at M = 1, 2,
// 4, 8, 16 (and the row groups below at M = 32 and 96); each row is within a
// few percent of the best on the matrices it covers.  Chunks of 4 steps need
// K % 512 == 0 (s4).
//   M <= 2: one tile per wave and a K split of 4 (8 up to 256 tiles; two
//     tiles per wave on long rows below 512 tiles).
template <int MP>
static hipError_t launch_f8p_narrow_m(const uint8_t *wp, const float *cs, int N, int K,
                                      const uint16_t *x, int M, uint16_t *y,
                                      hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
#define SKINNY_F8P(T, WR, KS, S) \
  return launch_f8p_cfg<T, WR, KS, S, MP>(wp, cs, N, K, x, M, y, stream)
  if (tiles >= 512) {
    if (s4) SKINNY_F8P(1, 1, 4, 4);
    SKINNY_F8P(1, 1, 4, 2);
  }
  if (tiles > 256) {
    if (K >= 8192) {
      if (s4) SKINNY_F8P(2, 1, 4, 4);
      SKINNY_F8P(2, 1, 4, 2);
    }
    SKINNY_F8P(1, 1, 4, 2);
  }
  SKINNY_F8P(1, 1, 8, 2);
#undef SKINNY_F8P
}

//   M = 3, 4: wide matrices a K split of 4; two waves sharing activations
//     from 1100 tiles, then mid-width ones unsplit, narrower ones a split of
//     4, or two waves sharing with a split of 2 (257..511 tiles).
static hipError_t launch_f8p_m4(const uint8_t *wp, const float *cs, int N, int K,
                                const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
#define SKINNY_F8P(T, WR, KS, S) \
  return launch_f8p_cfg<T, WR, KS, S, 4>(wp, cs, N, K, x, M, y, stream)
  if (tiles >= 1536) SKINNY_F8P(1, 1, 4, 2);
  if (tiles >= 1100) SKINNY_F8P(1, 2, 1, 2);
  if (tiles >= 600) {
    if (s4) SKINNY_F8P(1, 1, 1, 4);
    SKINNY_F8P(1, 1, 1, 2);
  }
  if (tiles >= 512) SKINNY_F8P(1, 1, 4, 2);
  if (tiles > 256) {
    if (s4) SKINNY_F8P(1, 2, 2, 4);
    SKINNY_F8P(1, 2, 2, 2);
  }
  SKINNY_F8P(1, 1, 4, 2);
#undef SKINNY_F8P
}

//   M = 5..16: two (from 1100 tiles) or four (600..1099) waves sharing each
//     activation chunk on wide matrices, two with a K split of 2 on narrower
//     ones, one tile per wave and a split of 4 up to 256 tiles.
template <int MP>
static hipError_t launch_f8p_wide_m(const uint8_t *wp, const float *cs, int N, int K,
                                    const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
#define SKINNY_F8P(T, WR, KS, S) \
  return launch_f8p_cfg<T, WR, KS, S, MP>(wp, cs, N, K, x, M, y, stream)
  if (MP == 16 && tiles >= 1536 && s4 && K >= 8192) SKINNY_F8P(2, 4, 1, 4);
  if (tiles >= 1100) {
    if (s4 && (MP == 8 || tiles >= 1536)) SKINNY_F8P(1, 2, 1, 4);
    SKINNY_F8P(1, 2, 1, 2);
  }
  if (tiles >= 600) {
    if (s4) SKINNY_F8P(1, 4, 1, 4);
    SKINNY_F8P(1, 4, 2, 2);
  }
  if (tiles > 256) {
    if (MP == 8) {
      if (s4 && tiles < 512) SKINNY_F8P(1, 2, 2, 4);
      SKINNY_F8P(1, 2, 2, 2);
    }
    if (s4) SKINNY_F8P(1, 2, 1, 4);
    SKINNY_F8P(1, 2, 1, 2);
  }
  if (MP == 16 && s4) SKINNY_F8P(1, 1, 4, 4);
  SKINNY_F8P(1, 1, 4, 2);
#undef SKINNY_F8P
}

// 17 <= M <= 96: one pass over the weights with MP / 16 column tiles on wide
// matrices (1536 tiles or more), groups of 16 rows (one grid row each, four
// waves sharing each activation chunk) on narrower ones, measured at M = 32
// and 96 on the four Qwen-shaped matrices: 5120 x 5120 at M = 96 24.7 ->
// 17.7 us, 17408 x 5120 69.0 -> 47.8 us against the canonical layout's
// chunked kernel.
static hipError_t launch_f8p_many(const uint8_t *wp, const float *cs, int N, int K,
                                  const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  if (tiles >= 1536) {
    switch ((M + 15) / 16) {
      case 2: return launch_f8p_cfg<2, 2, 1, 2, 32>(wp, cs, N, K, x, M, y, stream);
      case 3: return launch_f8p_cfg<2, 2, 1, 2, 48>(wp, cs, N, K, x, M, y, stream);
      case 4: return launch_f8p_cfg<1, 4, 1, 2, 64>(wp, cs, N, K, x, M, y, stream);
      case 5: return launch_f8p_cfg<1, 8, 1, 1, 80>(wp, cs, N, K, x, M, y, stream);
      default: return launch_f8p_cfg<1, 8, 1, 1, 96>(wp, cs, N, K, x, M, y, stream);
    }
  }
  if (M <= 48 && tiles < 512) {
    if (K % 512 == 0) return launch_f8p_cfg<1, 4, 1, 4, 16>(wp, cs, N, K, x, M, y, stream);
    return launch_f8p_cfg<1, 4, 1, 2, 16>(wp, cs, N, K, x, M, y, stream);
  }
  return launch_f8p_cfg<2, 4, 1, 2, 16>(wp, cs, N, K, x, M, y, stream);
}

hipError_t launch_gemv_fp8_packed(const uint8_t *wp, const float *cs, int N, int K,
                                  const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  if (M <= 1) return launch_f8p_narrow_m<1>(wp, cs, N, K, x, M, y, stream);
  if (M <= 2) return launch_f8p_narrow_m<2>(wp, cs, N, K, x, M, y, stream);
  if (M <= 4) return launch_f8p_m4(wp, cs, N, K, x, M, y, stream);
  if (M <= 8) return launch_f8p_wide_m<8>(wp, cs, N, K, x, M, y, stream);
  if (M <= 16) return launch_f8p_wide_m<16>(wp, cs, N, K, x, M, y, stream);
  return launch_f8p_many(wp, cs, N, K, x, M, y, stream);
}

// ------------------------------------------------------------------ prepack

// One thread per 16 packed bytes, grid-stride.
__global__ __launch_bounds__(256) void prepack_fp8_kernel(const uint8_t *__restrict__ w, int N,
                                                          int K, uint8_t *__restrict__ wp) {
  const size_t U = (size_t)(N + 15) / 16, Ks = (size_t)K / 128;
  const size_t total = U * Ks * 128;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(p & 63), e = (int)((p >> 6) & 1), i = l & 15, grp = l >> 4;
    const size_t blk = p >> 7, u = blk / Ks, s = blk - u * Ks;
    const size_t row = 16 * u + i;
    uint4_t v = uint4_t{0u, 0u, 0u, 0u};
    if (row < (size_t)N) v = load16(w + row * (size_t)K + 128 * s + 32 * grp + 16 * e);
    *reinterpret_cast<uint4_t *>(wp + 16 * p) = v;
  }
}

hipError_t launch_prepack_fp8(const uint8_t *w, int N, int K, uint8_t *wp, hipStream_t stream) {
  const size_t U = (size_t)(N + 15) / 16, Ks = (size_t)K / 128;
  const size_t total = U * Ks * 128;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(prepack_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, K,
                     wp);
  return hipGetLastError();
}

}  // namespace skinny
