// gemv_nvfp4_packed.hip -- NVFP4 weights permuted once, when they are
// loaded, into the matrix cores' operand order, and the skinny GEMM that
// streams them (M = 1..16 binary16 activation rows).
//
// "v100-skinny README", "How QPN works": the weights are rearranged at load
// time into the order in which the matrix instructions consume them, so the
// main loop moves each loaded register straight into an operand with no
// shuffle.  The order here is that of the A operand of
// v_mfma_f32_16x16x32_f16 as the NVFP4 matrix-core kernel feeds it: lane
// l = 16 g + i of a wave supplies row i of a 16-row tile and, for each
// 128-element step s, the 32 consecutive elements 128 s + 32 g .. + 31 (its
// four operands take 8 of them each); the B operands are the activations of
// the same elements.  The arithmetic is that kernel's: codes and group
// scales decode exactly to binary16, the matrix cores accumulate in float32
// over all of K, and the per-tensor scale multiplies the finished sum.
//
// Packed layout (K % 256 == 0; U = ceil(N / 16) tiles of 16 rows, S = K / 128
// steps, V = ceil(S / 8) scale blocks per tile):
//   codes plane: U S blocks of 1024 bytes, block (u, s) at byte 1024 (u S + s);
//     its bytes 16 l .. 16 l + 15 are the code bytes 64 s + 16 g .. + 15 of
//     row 16 u + i (elements 128 s + 32 g .. + 31);
//   scale plane, right after it: U V blocks of 1024 bytes, block (u, v) at
//     byte 1024 (U S + u V + v); its bytes 16 l + 2 t and 16 l + 2 t + 1
//     (t < 8) are the E4M3 scales of groups 8 (8 v + t) + 2 g and + 1 of row
//     16 u + i, the two groups of that lane's elements in step 8 v + t.
//   Rows at or past N and steps at or past S hold zero bytes.
// Size: 1024 U (S + V) bytes: the canonical bytes of 16 U rows, rounded up
// to whole 8-step scale blocks.
//
// A wave streams whole 1 KB blocks: each 128-bit load instruction reads
// 1 KB of contiguous codes and lands every lane's 16 bytes in the registers
// its operands are built from.  The activations are staged through LDS as
// in the canonical kernel (shared by the WR waves of a K slice).
// Bytes per call: 1024 U (S + V) weights + 2 M K activations + 2 M N out.
#include <type_traits>

#include "device.h"
#include "launch.h"
#include "nvfp4.h"

namespace skinny {

// Workgroup: WR x KS waves; WR waves own different tiles (T each) and share
// one K slice's activation chunks, KS slices split K.  A chunk is S steps.
// The activation chunk (MP rows; rows past M repeat row M - 1) is read by
// the WR waves in 1 KB pieces, written to the slice's LDS buffer
// (double-buffered when WR > 1, one barrier per chunk), and read back in the
// B-operand layout; the KS partial tiles are summed in LDS at the end.
namespace nvp {
template <int T, int WR, int KS, int S, int MP>
struct Cfg {
  static constexpr int kWaves = WR * KS;
  static constexpr int kRpa = 4 / S;                // activation rows per 1 KB piece
  // activation pieces per chunk (one piece, its rows repeating row 0, when
  // a single row is less than a piece)
  static constexpr int kAi = MP >= kRpa ? MP / kRpa : 1;
  static constexpr int kApw = (kAi + WR - 1) / WR;  // activation loads per wave
  static constexpr int kNab = WR > 1 ? 2 : 1;       // activation buffers per slice
  static constexpr int kAst = kAi * 1024;           // one activation buffer
  static constexpr int kAct = KS * kNab * kAst;
  static constexpr int kRed = KS > 1 ? kWaves * T * kWave * 16 : 0;
  static constexpr int kLds = kAct > kRed ? kAct : kRed;
  static_assert(S == 2 || S == 4, "chunk steps");
  static_assert(MP == 1 || MP == 2 || MP == 4 || MP == 8 || MP == 16, "padded rows");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};
}  // namespace nvp

template <int T, int S>
struct NvpWeights {
  uint4_t c[T * S];                                         // codes, [tile][step]
  std::conditional_t<S == 4, uint2_t, uint32_t> s[T];       // 2 scale bytes per step
};

// (No __restrict__ on the inputs: the issue fences below must be able to
// order their loads.)
template <int T, int WR, int KS, int S, int MP>
__global__ __launch_bounds__(64 * WR * KS) void gemv_nvfp4_packed_kernel(
    const uint8_t *wp, float g, int N, int K, const uint16_t *x, int M, uint16_t *y) {
  using C = nvp::Cfg<T, WR, KS, S, MP>;
  using R = NvpWeights<T, S>;
  extern __shared__ uint4_t smem4[];
  uint8_t *smem = reinterpret_cast<uint8_t *>(smem4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wr = wave % WR, ks = wave / WR;
  const int i = lane & 15, grp = lane >> 4;
  const int U = (N + 15) >> 4, Ks = K >> 7, Vs = (Ks + 7) >> 3;
  const int u0 = (blockIdx.x * WR + wr) * T;
  uint8_t *abuf = smem + ks * C::kNab * C::kAst;

  const int nct = Ks / S;
  const int cps = (nct + KS - 1) / KS;
  const int cb = ks * cps, ce = min(nct, cb + cps);

  // per-lane sources: tiles past the last repeat it (their rows are not stored)
  const uint8_t *cp[T];
  const uint8_t *sp[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const size_t u = (size_t)min(u0 + t, U - 1);
    cp[t] = wp + u * Ks * 1024 + 16 * lane;
    sp[t] = wp + ((size_t)U * Ks + u * Vs) * 1024 + 16 * lane;
  }
  const uint16_t *asrc[C::kApw];
  int apiece[C::kApw];
#pragma unroll
  for (int a = 0; a < C::kApw; ++a) {
    const int p = min(wr + WR * a, C::kAi - 1);
    apiece[a] = p;
    const int r = min(p * C::kRpa + (lane % C::kRpa), M - 1);
    const int j = (lane / C::kRpa) ^ p;
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
        rg.c[t * S + st] = load16_nt(cp[t] + (size_t)(c * S + st) * 1024);
    // a chunk takes 2 S of the 16 scale bytes each lane holds per 8 steps:
    // the default cache policy keeps the rest of the line for the next chunks
    const int s0 = c * S;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint8_t *p = sp[t] + (size_t)(s0 >> 3) * 1024 + 2 * (s0 & 7);
      if constexpr (S == 4) rg.s[t] = load8(p);
      else rg.s[t] = *reinterpret_cast<const uint32_t *>(p);
    }
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

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  // B operands: lane (i, grp) takes activation row i (columns >= MP wrap),
  // elements 128 st + 32 grp + 8 u .. + 7 for u < 4.  A 1 KB piece holds
  // kRpa rows; their 16-byte columns are XOR-swizzled by the piece index.
  const int ar = i & (MP - 1), aa = ar / C::kRpa;
  const int aoff = 1024 * aa + 16 * (ar % C::kRpa);
  auto consume = [&](const uint8_t *ab, const R &rg) {
#pragma unroll
    for (int st = 0; st < S; ++st) {
      uint4_t xv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = 16 * st + 4 * grp + u;
        xv[u] = *reinterpret_cast<const uint4_t *>(ab + aoff + 16 * C::kRpa * (j ^ aa));
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        uint32_t sc;
        if constexpr (S == 4) sc = rg.s[t][st >> 1] >> (16 * (st & 1));
        else sc = rg.s[t] >> (16 * st);
        nvfp4_step(rg.c[t * S + st], sc, xv, acc[t]);
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
    for (int t = 0; t < T; ++t) red[(wave * T + t) * kWave + lane] = acc[t];
    wg_barrier();
    if (ks == 0) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int v = 1; v < KS; ++v) acc[t] += red[((v * WR + wr) * T + t) * kWave + lane];
    }
  }
  if (ks == 0 && i < M) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = 16 * (u0 + t) + 4 * grp + r;
        if (n < N) y[(size_t)i * N + n] = f32_to_f16_bits(acc[t][r] * g);
      }
    }
  }
}

template <int T, int WR, int KS, int S, int MP>
static hipError_t launch_packed_cfg(const uint8_t *wp, float g, int N, int K, const uint16_t *x,
                                    int M, uint16_t *y, hipStream_t stream) {
  using C = nvp::Cfg<T, WR, KS, S, MP>;
  if (K % (128 * S) != 0) return hipErrorInvalidValue;   // chunks must tile K
  const hipError_t lds_ok =
      allow_lds((const void *)gemv_nvfp4_packed_kernel<T, WR, KS, S, MP>, C::kLds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int tiles = (N + 15) / 16;
  const int blocks = (tiles + T * WR - 1) / (T * WR);
  hipLaunchKernelGGL((gemv_nvfp4_packed_kernel<T, WR, KS, S, MP>), dim3(blocks),
                     dim3(64 * C::kWaves), C::kLds, stream, wp, g, N, K, x, M, y);
  return hipGetLastError();
}

// Tiles per wave T, waves sharing activations WR, K slices KS and chunk
// steps S, measured on MI355X over every configuration on 13 matrices (K
// 3072..17408, N 2048..34816; weights rotating over > 2 GiB) at M = 1, 2,
// 4, 8 and 16; each row below is within a few percent of the best on the
// matrices it covers.  Chunks of 4 steps need K % 512 == 0 (s4).
//   M <= 2: one tile per wave, a K split of 4 (8 up to 256 tiles) keeps
//     enough waves streaming; wide matrices need no split.
template <int MP>
static hipError_t launch_packed_narrow_m(const uint8_t *wp, float g, int N, int K,
                                         const uint16_t *x, int M, uint16_t *y,
                                         hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
#define SKINNY_NVP(T, WR, KS, S) \
  return launch_packed_cfg<T, WR, KS, S, MP>(wp, g, N, K, x, M, y, stream)
  if (tiles >= 1536) SKINNY_NVP(1, 1, 1, 2);
  if (tiles > 256) {
    if (s4 && K >= 8192) SKINNY_NVP(1, 1, 4, 4);
    SKINNY_NVP(1, 1, 4, 2);
  }
  SKINNY_NVP(1, 1, 8, 2);
#undef SKINNY_NVP
}

//   M = 3, 4: wide matrices unsplit, mid-width ones a split of 2 (with two
//     waves sharing activations from 800 tiles), narrow long rows two tiles
//     per wave and a split of 4.
static hipError_t launch_packed_m4(const uint8_t *wp, float g, int N, int K, const uint16_t *x,
                                   int M, uint16_t *y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
#define SKINNY_NVP(T, WR, KS, S) \
  return launch_packed_cfg<T, WR, KS, S, 4>(wp, g, N, K, x, M, y, stream)
  if (tiles >= 1536) {
    if (s4) SKINNY_NVP(1, 1, 1, 4);
    SKINNY_NVP(1, 1, 1, 2);
  }
  if (tiles >= 800) {
    if (s4) SKINNY_NVP(1, 2, 2, 4);
    SKINNY_NVP(1, 2, 2, 2);
  }
  if (tiles >= 512) {
    if (s4) SKINNY_NVP(1, 1, 2, 4);
    SKINNY_NVP(1, 1, 2, 2);
  }
  if (tiles > 256) {
    if (K >= 8192) {
      if (s4) SKINNY_NVP(2, 1, 4, 4);
      SKINNY_NVP(2, 1, 4, 2);
    }
    SKINNY_NVP(1, 1, 4, 2);
  }
  if (s4) SKINNY_NVP(1, 1, 4, 4);
  SKINNY_NVP(1, 1, 8, 2);
#undef SKINNY_NVP
}

//   M = 5..16: four waves share each activation chunk on wide matrices
//     (two from 1100 tiles, with a split of 2 from 600), narrow long rows
//     two tiles per wave and a split of 4, up to 256 tiles one tile per wave
//     and a split of 8 (4 for rows past 8192).
template <int MP>
static hipError_t launch_packed_wide_m(const uint8_t *wp, float g, int N, int K,
                                       const uint16_t *x, int M, uint16_t *y,
                                       hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
#define SKINNY_NVP(T, WR, KS, S) \
  return launch_packed_cfg<T, WR, KS, S, MP>(wp, g, N, K, x, M, y, stream)
  if (tiles >= 1536) {
    if (s4) SKINNY_NVP(1, 4, 1, 4);
    SKINNY_NVP(1, 4, 1, 2);
  }
  if (tiles >= 1100) {
    if (s4) SKINNY_NVP(1, 2, 1, 4);
    SKINNY_NVP(1, 2, 1, 2);
  }
  if (tiles >= 600) {
    if (s4) SKINNY_NVP(1, 4, 2, 4);
    SKINNY_NVP(1, 4, 2, 2);
  }
  if (tiles > 256) {
    if (s4 && K >= 8192 && MP <= 8) SKINNY_NVP(2, 1, 4, 4);
    SKINNY_NVP(2, 1, 4, 2);
  }
  if (s4) {
    if (K <= 8192) SKINNY_NVP(1, 1, 8, 4);
    SKINNY_NVP(1, 1, 4, 4);
  }
  SKINNY_NVP(1, 1, 8, 2);
#undef SKINNY_NVP
}

hipError_t launch_gemv_nvfp4_packed(const uint8_t *wp, float g, int N, int K, const uint16_t *x,
                                    int M, uint16_t *y, hipStream_t stream) {
  if (M <= 1) return launch_packed_narrow_m<1>(wp, g, N, K, x, M, y, stream);
  if (M <= 2) return launch_packed_narrow_m<2>(wp, g, N, K, x, M, y, stream);
  if (M <= 4) return launch_packed_m4(wp, g, N, K, x, M, y, stream);
  if (M <= 8) return launch_packed_wide_m<8>(wp, g, N, K, x, M, y, stream);
  return launch_packed_wide_m<16>(wp, g, N, K, x, M, y, stream);
}

// ------------------------------------------------------------------ prepack

// One thread per 16 packed bytes (a lane's piece of one block), grid-stride
// over both planes: codes pieces first, then scale pieces.
__global__ __launch_bounds__(256) void prepack_nvfp4_kernel(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, int N, int K,
    uint8_t *__restrict__ wp) {
  const size_t U = (size_t)(N + 15) / 16, Ks = (size_t)K / 128, Vs = (Ks + 7) / 8;
  const size_t nc = U * Ks * 64, total = nc + U * Vs * 64;
  const size_t rowc = (size_t)K / 2, rows_ = (size_t)K / 16;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(p & 63), i = l & 15, grp = l >> 4;
    uint4_t v = uint4_t{0u, 0u, 0u, 0u};
    if (p < nc) {
      const size_t blk = p >> 6, u = blk / Ks, s = blk - u * Ks;
      const size_t row = 16 * u + i;
      if (row < (size_t)N) v = load16(codes + row * rowc + 64 * s + 16 * grp);
    } else {
      const size_t blk = (p - nc) >> 6, u = blk / Vs, vb = blk - u * Vs;
      const size_t row = 16 * u + i;
      if (row < (size_t)N) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const size_t s = 8 * vb + t;
          if (s < Ks) {
            const uint32_t h =
                *reinterpret_cast<const uint16_t *>(scales + row * rows_ + 8 * s + 2 * grp);
            v[t >> 1] |= h << (16 * (t & 1));
          }
        }
      }
    }
    *reinterpret_cast<uint4_t *>(wp + 16 * p) = v;
  }
}

hipError_t launch_prepack_nvfp4(const uint8_t *codes, const uint8_t *scales, int N, int K,
                                uint8_t *wp, hipStream_t stream) {
  const size_t U = (size_t)(N + 15) / 16, Ks = (size_t)K / 128, Vs = (Ks + 7) / 8;
  const size_t total = U * (Ks + Vs) * 64;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(prepack_nvfp4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes,
                     scales, N, K, wp);
  return hipGetLastError();
}

}  // namespace skinny
