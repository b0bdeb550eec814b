// mmvq_q4_0_packed.hip -- Q4_0 and Q4_K weights permuted once, when they are
// loaded, into the matrix cores' operand order, and the MMVQ that streams
// them (M = 1..8 rows of Q8_1 activations).
//
// "v100-skinny README", "How QPN works": the weights are rearranged at load
// time into the order in which the matrix instructions consume them, so the
// main loop moves each loaded register straight into an operand with no
// shuffle.  The arithmetic is the mat x vec of "Machine Learning on NVIDIA
// CMP" ("llama.cpp results", "The DP2A patch"): exact int32 block sums of
// codes against Q8_1 codes, then acc += d4 * (d8 * isum - 8 * s8) in
// float32, as in the canonical matrix-core kernel.
//
// The order is that of the B operand of v_mfma_i32_16x16x64_i8 as the
// canonical Q4_0 matrix-core kernel feeds it.  A 64-element step spans two
// blocks; lane l = 16 g + j, g = 2 h + b, supplies weight row j of a 16-row
// tile for K slot g: code bytes 8 b .. 8 b + 7 of block h of the step (their
// low nibbles, then their high nibbles: 16 codes).  The A operand is the
// block-diagonal activation operand of that kernel.
//
// Packed layout (K % 256 == 0; U = ceil(N / 16) tiles of 16 rows, P = K / 128
// pairs of steps, V = ceil(K / 512)):
//   codes plane: U P blocks of 1024 bytes, block (u, p) at byte 1024 (u P + p);
//     its bytes 16 l + 8 e .. 16 l + 8 e + 7 (e < 2) are the code bytes
//     8 b .. 8 b + 7 of block 4 p + 2 e + h of row 16 u + j (block h of step
//     2 p + e);
//   scale plane, right after it: U V blocks of 512 bytes, block (u, v) at byte
//     1024 U P + 512 (u V + v); its bytes 256 h + 16 j + 2 t and + 1 (t < 8)
//     are the binary16 scale of block 16 v + 2 t + h of row 16 u + j (block h
//     of step 8 v + t).  Lanes (j, 2 h) and (j, 2 h + 1) read the same bytes.
//   Rows at or past N and blocks at or past K / 32 hold zero bytes.
// Size: 1024 U P + 512 U V bytes: the canonical bytes of 16 U rows, rounded
// up to whole 512-element scale blocks.
//
// Q4_K has the same 4-bit codes in the same nibble order, so its codes
// plane is the same; its headers (16 bytes per row and 256-element
// super-block: d, dmin, 12 bytes of 6-bit scales and mins) form the second
// plane, tile-major: U K/256 blocks of 256 bytes, block (u, q) at byte
// 1024 U P + 256 (u K/256 + q), whose bytes 16 j .. 16 j + 15 are the header
// of super-block q of row 16 u + j, unchanged.  Size 1024 U P + U K bytes.
// The four lanes of row j read the same 16 bytes; the epilogue takes its
// sub-block's scale and min from them.
//
// IQ4_XS has the same 4-bit indices in the same nibble order (decoded
// through the IQ4_NL table into signed int8 operands), so its codes plane is
// the same too; its 8-byte super-block headers (d, H, L) form the second
// plane: U K/256 blocks of 128 bytes, block (u, q) at byte 1024 U P +
// 128 (u K/256 + q), whose bytes 8 j .. 8 j + 7 are the header of
// super-block q of row 16 u + j, unchanged.  Size 1024 U P + U K / 2 bytes.
// Bytes per call: 1024 U P + 512 U V weights + M K (1 + 4 / 32) activations
// + 4 M N out.
#include <type_traits>

#include "device.h"
#include "launch.h"
#include "q4_mfma.h"

namespace skinny {

// Weight formats of the packed kernel (as in the canonical matrix-core
// kernel of mmvq_q4_0.hip).
constexpr int kPkQ40 = 0, kPkQ4K = 1, kPkIQ4 = 2;
struct PkNoRegs {};

// Workgroup: WR x KS waves; WR waves own different tiles (T each) and share
// one K slice's activation chunks, KS slices split K.  A chunk is S steps.
// The activation chunk (MP rows of Q8_1 codes, rows past M repeating row
// M - 1, and their scales) is read by the WR waves in 16-byte pieces,
// written to the slice's LDS buffer (double-buffered when WR > 1, one
// barrier per chunk; scales converted once to float pairs (d8, 8 s8)) and
// read back as the block-diagonal A operand; off-diagonal lanes read a zero
// area.  The KS partial tiles are summed in LDS at the end.
namespace q4p {
template <int T, int WR, int KS, int S, int MP>
struct Cfg {
  static constexpr int kWaves = WR * KS;
  static constexpr int kRpa = 16 / S;               // activation rows per 1 KB piece
  // activation code pieces per chunk (one piece, its rows repeating row 0,
  // when the rows are fewer than a piece holds)
  static constexpr int kAi = MP >= kRpa ? MP / kRpa : 1;
  static constexpr int kAp = kAi + 1;               // ... plus one scale piece
  static constexpr int kApw = (kAp + WR - 1) / WR;  // activation loads per wave
  static constexpr int kNd = S * MP / 4;            // lanes loading d8 (and as many s8)
  static constexpr int kNab = WR > 1 ? 2 : 1;       // activation buffers per slice
  static constexpr int kAsOff = kAi * 1024;         // float (d8, 8 s8)[2S][8]
  static constexpr int kAst = kAsOff + 2 * S * 8 * 8;
  static constexpr int kZeroOff = KS * kNab * kAst;   // 1 KB of zeros
  static constexpr int kRed = KS > 1 ? kWaves * T * kWave * 16 : 0;
  static constexpr int kLds = kZeroOff + 1024 > kRed ? kZeroOff + 1024 : kRed;
  static_assert(S == 4 || S == 8, "chunk steps");
  static_assert(MP == 1 || MP == 2 || MP == 4 || MP == 8, "padded activation rows");
  static_assert(2 * kNd <= 64, "one load per chunk for each kind of scale");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};
}  // namespace q4p

template <int T, int S, int APW, int FMT>
struct Q4pChunk {
  uint4_t c[T][S / 2];                                      // codes, two steps per load
  std::conditional_t<S == 8, uint4_t, uint2_t> s[T];        // Q4_0: 2 scale bytes per step
  // Q4_K: a 16-byte header per 4 steps; IQ4_XS: an 8-byte one
  std::conditional_t<FMT == kPkIQ4, uint2_t, uint4_t> h[FMT != kPkQ40 ? T : 1]
                                                        [FMT != kPkQ40 ? S / 4 : 1];
  uint4_t a[APW];                                           // activation pieces
};

// (No __restrict__ on the inputs: the issue fences below must be able to
// order their loads.)
template <int T, int WR, int KS, int S, int MP, int FMT = kPkQ40>
__global__ __launch_bounds__(64 * WR * KS) void mmvq_q4_0_packed_kernel(
    const uint8_t *wp, int N, int K, const int8_t *a_qs, const uint16_t *a_d,
    const uint16_t *a_s, int M, float *y) {
  using C = q4p::Cfg<T, WR, KS, S, MP>;
  using R = Q4pChunk<T, S, C::kApw, FMT>;
  const std::conditional_t<FMT == kPkIQ4, Iq4Regs, PkNoRegs> kr{};
  extern __shared__ uint4_t smem4[];
  uint8_t *smem = reinterpret_cast<uint8_t *>(smem4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wr = wave % WR, ks = wave / WR;
  const int j = lane & 15, grp = lane >> 4;
  const int hb = grp >> 1, bh = grp & 1;
  const int U = (N + 15) >> 4, P = K >> 7, V = (K + 511) >> 9, nb = K >> 5;
  const int u0 = (blockIdx.x * WR + wr) * T;
  uint8_t *abuf = smem + ks * C::kNab * C::kAst;

  const int nct = K / (64 * S);
  const int cps = (nct + KS - 1) / KS;
  const int cb = ks * cps, ce = min(nct, cb + cps);

  // weight sources: tiles past the last repeat it (their rows are not stored)
  const uint8_t *cp[T];
  const uint8_t *sp[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const size_t u = (size_t)min(u0 + t, U - 1);
    cp[t] = wp + u * P * 1024 + 16 * lane;
    if constexpr (FMT == kPkQ4K)
      sp[t] = wp + (size_t)U * P * 1024 + u * (size_t)(K >> 8) * 256 + 16 * j;
    else if constexpr (FMT == kPkIQ4)
      sp[t] = wp + (size_t)U * P * 1024 + u * (size_t)(K >> 8) * 128 + 8 * j;
    else
      sp[t] = wp + (size_t)U * P * 1024 + u * V * 512 + 256 * hb + 16 * j;
  }
  // activation pieces of this wave: p = wr, wr + WR, ... (the last repeated);
  // pieces 0 .. kAi-1 are code blocks, piece kAi the scales (lanes [0, kNd)
  // d8, [kNd, 2 kNd) s8, 16-byte pieces of 8 blocks of row am)
  const int al = lane < 2 * C::kNd ? lane : 0;
  const bool asd = al < C::kNd;
  const int apc = (al % C::kNd) % (S / 4), am = (al % C::kNd) / (S / 4);
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
      asrc[a] = reinterpret_cast<const uint8_t *>((asd ? a_d : a_s) + (size_t)min(am, M - 1) * nb +
                                                  8 * apc);
    }
  }

  auto load = [&](int c, R &rg) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int e = 0; e < S / 2; ++e)
        rg.c[t][e] = load16_nt(cp[t] + (size_t)(c * (S / 2) + e) * 1024);
    // a chunk takes 2 S of the 16 scale bytes each lane holds per 8 steps:
    // the default cache policy keeps the rest of the line for the next chunk
    const int s0 = c * S;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (FMT == kPkQ4K) {
#pragma unroll
        for (int q = 0; q < S / 4; ++q) rg.h[t][q] = load16(sp[t] + (size_t)(c * (S / 4) + q) * 256);
      } else if constexpr (FMT == kPkIQ4) {
#pragma unroll
        for (int q = 0; q < S / 4; ++q) rg.h[t][q] = load8(sp[t] + (size_t)(c * (S / 4) + q) * 128);
      } else {
        const uint8_t *p = sp[t] + (size_t)(s0 >> 3) * 512 + 2 * (s0 & 7);
        if constexpr (S == 8) rg.s[t] = load16(p);
        else rg.s[t] = load8(p);
      }
    }
#pragma unroll
    for (int a = 0; a < C::kApw; ++a)
      rg.a[a] = load16(asrc[a] + (size_t)c * (apiece[a] < C::kAi ? 64 * S : 4 * S));
    issue_fence();   // keep each chunk's loads together and ahead of later work
  };
  auto store_act = [&](const R &rg, uint8_t *ab) {
#pragma unroll
    for (int a = 0; a < C::kApw; ++a) {
      if (apiece[a] < C::kAi) {
        *reinterpret_cast<uint4_t *>(ab + 1024 * apiece[a] + 16 * lane) = rg.a[a];
      } else if (lane < 2 * C::kNd) {
        // 8 blocks of row am: float d8 at slot 0, 8 * s8 at slot 1
        float *as = reinterpret_cast<float *>(ab + C::kAsOff) + 2 * am + (asd ? 0 : 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = f16_bits_to_f32((uint16_t)(rg.a[a][e >> 1] >> (16 * (e & 1))));
          as[16 * (8 * apc + e)] = asd ? v : 8.0f * v;
        }
      }
    }
  };

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  // A operand sources: row m = j % 8 of block h = j / 8, live when h == g / 2;
  // both 8-byte pieces advance by a fixed stride per step
  const int m = j & (MP - 1) & 7, ablk = m / C::kRpa;
  const bool live = (j >> 3) == hb;
  const int abase = 1024 * ablk + 8 * bh + 16 * (m % C::kRpa);
  const int alo = abase + 16 * C::kRpa * ((2 * hb) ^ ablk);
  const int ahi = abase + 16 * C::kRpa * ((2 * hb + 1) ^ ablk);
  const uint8_t *zero = smem + C::kZeroOff;
  constexpr int kAStride = 64 * C::kRpa;                   // bytes per step (4 columns)
  static_assert(kAStride * (S - 1) + 16 <= 1024, "zero area covers the chunk");
  // The chunk's integer block dots come first, so the matrix-core latency
  // overlaps the following reads; the float epilogues follow.
  auto consume = [&](const uint8_t *ab, const R &rg) {
    const uint8_t *blo = live ? ab + alo : zero;
    const uint8_t *bhi = live ? ab + ahi : zero + 8;
    int4_t isum[S][T];
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const uint2_t lo = *reinterpret_cast<const uint2_t *>(blo + kAStride * st);
      const uint2_t hi = *reinterpret_cast<const uint2_t *>(bhi + kAStride * st);
      const int4_t aop = {(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint4_t &w2 = rg.c[t][st >> 1];
        const uint2_t wq = {w2[2 * (st & 1)], w2[2 * (st & 1) + 1]};
        if constexpr (FMT == kPkIQ4)
          isum[st][t] = iq4_mfma_isum(wq, aop, kr);
        else
          isum[st][t] = q4_mfma_isum(wq, aop);
      }
    }
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const int bl = 2 * st + hb;                          // this lane's block in the chunk
      const float4_t *asf = reinterpret_cast<const float4_t *>(ab + C::kAsOff + 64 * bl + 32 * bh);
      const float4_t sa = asf[0], sb = asf[1];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        if constexpr (FMT == kPkIQ4) {
          // sub-block 2 (st % 4) + hb of the step's super-block
          iq4_mfma_epilogue(isum[st][t], iq4_scale(rg.h[t][st >> 2], 2 * (st & 3) + hb), sa, sb,
                            acc[t]);
        } else if constexpr (FMT == kPkQ4K) {
          // sub-block sj = 2 (st % 4) + hb of the step's super-block: scale
          // byte 4 + sj, min high bits in nibble hb of byte 12 + st % 4
          const uint4_t &h = rg.h[t][st >> 2];
          const uint32_t pb = (h[1 + ((st & 3) >> 1)] >> (8 * (2 * (st & 1) + hb))) & 255u;
          const uint32_t ph = (h[3] >> (8 * (st & 3) + 4 * hb)) & 15u;
          const float dsc = f16_bits_to_f32((uint16_t)(h[0] & 0xFFFFu)) * (float)(pb & 63u);
          const float dmm8 = f16_bits_to_f32((uint16_t)(h[0] >> 16)) *
                             (float)((pb >> 6) | (ph << 2)) * 0.125f;
          q4k_mfma_epilogue(isum[st][t], dsc, dmm8, sa, sb, acc[t]);
        } else {
          const uint32_t dw = rg.s[t][st >> 1] >> (16 * (st & 1));
          q4_mfma_epilogue(isum[st][t], f16_bits_to_f32((uint16_t)dw), sa, sb, acc[t]);
        }
      }
    }
  };

  // One chunk: issue the next chunk's loads (LOAD), stage this chunk's
  // activations, and consume it.  Waves that share activations run cps
  // chunks in lockstep (the barrier); chunks past a slice's end re-read its
  // last chunk and compute nothing.  The last chunk issues no loads.
  *reinterpret_cast<uint4_t *>(smem + C::kZeroOff + 16 * lane) = uint4_t{0u, 0u, 0u, 0u};
  const int steps = WR > 1 ? cps : ce - cb;
  const int cl = max(ce - 1, 0);
  auto chunk = [&](int k, R &cur, R &nxt, auto load_next) {
    const int c = cb + k;
    if constexpr (decltype(load_next)::value) load(min(c + 1, cl), nxt);
    uint8_t *ab = abuf + (k & (C::kNab - 1)) * C::kAst;
    store_act(cur, ab);
    if constexpr (WR > 1) wg_barrier();
    if (c < ce) consume(ab, cur);
  };
  if (steps > 0) {
    R ra, rb;
    load(min(cb, cl), ra);
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
  // lanes l and l ^ 32 hold the two blocks of each step: add them
  if (ks == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float4_t v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = add_swap32(acc[t][r]);
      const int n = 16 * (u0 + t) + j;
      if (lane < 32 && n < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mm = 4 * bh + r;
          if (mm < M) y[(size_t)mm * N + n] = v[r];
        }
      }
    }
  }
}

template <int T, int WR, int KS, int S, int MP, int FMT = kPkQ40>
static hipError_t launch_q4p_cfg(const uint8_t *wp, int N, int K, const int8_t *a_qs,
                                 const uint16_t *a_d, const uint16_t *a_s, int M, float *y,
                                 hipStream_t stream) {
  using C = q4p::Cfg<T, WR, KS, S, MP>;
  if (K % (64 * S) != 0) return hipErrorInvalidValue;   // chunks must tile K
  const hipError_t lds_ok =
      allow_lds((const void *)mmvq_q4_0_packed_kernel<T, WR, KS, S, MP, FMT>, C::kLds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int tiles = (N + 15) / 16;
  const int blocks = (tiles + T * WR - 1) / (T * WR);
  hipLaunchKernelGGL((mmvq_q4_0_packed_kernel<T, WR, KS, S, MP, FMT>), dim3(blocks),
                     dim3(64 * C::kWaves), C::kLds, stream, wp, N, K, a_qs, a_d, a_s, M, y);
  return hipGetLastError();
}

// Tiles per wave T, waves sharing activations WR, K slices KS and chunk
// steps S, measured on MI355X over every configuration on 14 matrices (K
// 2048..14336, N 4096..32000; weights rotating over > 2 GiB) at M = 1, 2, 4,
// 6 and 8; each row is within a few percent of the best on the matrices it
// covers.  Chunks of 8 steps need K % 512 == 0 (s8).  Wide matrices want
// two waves sharing each activation chunk and no split; mid-width ones a
// K split of 2 (with sharing at M >= 5); narrower ones a split of 4 (two
// tiles per wave at M >= 5, and at M = 3, 4 on rows of 8192 or more); up to
// 256 tiles a split of 8.
template <int MP, int FMT>
static hipError_t launch_q4p_mp(const uint8_t *wp, int N, int K, const int8_t *a_qs,
                                const uint16_t *a_d, const uint16_t *a_s, int M, float *y,
                                hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s8 = K % 512 == 0;
#define SKINNY_Q4P(T, WR, KS, S) \
  return launch_q4p_cfg<T, WR, KS, S, MP, FMT>(wp, N, K, a_qs, a_d, a_s, M, y, stream)
  if constexpr (FMT != kPkQ40) {
    // Q4_K: its per-step header decode makes chunks of 4 steps pay at every
    // width (measured on the Qwen3-8B projections and six more matrices at
    // M = 1, 4, 5, 8: 4096 x 24576 at M = 8 15.2 -> 14.1 us against the
    // Q4_0 rows, 4096 x 16384 11.7 -> 10.7 us); IQ4_XS, with its table
    // decode per step, takes the same rows except on wide matrices, where
    // two K slices without activation sharing lead (measured over 14
    // configurations at M = 4, 6, 8 on six matrices: 4096 x 24576 at M = 4
    // 15.4 -> 13.5 us, at M = 8 15.7 -> 15.2 us)
    if (tiles >= 1100) {
      if constexpr (FMT == kPkIQ4) SKINNY_Q4P(1, 1, 2, 4);
      SKINNY_Q4P(1, 2, 2, 4);
    }
    if (tiles >= 800) SKINNY_Q4P(1, 2, 4, 4);
    if (tiles > 256) SKINNY_Q4P(1, 1, 4, 4);
    SKINNY_Q4P(1, 1, 8, 4);
  }
  if (tiles >= 1100) {
    if (s8 && MP >= 4) SKINNY_Q4P(1, 2, 1, 8);
    SKINNY_Q4P(1, 2, 1, 4);
  }
  if (tiles >= 800) {
    if (MP == 8) {
      if (s8) SKINNY_Q4P(1, 2, 2, 8);
      SKINNY_Q4P(1, 2, 2, 4);
    }
    SKINNY_Q4P(1, 1, 2, 4);
  }
  if (tiles >= 512) SKINNY_Q4P(1, 1, 4, 4);
  if (tiles > 256) {
    if (MP == 8) {
      if (s8 && K >= 8192) SKINNY_Q4P(2, 1, 4, 8);
      SKINNY_Q4P(2, 1, 4, 4);
    }
    if (MP == 4 && s8 && K >= 8192) SKINNY_Q4P(2, 1, 4, 8);
    SKINNY_Q4P(1, 1, 4, 4);
  }
  SKINNY_Q4P(1, 1, 8, 4);
#undef SKINNY_Q4P
}

hipError_t launch_mmvq_q4_0_packed(const uint8_t *wp, int N, int K, const int8_t *a_qs,
                                   const uint16_t *a_d, const uint16_t *a_s, int M, float *y,
                                   hipStream_t stream) {
  if (M <= 1) return launch_q4p_mp<1, kPkQ40>(wp, N, K, a_qs, a_d, a_s, M, y, stream);
  if (M <= 2) return launch_q4p_mp<2, kPkQ40>(wp, N, K, a_qs, a_d, a_s, M, y, stream);
  if (M <= 4) return launch_q4p_mp<4, kPkQ40>(wp, N, K, a_qs, a_d, a_s, M, y, stream);
  return launch_q4p_mp<8, kPkQ40>(wp, N, K, a_qs, a_d, a_s, M, y, stream);
}

hipError_t launch_mmvq_q4_k_packed(const uint8_t *wp, int N, int K, const int8_t *a_qs,
                                   const uint16_t *a_d, const uint16_t *a_s, int M, float *y,
                                   hipStream_t stream) {
  if (M <= 1) return launch_q4p_mp<1, kPkQ4K>(wp, N, K, a_qs, a_d, a_s, M, y, stream);
  if (M <= 2) return launch_q4p_mp<2, kPkQ4K>(wp, N, K, a_qs, a_d, a_s, M, y, stream);
  if (M <= 4) return launch_q4p_mp<4, kPkQ4K>(wp, N, K, a_qs, a_d, a_s, M, y, stream);
  return launch_q4p_mp<8, kPkQ4K>(wp, N, K, a_qs, a_d, a_s, M, y, stream);
}

// IQ4_XS on the packed kernel: the Q8_1 sum term is not used, so d8 stands
// in for it in the staging.
hipError_t launch_mmvq_iq4_xs_packed(const uint8_t *wp, int N, int K, const int8_t *a_qs,
                                     const uint16_t *a_d, int M, float *y, hipStream_t stream) {
  if (M <= 1) return launch_q4p_mp<1, kPkIQ4>(wp, N, K, a_qs, a_d, a_d, M, y, stream);
  if (M <= 2) return launch_q4p_mp<2, kPkIQ4>(wp, N, K, a_qs, a_d, a_d, M, y, stream);
  if (M <= 4) return launch_q4p_mp<4, kPkIQ4>(wp, N, K, a_qs, a_d, a_d, M, y, stream);
  return launch_q4p_mp<8, kPkIQ4>(wp, N, K, a_qs, a_d, a_d, M, y, stream);
}

// ------------------------------------------------------------------ prepack

// One thread per 16 packed bytes, grid-stride over both planes: codes
// pieces first (a lane's two 8-byte halves), then scale pieces (Q4_0: the 16
// bytes at 256 h + 16 j of a scale block; Q4_K: one row's header; IQ4_XS:
// the headers of two consecutive rows).
constexpr size_t q4p_scale_pieces(int FMT, size_t U, size_t V, size_t nsb) {
  return FMT == kPkQ4K ? U * nsb * 16 : FMT == kPkIQ4 ? U * nsb * 8 : U * V * 32;
}

template <int FMT>
__global__ __launch_bounds__(256) void prepack_q4_0_kernel(
    const uint8_t *__restrict__ w_qs, const uint8_t *__restrict__ scl, int N, int K,
    uint8_t *__restrict__ wp) {
  const size_t U = (size_t)(N + 15) / 16, P = (size_t)K / 128, V = ((size_t)K + 511) / 512;
  const size_t nb = (size_t)K / 32, nsb = (size_t)K / 256;
  const size_t nc = U * P * 64, total = nc + q4p_scale_pieces(FMT, U, V, nsb);
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (size_t)gridDim.x * blockDim.x) {
    uint4_t v = uint4_t{0u, 0u, 0u, 0u};
    if (q < nc) {
      const int l = (int)(q & 63), jj = l & 15, g = l >> 4, h = g >> 1, b = g & 1;
      const size_t blk = q >> 6, u = blk / P, p = blk - u * P;
      const size_t row = 16 * u + jj;
      if (row < (size_t)N) {
        const uint8_t *src = w_qs + row * (nb * 16) + 8 * b;
        const uint2_t e0 = load8(src + 16 * (4 * p + h));
        const uint2_t e1 = load8(src + 16 * (4 * p + 2 + h));
        v = uint4_t{e0.x, e0.y, e1.x, e1.y};
      }
    } else if constexpr (FMT == kPkQ4K) {
      const size_t r = q - nc, blk = r >> 4, u = blk / nsb, sb = blk - u * nsb;
      const size_t row = 16 * u + (r & 15);
      if (row < (size_t)N) v = load16(scl + row * (nsb * 16) + 16 * sb);
    } else if constexpr (FMT == kPkIQ4) {
      const size_t r = q - nc, blk = r >> 3, u = blk / nsb, sb = blk - u * nsb;
      const size_t row = 16 * u + 2 * (r & 7);
      if (row < (size_t)N) {
        const uint2_t h0 = load8(scl + row * (nsb * 8) + 8 * sb);
        v[0] = h0.x;
        v[1] = h0.y;
      }
      if (row + 1 < (size_t)N) {
        const uint2_t h1 = load8(scl + (row + 1) * (nsb * 8) + 8 * sb);
        v[2] = h1.x;
        v[3] = h1.y;
      }
    } else {
      const uint16_t *w_d = reinterpret_cast<const uint16_t *>(scl);
      const size_t r = q - nc, blk = r >> 5, u = blk / V, vb = blk - u * V;
      const int piece = (int)(r & 31), h = piece >> 4, jj = piece & 15;
      const size_t row = 16 * u + jj;
      if (row < (size_t)N) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const size_t b = 16 * vb + 2 * t + h;
          if (b < nb) v[t >> 1] |= (uint32_t)w_d[row * nb + b] << (16 * (t & 1));
        }
      }
    }
    *reinterpret_cast<uint4_t *>(wp + 16 * q) = v;
  }
}

template <int FMT>
static hipError_t launch_prepack(const uint8_t *w_qs, const uint8_t *scl, int N, int K,
                                 uint8_t *wp, hipStream_t stream) {
  const size_t U = (size_t)(N + 15) / 16, P = (size_t)K / 128, V = ((size_t)K + 511) / 512;
  const size_t total = U * P * 64 + q4p_scale_pieces(FMT, U, V, (size_t)K / 256);
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(prepack_q4_0_kernel<FMT>, dim3((unsigned)blocks), dim3(256), 0, stream, w_qs,
                     scl, N, K, wp);
  return hipGetLastError();
}

hipError_t launch_prepack_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                               uint8_t *wp, hipStream_t stream) {
  return launch_prepack<kPkQ40>(w_qs, reinterpret_cast<const uint8_t *>(w_d), N, K, wp, stream);
}

hipError_t launch_prepack_q4_k(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                               uint8_t *wp, hipStream_t stream) {
  return launch_prepack<kPkQ4K>(w_qs, w_hdr, N, K, wp, stream);
}

hipError_t launch_prepack_iq4_xs(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                 uint8_t *wp, hipStream_t stream) {
  return launch_prepack<kPkIQ4>(w_qs, w_hdr, N, K, wp, stream);
}

}  // namespace skinny
