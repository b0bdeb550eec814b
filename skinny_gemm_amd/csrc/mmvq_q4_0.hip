// mmvq_q4_0.hip -- Q4_0 weights x Q8_1 activations, M = 1..8 rows.
//
// "Machine Learning on NVIDIA CMP" ("llama.cpp results", "The DP2A patch"):
// decode is a quantized mat x vec whose inner loop is a 4-way int8 dot with
// int32 accumulation; any rewrite must stay bit-exact integer arithmetic.
// gfx950 has that dot at full rate (v_dot4_i32_i8), so the block sum is
//   isum = sum_{i<32} code_i * q8_i       (8 x v_dot4, codes 0..15 as int8)
// and the -8 offset of every weight is applied once per block through the
// Q8_1 sum term:  acc += d4 * (d8 * isum - 8 * s8).
//
// Mapping (one wave = R weight rows, full K):
//   * lane l takes blocks b = l, l + 64, ...: each weight load is one
//     128-bit load per lane, 1 KB contiguous per wave and row; each block's
//     16 code bytes unpack to two words of four codes per 32-bit word with
//     one AND and one shift+AND;
//   * the lane's Q8_1 block (M x 32 codes, d8, s8) is loaded once and reused
//     for all R rows, so activation bytes per weight byte are 2M/R;
//   * after the K loop every lane holds R*M partial sums, combined by a
//     transposing butterfly (permlane swaps, DPP, swizzle) that leaves one
//     finished output per lane; no atomics, fully deterministic.
// Bytes per call: N*K*(1/2 + 2/32) weights + M*K*(1 + 4/32) activations +
// 4*M*N output.
#include <type_traits>

#include "device.h"
#include "q4_mfma.h"
#include "launch.h"
#include "q8_1.h"
#include "skinny_gemm.h"

namespace skinny {

// Activation rows from which the matrix-core kernel is used, and below
// which the vector kernel keeps small, short matrices (measured on MI355X:
// at M <= 4 it wins only for N <= 8191 with K < 8192).
constexpr int kQ4MfmaMinM = 3;
constexpr int kQ4VectorMaxM = 4;

constexpr int next_pow2(int v) { return v <= 1 ? 1 : 2 * next_pow2((v + 1) / 2); }

// (No __restrict__ on the inputs: the issue fence below must be able to
// keep a round's loads ahead of its arithmetic.)
//
// KS > 1 splits K: the KS waves w, w + 1, .. of a group take the same R rows
// and consecutive slices of ceil(nb / KS) blocks, and the group's first wave
// adds the others' reduced sums (in slice order, so results repeat bit for
// bit) and stores.  Long rows then take one memory round per wave instead
// of several.
template <int M, int R, int U, bool NT, int KS = 1>
__global__ __launch_bounds__(256) void mmvq_q4_0_kernel(
    const uint8_t *w_qs, const uint16_t *w_d, int N, int K, const int8_t *a_qs,
    const uint16_t *a_d, const uint16_t *a_s, float *y) {
  static_assert(KS == 1 || KS == 2 || KS == 4, "K slices per row group");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ks = wave % KS;
  const int n0 = (blockIdx.x * (4 / KS) + wave / KS) * R;
  if (KS == 1 && n0 >= N) return;   // with KS > 1 every wave meets the barrier below
  const int nb = K >> 5;
  const int nbs = (nb + KS - 1) / KS;
  const int bb = ks * nbs, be = min(nb, bb + nbs);   // this wave's blocks [bb, be)

  const uint8_t *wrow[R];
  const uint16_t *drow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(n0 + r, N - 1);          // ragged tail: recompute the last row
    wrow[r] = w_qs + (size_t)n * (size_t)(K >> 1);
    drow[r] = w_d + (size_t)n * (size_t)nb;
  }

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  // U blocks per lane per round, all loaded before any is used, so a row of
  // up to 64 U blocks costs one memory round trip.  Blocks past the slice
  // end load block be - 1 again and are not accumulated.
  for (int b0 = bb + lane; b0 < be; b0 += U * kWave) {
    uint4_t wq[U][R];
    uint16_t d4h[U][R];
    uint4_t aq0[U][M], aq1[U][M];
    uint16_t d8h[U][M], s8h[U][M];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = min(b0 + u * kWave, be - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wq[u][r] = NT ? load16_nt(wrow[r] + 16 * b) : load16(wrow[r] + 16 * b);
        d4h[u][r] = NT ? load_u16_nt(drow[r] + b) : drow[r][b];
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int8_t *ap = a_qs + (size_t)m * K + 32 * b;
        aq0[u][m] = load16(ap);
        aq1[u][m] = load16(ap + 16);
        d8h[u][m] = a_d[(size_t)m * nb + b];
        s8h[u][m] = a_s[(size_t)m * nb + b];
      }
    }
    issue_all();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = b0 + u * kWave < be;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // low nibbles = codes 0..15 of the block, high nibbles = codes 16..31
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo[i] = wq[u][r][i] & 0x0F0F0F0Fu;
          hi[i] = (wq[u][r][i] >> 4) & 0x0F0F0F0Fu;
        }
        const float d4 = f16_bits_to_f32(d4h[u][r]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          int32_t isum = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            isum = dot4_i8(lo[i], aq0[u][m][i], isum);
            isum = dot4_i8(hi[i], aq1[u][m][i], isum);
          }
          const float t = fmaf(f16_bits_to_f32(d8h[u][m]), (float)isum,
                               -8.0f * f16_bits_to_f32(s8h[u][m]));
          const float a = fmaf(d4, t, acc[r][m]);
          acc[r][m] = live ? a : acc[r][m];
        }
      }
    }
  }

  constexpr int V = next_pow2(R * M);
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = (i < R * M) ? acc[i / M][i % M] : 0.0f;
  float total = wave_reduce_transpose<V>(v, lane);
  if constexpr (KS > 1) {
    __shared__ float part[4][kWave];
    part[wave][lane] = total;
    wg_barrier();
    if (ks != 0) return;
#pragma unroll
    for (int v2 = 1; v2 < KS; ++v2) total += part[wave + v2][lane];
  }
  constexpr int SHIFT = 6 - Log2<V>::value;
  const int idx = lane >> SHIFT;
  if ((lane & ((1 << SHIFT) - 1)) == 0 && idx < R * M) {
    const int r = idx / M, m = idx % M;
    const int n = n0 + r;
    if (n < N) y[(size_t)m * N + n] = total;
  }
}

// Matrix-core variant for wider M.  One v_mfma_i32_16x16x64_i8 computes the
// exact int32 block sums of 16 weight rows x 2 blocks x 8 activation rows
// (one 64-element step).  K slot g (lane group l / 16) of a step covers
// block 2s + g/2, bytes 8(g%2) .. 8(g%2)+7 of its 16 code bytes, i.e.
// elements 8(g%2) + 0..7 (low nibbles) and 16 + 8(g%2) + 0..7 (high
// nibbles):
//   * B operand (columns = weight rows): lane (j = l % 16, g) takes those 8
//     bytes of row 16t + j and splits them into 16 codes with two ANDs and
//     two shift+ANDs;
//   * A operand (rows a = 8h + m): block-diagonal, so a row only meets the
//     K slots of its own block h -- lane (j, g) holds the matching 16 Q8_1
//     codes of row m = j % 8 when j / 8 == g / 2, else zeros (read from a
//     zero area of LDS); rows m >= M repeat row M - 1 and are dropped;
//   * lane l then owns isum for weight row 16t + l%16, block 2s + g/2 and
//     activation rows 4(g%2) .. 4(g%2)+3, and applies the float32 block
//     epilogue acc += d4 * (d8 * isum - 8 * s8).
// Data movement.  A workgroup is WR x KS waves: WR waves own different
// tiles (T each) and share one K slice, KS slices split K.  K is walked in
// chunks of S steps.  Every wave reads its own weight codes and scales, and
// a 1/WR share of the slice's activation chunk (Q8_1 codes and scales),
// with 128-bit loads in row-contiguous order into registers, D chunks ahead
// of their use; registers, not LDS, hold the bytes in flight.  When a
// chunk's turn comes its weights are written to a wave-private LDS buffer
// and its activation share to a double-buffered buffer of the slice
// (activation scales converted once to float pairs (d8, 8 s8)); one barrier
// later every wave reads both back in the operand layout.  LDS blocks are
// 1 KB as written by one store instruction, their 16-byte columns
// XOR-swizzled so the operand-layout reads hit distinct banks.  Loads are
// issued in the order they are consumed, so each wait covers one chunk.
// The KS partial tiles are summed in LDS.
namespace q4 {
template <int T, int WR, int KS, int S, int MP, int WSB = 4>
struct Cfg {
  static constexpr int kWaves = WR * KS;
  static constexpr int kRows = 16 * T;              // weight rows per wave
  static constexpr int kCB = 32 * S;                // code bytes per row per chunk
  static constexpr int kRpi = 1024 / kCB;           // code rows per 1 KB block
  static constexpr int kSwz = S / 2 - 1;            // code column swizzle mask
  static constexpr int kCi = kRows / kRpi;          // code loads per chunk
  static constexpr int kWsB = kRows * WSB * S;      // weight-scale bytes per chunk
  static constexpr int kWst = kCi * 1024 + kWsB;    // wave weight buffer
  static constexpr int kRpa = 16 / S;               // activation rows per 1 KB block
  static constexpr int kAi = MP / kRpa;             // activation code loads per chunk
  static constexpr int kAp = kAi + 1;               // ... plus one scale load
  static constexpr int kApw = (kAp + WR - 1) / WR;  // activation loads per wave
  static constexpr int kNd = S * MP / 4;            // lanes loading d8 (and as many s8)
  static constexpr int kAsOff = kAi * 1024;         // float (d8, 8 s8)[2S][8]
  static constexpr int kAst = kAsOff + 2 * S * 8 * 8;   // activation buffer
  static constexpr int kActBase = kWaves * kWst;
  static constexpr int kZeroOff = kActBase + KS * 2 * kAst;  // 1 KB of zeros
  static constexpr int kLds = kZeroOff + 1024;
  static_assert(S == 4 || S == 8, "chunk steps");
  static_assert(MP == 4 || MP == 8, "padded activation rows");
  static_assert(kWsB <= 1024 && 2 * kNd <= 64, "one load per chunk for each kind of scale");
  static_assert(kWaves * T * kWave * 16 <= kActBase, "reduction buffer");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};
template <int T, int S, int APW>
struct Chunk {
  uint4_t c[T * S / 2];
  uint4_t ws;
  uint4_t a[APW];
};
}  // namespace q4

// (No __restrict__ on the inputs: the issue fence below must be able to
// order their loads.)
//
// FMT selects the weight format.  kFmtQ4K: Q4_K weights, the same 4-bit
// codes, and in place of the block scales w_d a header array of the same
// geometry (K/16 bytes per row: one 16-byte header {d, dmin, 12 scale/min
// bytes} per 8 blocks), so staging is unchanged and only the epilogue
// decodes the lane's sub-block scale and min.  kFmtIQ4: IQ4_XS weights, the
// 4-bit indices in the same nibble order decoded through the IQ4_NL table
// into signed int8 operands, and an 8-byte header {d, H, L} per 8 blocks
// (K/32 bytes per row: 16 bytes per row per 8-step chunk, loaded like the
// Q4_0 scales, or 8 bytes per 4-step chunk, one lane per row).
constexpr int kFmtQ40 = 0, kFmtQ4K = 1, kFmtIQ4 = 2;
struct NoRegs {};

template <int T, int WR, int KS, int S, int MP, int D, int FMT = kFmtQ40>
__global__ __launch_bounds__(64 * WR * KS) void mmvq_q4_0_mfma_kernel(
    const uint8_t *w_qs, const uint16_t *w_d, int N, int K, const int8_t *a_qs,
    const uint16_t *a_d, const uint16_t *a_s, int M, float *y) {
  constexpr int kWsb = FMT == kFmtIQ4 ? 2 : 4;   // scale bytes per row per step
  // IQ4_XS chunks of 4 steps take one 8-byte header per row, one lane per row
  constexpr bool kHdr8 = FMT == kFmtIQ4 && S == 4;
  using C = q4::Cfg<T, WR, KS, S, MP, kWsb>;
  using R = q4::Chunk<T, S, C::kApw>;
  static_assert(D == 1 || D == 2, "chunks in flight");
  extern __shared__ uint4_t smem4[];
  uint8_t *smem = reinterpret_cast<uint8_t *>(smem4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wr = wave % WR, ks = wave / WR;
  const int j = lane & 15, grp = lane >> 4;
  const int hb = grp >> 1, bh = grp & 1;
  const int n0 = blockIdx.x * (C::kRows * WR) + C::kRows * wr;
  const int nb = K >> 5;
  uint8_t *wbuf = smem + wave * C::kWst;
  uint8_t *abuf = smem + C::kActBase + ks * 2 * C::kAst;

  const int nct = K / (64 * S);
  const int cps = (nct + KS - 1) / KS;
  const int cb = ks * cps, ce = min(nct, cb + cps);

  // weight sources (chunk 0)
  const uint8_t *csrc[C::kCi];
#pragma unroll
  for (int q = 0; q < C::kCi; ++q) {
    const int r = q * C::kRpi + (lane % C::kRpi);
    const int col = (lane / C::kRpi) ^ (q & C::kSwz);
    csrc[q] = w_qs + (size_t)min(n0 + r, N - 1) * (size_t)(K >> 1) + 16 * col;
  }
  const bool wsact = kHdr8 ? lane < C::kRows : lane < C::kWsB / 16;
  const int wl = lane % (kHdr8 ? C::kRows : C::kWsB / 16);   // lanes past them repeat one
  const uint8_t *wssrc = reinterpret_cast<const uint8_t *>(w_d) +
                         (size_t)min(n0 + wl % C::kRows, N - 1) * (size_t)(kWsb * (K >> 6)) +
                         (kHdr8 ? 0 : 16 * (wl / C::kRows));
  const std::conditional_t<FMT == kFmtIQ4, Iq4Regs, NoRegs> kr{};
  // activation pieces of this wave: p = wr, wr + WR, ... (the last repeated);
  // pieces 0 .. kAi-1 are code blocks, piece kAi the scales (lanes [0, kNd)
  // d8, [kNd, 2 kNd) s8, 16-byte pieces of 8 blocks of row am)
  const int al = lane < 2 * C::kNd ? lane : 0;
  const bool asd = al < C::kNd;
  const int apc = (al % C::kNd) % (S / 4), am = (al % C::kNd) / (S / 4);
  const uint8_t *asrc[C::kApw];
  int apiece[C::kApw];
#pragma unroll
  for (int u = 0; u < C::kApw; ++u) {
    const int p = min(wr + WR * u, C::kAp - 1);
    apiece[u] = p;
    if (p < C::kAi) {
      const int r = min(p * C::kRpa + (lane % C::kRpa), M - 1);
      const int col = (lane / C::kRpa) ^ p;
      asrc[u] = reinterpret_cast<const uint8_t *>(a_qs + (size_t)r * K + 16 * col);
    } else {
      asrc[u] = reinterpret_cast<const uint8_t *>((asd ? a_d : a_s) + (size_t)min(am, M - 1) * nb +
                                                  8 * apc);
    }
  }

  auto load = [&](int c, R &rg) {
#pragma unroll
    for (int q = 0; q < C::kCi; ++q) rg.c[q] = load16_nt(csrc[q] + (size_t)c * C::kCB);
    if constexpr (kHdr8) {
      const uint2_t h = load8_nt(wssrc + (size_t)c * 8);
      rg.ws = uint4_t{h.x, h.y, 0u, 0u};
    } else {
      rg.ws = load16_nt(wssrc + (size_t)c * (kWsb * S));
    }
#pragma unroll
    for (int u = 0; u < C::kApw; ++u)
      rg.a[u] = load16(asrc[u] + (size_t)c * (apiece[u] < C::kAi ? 64 * S : 4 * S));
    issue_fence();   // keep each chunk's loads together and ahead of later work
  };
  auto store = [&](const R &rg, uint8_t *ab) {
#pragma unroll
    for (int q = 0; q < C::kCi; ++q) *reinterpret_cast<uint4_t *>(wbuf + 1024 * q + 16 * lane) = rg.c[q];
    if constexpr (kHdr8) {
      if (wsact)
        *reinterpret_cast<uint2_t *>(wbuf + C::kCi * 1024 + 8 * lane) = uint2_t{rg.ws.x, rg.ws.y};
    } else {
      if (wsact) *reinterpret_cast<uint4_t *>(wbuf + C::kCi * 1024 + 16 * lane) = rg.ws;
    }
#pragma unroll
    for (int u = 0; u < C::kApw; ++u) {
      if (apiece[u] < C::kAi) {
        *reinterpret_cast<uint4_t *>(ab + 1024 * apiece[u] + 16 * lane) = rg.a[u];
      } else if (lane < 2 * C::kNd) {
        // 8 blocks of row am: float d8 at slot 0, 8 * s8 at slot 1
        float *as = reinterpret_cast<float *>(ab + C::kAsOff) + 2 * am + (asd ? 0 : 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = f16_bits_to_f32((uint16_t)(rg.a[u][e >> 1] >> (16 * (e & 1))));
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
  // The chunk's operand reads and integer block dots come first, so the
  // matrix-core latency overlaps the following reads; the float epilogues
  // follow.  Off-diagonal lanes read the zero area, whose 1 KB covers every
  // step's offset, so the choice is made once per chunk.
  static_assert(kAStride * (S - 1) + 16 <= 1024, "zero area covers the chunk");
  auto consume = [&](const uint8_t *ab) {
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
        const int r = 16 * t + j, q = r / C::kRpi;
        const int col = (2 * st + hb) ^ (q & C::kSwz);
        const uint2_t wq = *reinterpret_cast<const uint2_t *>(
            wbuf + 1024 * q + 16 * (C::kRpi * col + r % C::kRpi) + 8 * bh);
        if constexpr (FMT == kFmtIQ4)
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
        const int r = 16 * t + j;
        if constexpr (FMT == kFmtIQ4) {
          const uint2_t hd = *reinterpret_cast<const uint2_t *>(
              wbuf + C::kCi * 1024 + (kHdr8 ? 8 * r : 16 * r + 8 * (bl >> 3)));
          iq4_mfma_epilogue(isum[st][t], iq4_scale(hd, bl & 7), sa, sb, acc[t]);
        } else if constexpr (FMT == kFmtQ4K) {
          const uint8_t *h = wbuf + C::kCi * 1024 + 16 * ((bl >> 3) * C::kRows + r);
          const int sj = bl & 7;                           // sub-block in the super-block
          const uint32_t dd = *reinterpret_cast<const uint32_t *>(h);
          const uint32_t pb = h[4 + sj], ph = h[12 + (sj >> 1)];
          const uint32_t sc = pb & 63u;
          const uint32_t mn = (pb >> 6) | (((ph >> (4 * (sj & 1))) & 15u) << 2);
          const float dsc = f16_bits_to_f32((uint16_t)(dd & 0xFFFFu)) * (float)sc;
          const float dmm8 = f16_bits_to_f32((uint16_t)(dd >> 16)) * (float)mn * 0.125f;
          q4k_mfma_epilogue(isum[st][t], dsc, dmm8, sa, sb, acc[t]);
        } else {
          const float d4 = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(
              wbuf + C::kCi * 1024 + 16 * ((bl >> 3) * C::kRows + r) + 2 * (bl & 7)));
          q4_mfma_epilogue(isum[st][t], d4, sa, sb, acc[t]);
        }
      }
    }
  };

  // Every wave runs cps steps in lockstep (the barrier); steps past its
  // slice load the slice's last chunk again and compute nothing, so every
  // path issues the same loads.
  if (cb < ce || WR * KS > 1) {
    *reinterpret_cast<uint4_t *>(smem + C::kZeroOff + 16 * lane) = uint4_t{0u, 0u, 0u, 0u};
    const int cl = max(ce - 1, 0);                       // a valid chunk to re-read
    auto step = [&](int k, R &rg) {
      const int c = cb + k;
      uint8_t *ab = abuf + (k & 1) * C::kAst;
      store(rg, ab);
      if constexpr (WR > 1) wg_barrier();
      load(min(c + D, cl), rg);
      if (c < ce) consume(ab);
    };
    if constexpr (D == 1) {
      R r0;
      load(min(cb, cl), r0);
      for (int k = 0; k < cps; ++k) step(k, r0);
    } else {
      R r0, r1;
      load(min(cb, cl), r0);
      load(min(cb + 1, cl), r1);
      for (int k = 0; k < cps; k += 2) {
        step(k, r0);
        step(k + 1, r1);
      }
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
      const int n = n0 + 16 * t + j;
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

template <int T, int WR, int KS, int S, int MP, int D, int FMT>
static hipError_t launch_mfma_cfg(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                                  const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                  int M, float *y, hipStream_t stream) {
  using C = q4::Cfg<T, WR, KS, S, MP, FMT == kFmtIQ4 ? 2 : 4>;
  if (K % (64 * S) != 0) return hipErrorInvalidValue;   // chunks must tile K
  const hipError_t lds_ok =
      allow_lds((const void *)mmvq_q4_0_mfma_kernel<T, WR, KS, S, MP, D, FMT>, C::kLds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int rows = C::kRows * WR;
  const int blocks = (N + rows - 1) / rows;
  hipLaunchKernelGGL((mmvq_q4_0_mfma_kernel<T, WR, KS, S, MP, D, FMT>), dim3(blocks),
                     dim3(64 * C::kWaves), C::kLds, stream, w_qs, w_d, N, K, a_qs, a_d, a_s,
                     M, y);
  return hipGetLastError();
}

// One tile per wave throughout.  Wide matrices share each activation chunk
// between two (>= 1100 tiles) or four (>= 1800 tiles) waves; narrower ones
// split K instead so that enough waves stream, and from 800 tiles both.
// Measured on MI355X at M = 6 and 8 over every configuration, with weights
// rotating over > 2 GiB: 2000 tiles (4096 x 32000) four-way sharing, 1376
// and 1536 two-way, 864-1024 tiles two-way sharing with a two-way split
// (4096 x 16384 at M = 8 12.8 -> 11.4 us, 5120 x 13824 15.3 -> 13.3 us), 512
// to 768 a two-way split; below 512 tiles a two-way split of 8-step chunks
// on rows up to K = 8191 (7168 x 7168 at M = 8 15.7 -> 11.8 us, 5120 x 5120
// 12.4 -> 9.3 us), two tiles per wave with a four-way split on longer rows
// (13824 x 5120 23.9 -> 17.6 us), four-way below 256 tiles; chunks of 4
// steps (K % 512 == 256) keep the eight-way split there.  Q4_K has rows of
// its own below 1100 tiles.
template <int MP, int FMT>
static hipError_t launch_mfma_mp(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                                 const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                 int M, float *y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s8 = K % 512 == 0;
#define SKINNY_Q4(T, WR, KS, S) \
  return launch_mfma_cfg<T, WR, KS, S, MP, 1, FMT>(w_qs, w_d, N, K, a_qs, a_d, a_s, M, y, stream)
  if constexpr (FMT == kFmtIQ4) {
    // IQ4_XS: chunks of 4 steps, whose shorter per-chunk chain suits its
    // table decode (measured on MI355X at M = 3, 4, 6, 8 over 24
    // configurations on seven matrices: 4096 x 24576 at M = 8 19.3 -> 18.6
    // us with two waves sharing activations and a two-way split against 8
    // steps, 5120 x 13824 16.2 -> 15.4 us with the split alone, 8192 x 8192
    // and 13824 x 5120 15.5 -> 14.4 and 20.6 -> 20.1 us with a four-way
    // split, 12288 x 4096 (256 tiles) 11.9 us with an eight-way split)
    if (tiles >= 1100) SKINNY_Q4(1, 2, 2, 4);
    if (tiles >= 600) SKINNY_Q4(1, 1, 2, 4);
    if (tiles > 256) SKINNY_Q4(1, 1, 4, 4);
    SKINNY_Q4(1, 1, 8, 4);
  } else {
    if constexpr (FMT == kFmtQ4K) {
      // Q4_K (its per-step header decode makes shorter chunks pay below 800
      // tiles; measured as above: 7168 x 7168 at M = 8 13.6 -> 12.9 us,
      // 2560 x 10240 8.5 -> 7.9 us against the Q4_0 choices)
      if (tiles < 1100) {
        if (tiles >= 800) {
          if (s8) SKINNY_Q4(1, 2, 2, 8);
          SKINNY_Q4(1, 2, 2, 4);
        }
        if (tiles >= 600) SKINNY_Q4(1, 1, 2, 4);
        if (tiles > 256) SKINNY_Q4(1, 1, 4, 4);
        if (s8) SKINNY_Q4(1, 1, 4, 8);
        SKINNY_Q4(1, 1, 8, 4);
      }
    }
    if (tiles >= 1800) {
      if (s8) SKINNY_Q4(1, 4, 1, 8);
      SKINNY_Q4(1, 4, 1, 4);
    }
    if (tiles >= 1100) {
      if (s8) SKINNY_Q4(1, 2, 1, 8);
      SKINNY_Q4(1, 2, 1, 4);
    }
    if (tiles >= 800) {
      if (s8) SKINNY_Q4(1, 2, 2, 8);
      SKINNY_Q4(1, 2, 2, 4);
    }
    if (tiles >= 512) {
      if (s8) SKINNY_Q4(1, 1, 2, 8);
      SKINNY_Q4(1, 1, 2, 4);
    }
    if (s8) {
      if (tiles <= 256) SKINNY_Q4(1, 1, 4, 8);
      if (K >= 8192) SKINNY_Q4(2, 1, 4, 8);
      SKINNY_Q4(1, 1, 2, 8);
    }
    SKINNY_Q4(1, 1, 8, 4);
  }
#undef SKINNY_Q4
}

template <int FMT>
static hipError_t launch_mfma(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                              const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                              int M, float *y, hipStream_t stream) {
  if (M <= 4) return launch_mfma_mp<4, FMT>(w_qs, w_d, N, K, a_qs, a_d, a_s, M, y, stream);
  return launch_mfma_mp<8, FMT>(w_qs, w_d, N, K, a_qs, a_d, a_s, M, y, stream);
}

// Vector kernel with the activation rows staged in LDS (any M <= 8, one round
// of U blocks per lane, K <= 2048 U).  A workgroup of W waves (two weight rows
// each) reads the Q8_1 activation rows once -- or, FUSED, reads the float32
// rows and quantizes them into LDS itself with the same block arithmetic as
// quantize_act_q8_1 -- so activation bytes per weight byte drop W-fold
// (each wave of the plain kernel re-reads the whole row from L2, as many
// bytes as its weights).  Activation loads are issued first, then the
// wave's whole round of weight loads; the activations are stored (or
// quantized) while the weights are in flight, one barrier, then the dot.
// LDS: codes int8 [M][K] | d8 float [M][K/32] | 8 s8 float [M][K/32].
// The dot is exactly the plain kernel's (same blocks per lane, same order,
// same reduction), so the result equals mmvq_q4_0 on the same Q8_1 input.
template <int M, int U, bool FUSED, int W = 8>
struct LdsAct {
  static constexpr int kW = W;                                     // waves per workgroup
  static constexpr int kMaxNb = kWave * U;                         // blocks per row (max)
  // activation 16-byte loads per lane: plain = codes + d + s pieces;
  // fused = two per 8-element group
  // (plain: M * K / 32 must be a multiple of 8, checked by the launcher)
  static constexpr int kPieces = FUSED ? (M * kMaxNb * 4) : (M * kMaxNb * 2 + M * kMaxNb / 4);
  static constexpr int kA = (kPieces + kW * kWave - 1) / (kW * kWave);
};

// (No __restrict__ on the inputs: the issue fence below must be able to
// keep the activation loads ahead of the weight loads.)
template <int M, int U, bool FUSED, int W = 8>
__global__ __launch_bounds__(64 * W) void mmvq_q4_0_lds_kernel(
    const uint8_t *w_qs, const uint16_t *w_d, int N, int K, const int8_t *a_qs,
    const uint16_t *a_d, const uint16_t *a_s, const float *x, float *y) {
  using P = LdsAct<M, U, FUSED, W>;
  constexpr int R = 2;
  extern __shared__ uint4_t smem4[];
  int8_t *lq = reinterpret_cast<int8_t *>(smem4);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = K >> 5;
  float *ld8 = reinterpret_cast<float *>(lq + M * K);
  float *ls8 = ld8 + M * nb;
  const int n0 = (blockIdx.x * P::kW + wave) * R;

  // 1. activation loads (flat pieces over the workgroup, the last repeated)
  uint4_t av[P::kA][FUSED ? 2 : 1];
  int apiece[P::kA];
  const int npieces = FUSED ? M * K / 8 : M * K / 16 + M * nb / 4;
#pragma unroll
  for (int a = 0; a < P::kA; ++a) {
    const int p = min(tid + a * P::kW * kWave, npieces - 1);
    apiece[a] = tid + a * P::kW * kWave;
    if constexpr (FUSED) {
      const float4_t *src = reinterpret_cast<const float4_t *>(x + (size_t)p * 8);
      av[a][0] = __builtin_bit_cast(uint4_t, src[0]);
      av[a][1] = __builtin_bit_cast(uint4_t, src[1]);
    } else {
      const int ncode = M * K / 16, nd = M * nb / 8;
      const uint8_t *src =
          p < ncode ? reinterpret_cast<const uint8_t *>(a_qs) + 16 * p
          : p < ncode + nd ? reinterpret_cast<const uint8_t *>(a_d) + 16 * (p - ncode)
                           : reinterpret_cast<const uint8_t *>(a_s) + 16 * (p - ncode - nd);
      av[a][0] = load16(src);
    }
  }
  issue_fence();

  // 2. this wave's round of weight loads
  const int nw = min(n0, N - 1);            // waves past N load row N - 1 and store nothing
  const uint8_t *wrow[R];
  const uint16_t *drow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(nw + r, N - 1);
    wrow[r] = w_qs + (size_t)n * (size_t)(K >> 1);
    drow[r] = w_d + (size_t)n * (size_t)nb;
  }
  uint4_t wq[U][R];
  uint16_t d4h[U][R];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int b = min(lane + u * kWave, nb - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wq[u][r] = load16_nt(wrow[r] + 16 * b);
      d4h[u][r] = load_u16_nt(drow[r] + b);
    }
  }
  issue_fence();

  // 3. activations into LDS (waits only for the activation loads)
#pragma unroll
  for (int a = 0; a < P::kA; ++a) {
    const int p = apiece[a];
    if constexpr (FUSED) {
      // groups of a quad form one block; a quad is all in or all out
      uint32_t lo, hi;
      uint16_t db, sb;
      quantize_q8_1_group(__builtin_bit_cast(float4_t, av[a][0]),
                          __builtin_bit_cast(float4_t, av[a][1]), lo, hi, db, sb);
      if (p < npieces) {
        *reinterpret_cast<uint2_t *>(lq + 8 * p) = uint2_t{lo, hi};
        if ((p & 3) == 0) {
          const int blk = p >> 2;                     // flat block index m * nb + b
          ld8[blk] = f16_bits_to_f32(db);
          ls8[blk] = 8.0f * f16_bits_to_f32(sb);
        }
      }
    } else if (p < npieces) {
      const int ncode = M * K / 16, nd = M * nb / 8;
      if (p < ncode) {
        *reinterpret_cast<uint4_t *>(lq + 16 * p) = av[a][0];
      } else {
        const bool isd = p < ncode + nd;
        float *dst = isd ? ld8 + 8 * (p - ncode) : ls8 + 8 * (p - ncode - nd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = f16_bits_to_f32((uint16_t)(av[a][0][e >> 1] >> (16 * (e & 1))));
          dst[e] = isd ? v : 8.0f * v;
        }
      }
    }
  }
  wg_barrier();

  // 4. the dot, exactly as in mmvq_q4_0_kernel
  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int b = min(lane + u * kWave, nb - 1);
    const bool live = lane + u * kWave < nb;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = wq[u][r][i] & 0x0F0F0F0Fu;
        hi[i] = (wq[u][r][i] >> 4) & 0x0F0F0F0Fu;
      }
      const float d4 = f16_bits_to_f32(d4h[u][r]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4_t aq0 = *reinterpret_cast<const uint4_t *>(lq + (size_t)m * K + 32 * b);
        const uint4_t aq1 = *reinterpret_cast<const uint4_t *>(lq + (size_t)m * K + 32 * b + 16);
        int32_t isum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          isum = dot4_i8(lo[i], aq0[i], isum);
          isum = dot4_i8(hi[i], aq1[i], isum);
        }
        const float t = fmaf(ld8[m * nb + b], (float)isum, -ls8[m * nb + b]);
        const float a = fmaf(d4, t, acc[r][m]);
        acc[r][m] = live ? a : acc[r][m];
      }
    }
  }

  constexpr int V = next_pow2(R * M);
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = (i < R * M) ? acc[i / M][i % M] : 0.0f;
  const float total = wave_reduce_transpose<V>(v, lane);
  constexpr int SHIFT = 6 - Log2<V>::value;
  const int idx = lane >> SHIFT;
  if ((lane & ((1 << SHIFT) - 1)) == 0 && idx < R * M) {
    const int r = idx / M, m = idx % M;
    const int n = n0 + r;
    if (n < N) y[(size_t)m * N + n] = total;
  }
}

// Staged kernel in rounds (3 <= M <= 8, narrow matrices): the activation
// rows are staged in LDS as above (codes int8 [M][K] | d8 float | 8 s8
// float), but each lane then walks its blocks b = lane, lane + 64, ... one
// per round, two register buffers alternating, so a wave holds two blocks
// per row in flight instead of its whole share of K; the per-block dot and
// epilogue are the plain kernel's.
template <int M, int R, int W, int A>
__global__ __launch_bounds__(64 * W) void mmvq_q4_0_lds_rounds_kernel(
    const uint8_t *w_qs, const uint16_t *w_d, int N, int K, const int8_t *a_qs,
    const uint16_t *a_d, const uint16_t *a_s, float *y) {
  extern __shared__ uint4_t smem4[];
  int8_t *lq = reinterpret_cast<int8_t *>(smem4);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // row addresses stay scalar
  const int nb = K >> 5;
  float *ld8 = reinterpret_cast<float *>(lq + M * K);
  float *ls8 = ld8 + M * nb;
  const int n0 = (blockIdx.x * W + wave) * R;
  // 16-byte pieces: codes (M K / 16), d (M nb / 8), s (M nb / 8)
  const int ncode = M * K / 16, nd = M * nb / 8, npieces = ncode + 2 * nd;
  auto piece = [&](int p) {
    return p < ncode ? reinterpret_cast<const uint8_t *>(a_qs) + 16 * (size_t)p
         : p < ncode + nd ? reinterpret_cast<const uint8_t *>(a_d) + 16 * (size_t)(p - ncode)
                          : reinterpret_cast<const uint8_t *>(a_s) + 16 * (size_t)(p - ncode - nd);
  };
  uint4_t av[A];
#pragma unroll
  for (int a = 0; a < A; ++a) av[a] = load16(piece(min(tid + a * W * kWave, npieces - 1)));
  issue_fence();

  const int nw = min(n0, N - 1);            // waves past N read row N - 1 and store nothing
  const uint8_t *wrow[R];
  const uint16_t *drow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(nw + r, N - 1);
    wrow[r] = w_qs + (size_t)n * (size_t)(K >> 1);
    drow[r] = w_d + (size_t)n * (size_t)nb;
  }
  struct Round {
    uint4_t wq[R];
    uint16_t d4[R];
  };
  auto load = [&](int b, Round &rd) {
    b = min(b, nb - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      rd.wq[r] = load16_nt(wrow[r] + 16 * b);
      rd.d4[r] = load_u16_nt(drow[r] + b);
    }
  };
  Round r0, r1;
  load(lane, r0);
  issue_fence();
  auto store = [&](int p0) {
#pragma unroll
    for (int a = 0; a < A; ++a) {
      const int p = p0 + tid + a * W * kWave;
      if (p < ncode) {
        *reinterpret_cast<uint4_t *>(lq + 16 * p) = av[a];
      } else if (p < npieces) {
        const bool isd = p < ncode + nd;
        float *dst = isd ? ld8 + 8 * (p - ncode) : ls8 + 8 * (p - ncode - nd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = f16_bits_to_f32((uint16_t)(av[a][e >> 1] >> (16 * (e & 1))));
          dst[e] = isd ? v : 8.0f * v;
        }
      }
    }
  };
  store(0);                                 // straight-line: waits only for the activations
  for (int p0 = A * W * kWave; p0 < npieces; p0 += A * W * kWave) {
#pragma unroll
    for (int a = 0; a < A; ++a) av[a] = load16(piece(min(p0 + tid + a * W * kWave, npieces - 1)));
    store(p0);
  }
  wg_barrier();
  if (n0 >= N) return;

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
  auto compute = [&](int b, const Round &rd) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = rd.wq[r][i] & 0x0F0F0F0Fu;
        hi[i] = (rd.wq[r][i] >> 4) & 0x0F0F0F0Fu;
      }
      const float d4 = f16_bits_to_f32(rd.d4[r]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4_t aq0 = *reinterpret_cast<const uint4_t *>(lq + (size_t)m * K + 32 * b);
        const uint4_t aq1 = *reinterpret_cast<const uint4_t *>(lq + (size_t)m * K + 32 * b + 16);
        int32_t isum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          isum = dot4_i8(lo[i], aq0[i], isum);
          isum = dot4_i8(hi[i], aq1[i], isum);
        }
        const float t = fmaf(ld8[m * nb + b], (float)isum, -ls8[m * nb + b]);
        acc[r][m] = fmaf(d4, t, acc[r][m]);
      }
    }
  };
  for (int b = lane; b < nb; b += 2 * kWave) {
    if (b + kWave < nb) load(b + kWave, r1);
    issue_fence();
    compute(b, r0);
    if (b + kWave >= nb) break;
    if (b + 2 * kWave < nb) load(b + 2 * kWave, r0);
    issue_fence();
    compute(b + kWave, r1);
  }

  constexpr int V = next_pow2(R * M);
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = (i < R * M) ? acc[i / M][i % M] : 0.0f;
  const float total = wave_reduce_transpose<V>(v, lane);
  constexpr int SHIFT = 6 - Log2<V>::value;
  const int idx = lane >> SHIFT;
  if ((lane & ((1 << SHIFT) - 1)) == 0 && idx < R * M) {
    const int r = idx / M, m = idx % M;
    const int n = n0 + r;
    if (n < N) y[(size_t)m * N + n] = total;
  }
}

template <int M, int A>
static hipError_t launch_lds_rounds_a(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                                      const int8_t *a_qs, const uint16_t *a_d,
                                      const uint16_t *a_s, float *y, hipStream_t stream) {
  constexpr int R = 2, W = 8;
  const int lds = M * K + 8 * M * (K >> 5);
  const hipError_t lds_ok = allow_lds((const void *)mmvq_q4_0_lds_rounds_kernel<M, R, W, A>, lds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int rows = R * W;
  hipLaunchKernelGGL((mmvq_q4_0_lds_rounds_kernel<M, R, W, A>), dim3((N + rows - 1) / rows),
                     dim3(64 * W), lds, stream, w_qs, w_d, N, K, a_qs, a_d, a_s, y);
  return hipGetLastError();
}

// Two rows per wave, eight waves (measured on MI355X over the Llama-2-7B
// shapes: 11008 x 4096 at M = 4 9.4 -> 8.5 us, at M = 8 11.8 -> 11.2 us on the
// matrix cores; 4096 x 4096 at M = 6 5.25 -> 4.8 us).  At M <= 6 it keeps
// the lead up to N = 8192 (7168 x 7168 at M = 6 14.6 -> 10.8 us, 2048 x 8192
// at M = 4 5.3 -> 4.4 us; at M = 4 13824 x 5120, past the plain staged
// kernel's K limit, 19.9 -> 13.3 us); at M = 7 and 8 only up to N = 4096,
// as the matrix cores' narrow table is faster above (5120 x 5120 at M = 8
// 10.8 against 9.3 us).
constexpr int kQ4RoundsMaxN = 8192;
constexpr int kQ4RoundsMaxNWide = 4096;   // at M >= 7
constexpr int kQ4RoundsWideM = 7;
// Up to N = 2048 and K = 8192 the vector kernel is the fastest at M <= 4
// (a handful of staged workgroups cannot fill the chip: 8192 x 2048 at M = 3
// 5.9 -> 5.1 us, 4096 x 2048 at M = 4 3.8 -> 3.4 us).
constexpr int kQ4VectorNarrowN = 2048;

static int lds_rounds_bytes(int M, int K) { return M * K + 8 * M * (K >> 5); }

template <int M>
static hipError_t launch_lds_rounds(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                                    const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                    float *y, hipStream_t stream) {
  const int pieces = M * K / 16 + 2 * (M * (K >> 5) / 8);
  const int per_thread = (pieces + 511) / 512;   // first staging batch
  if (per_thread <= 4) return launch_lds_rounds_a<M, 4>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
  if (per_thread <= 8) return launch_lds_rounds_a<M, 8>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
  return launch_lds_rounds_a<M, 16>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
}

template <int M, int U, bool FUSED, int W = 8>
static hipError_t launch_lds_u(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                               const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                               const float *x, float *y, hipStream_t stream) {
  using P = LdsAct<M, U, FUSED, W>;
  const int rows = 2 * P::kW;
  const int blocks = (N + rows - 1) / rows;
  const size_t lds = (size_t)M * K + 8 * (size_t)M * (K >> 5);
  const hipError_t lds_ok = allow_lds((const void *)mmvq_q4_0_lds_kernel<M, U, FUSED, W>, (int)lds);
  if (lds_ok != hipSuccess) return lds_ok;
  hipLaunchKernelGGL((mmvq_q4_0_lds_kernel<M, U, FUSED, W>), dim3(blocks), dim3(64 * P::kW), lds,
                     stream, w_qs, w_d, N, K, a_qs, a_d, a_s, x, y);
  return hipGetLastError();
}

// K limit of the LDS-staged kernel: one round of at most 6 blocks per lane
// (SKINNY_MAX_K_F32ACT).
constexpr int kLdsMaxK = 2048 * 6;
static_assert(kLdsMaxK == SKINNY_MAX_K_F32ACT, "documented limit");

template <int M, bool FUSED, int W = 8>
static hipError_t launch_lds(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                             const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                             const float *x, float *y, hipStream_t stream) {
  const int per_lane = ((K >> 5) + kWave - 1) / kWave;
#define SKINNY_LDS(U) return launch_lds_u<M, U, FUSED, W>(w_qs, w_d, N, K, a_qs, a_d, a_s, x, y, stream)
  if (per_lane <= 2) SKINNY_LDS(2);
  if (per_lane <= 3) SKINNY_LDS(3);
  if (per_lane <= 4) SKINNY_LDS(4);
  SKINNY_LDS(6);
#undef SKINNY_LDS
}

template <int M, int R, int U, int KS = 1>
static hipError_t launch_mru(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                             const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                             float *y, hipStream_t stream) {
  const int groups = (N + R - 1) / R;                 // row groups of KS waves each
  const int per_block = 4 / KS;
  const int blocks = (groups + per_block - 1) / per_block;
  hipLaunchKernelGGL((mmvq_q4_0_kernel<M, R, U, true, KS>), dim3(blocks), dim3(256), 0, stream,
                     w_qs, w_d, N, K, a_qs, a_d, a_s, y);
  return hipGetLastError();
}

// Vector kernel shape: two rows per wave (a handful of 128-bit weight loads
// in flight per lane, many waves) measured best on MI355X at M <= 4 on
// every Llama-2-7B shape.  At M <= 2 each lane loads all of its blocks of a
// row in one round (U = blocks per lane, up to 8 = K 16384) -- long rows are
// otherwise bound by successive memory round trips (7.8 -> 6.3 us for an
// 11008 x 4096 matrix; with U = 8, 14336 x 4096 9.7 -> 7.7 us and
// 13824 x 5120 11.9 -> 9.8 us at M = 1).  The round holds exactly the lane's
// share (5 or 7 blocks too: a padded slot costs a block's loads and dots;
// 14336 x 4096 8.2 -> 6.9 us, 10240 x 4096 6.3 -> 5.7 us at M = 1).  Up to 12 blocks per lane (K 24576)
// two waves split each row, one round of up to 6 blocks each (17408 x 5120
// 12.8 -> 11.2 us at M = 1, 16.1 -> 14.6 at M = 2); longer rows take rounds
// of 6, which measured as fast as a split or rounds of 8 there (28672 x 4096
// and 40960 x 2048).
template <int M>
static hipError_t launch_m(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                           const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                           float *y, hipStream_t stream) {
  if constexpr (M <= 2) {
    const int per_lane = ((K >> 5) + kWave - 1) / kWave;
    if (per_lane > 12) return launch_mru<M, 2, 6>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    if (per_lane > 8) return launch_mru<M, 2, 6, 2>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    if (per_lane > 7) return launch_mru<M, 2, 8>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    if (per_lane > 6) return launch_mru<M, 2, 7>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    if (per_lane > 5) return launch_mru<M, 2, 6>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    if (per_lane > 4) return launch_mru<M, 2, 5>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    if (per_lane > 3) return launch_mru<M, 2, 4>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    if (per_lane > 2) return launch_mru<M, 2, 3>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    return launch_mru<M, 2, 2>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
  } else if constexpr (M <= 4) {
    return launch_mru<M, 2, 2>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
  } else {
    return launch_mru<M, 4, 2>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
  }
}

// Plain LDS-staged vector kernel for 3 <= M <= 5 on matrices wider than
// N = 8192 (narrower ones take the staged kernel in rounds): eight waves per
// workgroup.
template <int M>
static hipError_t launch_lds_plain(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                                   const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                   float *y, hipStream_t stream) {
  return launch_lds<M, false, 8>(w_qs, w_d, N, K, a_qs, a_d, a_s, nullptr, y, stream);
}

hipError_t launch_mmvq_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                            const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                            int M, float *y, hipStream_t stream) {
  // Long rows at M <= 2 on matrices of 4096 rows or more: the staged kernel
  // in rounds (measured on MI355X: at M = 2 rows past K = 12288, 13824 x 5120
  // 14.2 -> 10.2 us, 14336 x 4096 10.3 -> 8.6 us, 28672 x 4096 16.5 -> 14.8
  // us; at M = 1 rows past 12 blocks per lane, 28672 x 4096 14.7 -> 13.4
  // us; shorter rows, and N = 2048, stay on the vector kernel).
  {
    const int per_lane = ((K >> 5) + kWave - 1) / kWave;
    const bool long_rows = M == 2 ? per_lane > 6 : M == 1 && per_lane > 12;
    if (long_rows && N >= 4096 && (M * (K >> 5)) % 8 == 0 && lds_rounds_bytes(M, K) <= 160 * 1024)
      return M == 1 ? launch_lds_rounds<1>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream)
                    : launch_lds_rounds<2>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
  }
  // Small matrices at M <= 4: the vector kernel.
  if (M >= 3 && M <= 4 && N <= kQ4VectorNarrowN && K <= 8192)
    return M == 3 ? launch_m<3>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream)
                  : launch_m<4>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
  // Narrow matrices from M = 3: the staged kernel in rounds.  Both staged
  // kernels copy the Q8_1 scales in 16-byte pieces of 8, so they need
  // M * K / 32 to be a multiple of 8.
  const int rounds_max_n = M >= kQ4RoundsWideM ? kQ4RoundsMaxNWide : kQ4RoundsMaxN;
  if (M >= 3 && N <= rounds_max_n && (M * (K >> 5)) % 8 == 0 &&
      lds_rounds_bytes(M, K) <= 160 * 1024) {
    switch (M) {
      case 3: return launch_lds_rounds<3>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
      case 4: return launch_lds_rounds<4>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
      case 5: return launch_lds_rounds<5>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
      case 6: return launch_lds_rounds<6>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
      case 7: return launch_lds_rounds<7>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
      default: return launch_lds_rounds<8>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    }
  }
  // M = 3..5 on wider matrices: the activation rows staged in LDS once per
  // workgroup beat the matrix cores (measured on MI355X over the Llama-2-7B
  // shapes: 4096 x 22016 at M = 3 15.0 -> 10.8 us, at M = 4 15.2 -> 12.9 us,
  // at M = 5 14.2 -> 13.1 us); from M = 6 wider matrices take the matrix
  // cores.
  const bool lds_ok = K <= kLdsMaxK && (M * (K >> 5)) % 8 == 0;
  if (M >= 3 && M <= 5 && lds_ok) {
    switch (M) {
      case 3: return launch_lds_plain<3>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
      case 4: return launch_lds_plain<4>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
      default: return launch_lds_plain<5>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    }
  }
  const bool small = M <= kQ4VectorMaxM && N < 8192 && K < 8192;
  if (M >= kQ4MfmaMinM && K % 256 == 0 && !small)
    return launch_mfma<kFmtQ40>(w_qs, w_d, N, K, a_qs, a_d, a_s, M, y, stream);
  // Two rows re-read twice the activation bytes per weight byte of one: on
  // wide matrices staging them in LDS once per workgroup pays (measured on
  // MI355X: 4096 x 22016 10.8 -> 10.2 us, 4096 x 32000 15.0 -> 13.4 us); at
  // M = 1 and on narrow matrices the direct kernel is as fast or faster.
  if (M == 2 && N >= 8192 && lds_ok)
    return launch_lds<2, false>(w_qs, w_d, N, K, a_qs, a_d, a_s, nullptr, y, stream);
  switch (M) {
    case 1: return launch_m<1>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    case 2: return launch_m<2>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    case 3: return launch_m<3>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    case 4: return launch_m<4>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    case 5: return launch_m<5>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    case 6: return launch_m<6>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    case 7: return launch_m<7>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    default: return launch_m<8>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
  }
}

hipError_t launch_mmvq_q4_0_f32act(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                                   const float *x, int M, float *y, hipStream_t stream) {
  if (M == 1) return launch_lds<1, true>(w_qs, w_d, N, K, nullptr, nullptr, nullptr, x, y, stream);
  return launch_lds<2, true>(w_qs, w_d, N, K, nullptr, nullptr, nullptr, x, y, stream);
}

// Q4_K weights on the matrix-core kernel (3 <= M <= 8, K % 256 == 0): the
// super-block headers take the place of the Q4_0 block scales.
hipError_t launch_mmvq_q4_k_mfma(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                 const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                 int M, float *y, hipStream_t stream) {
  return launch_mfma<kFmtQ4K>(w_qs, reinterpret_cast<const uint16_t *>(w_hdr), N, K, a_qs, a_d,
                              a_s, M, y, stream);
}

// IQ4_XS weights on the matrix-core kernel (3 <= M <= 8, K % 256 == 0, the
// headers 16-byte aligned): the 8-byte super-block headers take the place
// of the Q4_0 block scales; the Q8_1 sum term is not used, so d8 stands in
// for it in the staging.
hipError_t launch_mmvq_iq4_xs_mfma(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                   const int8_t *a_qs, const uint16_t *a_d, int M, float *y,
                                   hipStream_t stream) {
  if (K % 256 != 0) return hipErrorInvalidValue;
  return launch_mfma<kFmtIQ4>(w_qs, reinterpret_cast<const uint16_t *>(w_hdr), N, K, a_qs, a_d,
                              a_d, M, y, stream);
}

}  // namespace skinny
