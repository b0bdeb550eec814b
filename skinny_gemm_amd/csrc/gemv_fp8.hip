// gemv_fp8.hip -- FP8 E4M3 weights x binary16 activations, M = 1..96 rows,
// per-output-channel float32 scale.
//
// "v100-skinny README", "How QPN works": the FP8 weights are one contiguous
// E4M3 byte stream with a simpler decoder than NVFP4, run through the same
// skinny geometry.  Every E4M3 value is a binary16 value, so two bytes at a
// time decode exactly with v_cvt_scalef32_pk_f16_fp8 (scale 1.0) and feed
// v_dot2_f32_f16 (float32 accumulation).  The channel scale is applied once
// to the finished dot (the pages do not state the scale granularity).
//
// Mapping (one wave = R weight rows, full K): lane l takes 16-element
// chunks c = l, l + 64, ...: one 128-bit weight load per row, the chunk's
// activations (M x 32 B) loaded once and reused for all R rows, and a
// transposing butterfly for the R*M partial sums at the end.  At M <= 5
// (and M = 6 up to 8192 rows) the same mapping runs with the activation
// rows staged in LDS once per workgroup (gemv_fp8_lds_kernel), except from
// M = 3 on matrices of at most 4096 rows with K >= 8192 (matrix cores).
// Bytes per call: N*K + 4*N weights and scales + 2*M*K + 2*M*N.
#include "device.h"
#include "fp8.h"
#include "launch.h"

namespace skinny {

// Activation rows from which the matrix-core kernel is used.
constexpr int kFp8MfmaMinM = 3;

constexpr int next_pow2_f(int v) { return v <= 1 ? 1 : 2 * next_pow2_f((v + 1) / 2); }

// (No __restrict__ on the inputs: the issue barrier below must be able to
// keep a round's loads ahead of its arithmetic.)
template <int M, int R, int U>
__global__ __launch_bounds__(256) void gemv_fp8_kernel(
    const uint8_t *w, const float *cs, int N, int K, const uint16_t *x, uint16_t *y) {
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6)) * R;
  if (n0 >= N) return;
  const int nc = K >> 4;                    // 16-element chunks per row

  const uint8_t *wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(n0 + r, N - 1);
    wrow[r] = w + (size_t)n * (size_t)K;
  }

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  // U chunks per lane per round, all loaded before any is used (one memory
  // round trip per round); chunks past the row end load chunk nc - 1 again
  // and are not accumulated.
  // U == 0: one chunk per iteration, unrolled twice, the compiler free to
  // pipeline loads of later iterations under the arithmetic.
  constexpr int UU = U > 0 ? U : 1;
  constexpr int kUnroll = U > 0 ? 1 : 2;
#pragma unroll kUnroll
  for (int c0 = lane; c0 < nc; c0 += UU * kWave) {
    uint4_t wq[UU][R];
    uint4_t xv[UU][M][2];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      const int c = min(c0 + u * kWave, nc - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) wq[u][r] = load16_nt(wrow[r] + 16 * c);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint16_t *xp = x + (size_t)m * K + 16 * c;
        xv[u][m][0] = load16(xp);
        xv[u][m][1] = load16(xp + 8);
      }
    }
    if constexpr (U > 0) issue_all();
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      const bool live = c0 + u * kWave < nc;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // word i holds elements 4i..4i+3: pair (4i, 4i+1) and (4i+2, 4i+3)
        uint32_t wh[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wh[2 * i + 0] = __builtin_bit_cast(uint32_t, e4m3x2_to_h2<false>(wq[u][r][i]));
          wh[2 * i + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_h2<true>(wq[u][r][i]));
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float a = acc[r][m];
#pragma unroll
          for (int p = 0; p < 8; ++p) a = dot2_f16(wh[p], xv[u][m][p >> 2][p & 3], a);
          acc[r][m] = live ? a : acc[r][m];
        }
      }
    }
  }

  constexpr int V = next_pow2_f(R * M);
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = (i < R * M) ? acc[i / M][i % M] : 0.0f;
  const float total = wave_reduce_transpose<V>(v, lane);
  constexpr int SHIFT = 6 - Log2<V>::value;
  const int idx = lane >> SHIFT;
  if ((lane & ((1 << SHIFT) - 1)) == 0 && idx < R * M) {
    const int r = idx / M, m = idx % M;
    const int n = n0 + r;
    if (n < N) y[(size_t)m * N + n] = f32_to_f16_bits(total * cs[n]);
  }
}

// Matrix-core variant (3 <= M <= 96, K % 256 == 0).
//
// Tile: 16 weight rows.  Lane l = (i = l % 16, g = l / 16) of a wave feeds
// row 16t + i of the A operand of four v_mfma_f32_16x16x32_f16 per 128-K
// step: its 32 weight bytes (elements k0 .. k0+31, k0 = 128 s + 32 g)
// decode exactly to binary16 (every E4M3 value is a binary16 value).  The B
// operands are the activations x[16c + i][k0 + 8u .. +8] of column tile c:
// one column tile for M <= 16 (columns i >= M computed and dropped), MT =
// MP / 16 of them above, each decoded A operand feeding MT matrix-core
// instructions (the "chunked" FP8 band of the pages' dispatch table).
// Float32 accumulation across all of K; the channel scale multiplies the
// finished sum.
//
// Data movement, as for the NVFP4 kernel.  A workgroup is WR x KS waves:
// WR waves own different tiles (T each) and share one K slice, KS slices
// split K.  K is walked in chunks of S steps.  Every wave reads its own
// weight bytes and a 1/WR share of the slice's activation chunk (MP rows;
// rows past M repeat row M - 1), with 128-bit loads in row-contiguous order
// into registers one chunk ahead of its use; at its turn the chunk goes to
// LDS -- weights to a wave-private buffer, activations to the slice's buffer
// (double-buffered when WR > 1, with one barrier per chunk) -- in 1 KB blocks
// whose 16-byte columns are XOR-swizzled so the operand-layout reads hit
// distinct banks, and is read back in the operand layout.  Loads are issued
// in the order they are consumed, so each wait covers exactly one chunk.
// The KS partial tiles are summed in LDS.
namespace f8 {
template <int T, int WR, int KS, int S, int MP>
struct Cfg {
  static constexpr int kWaves = WR * KS;
  static constexpr int kMT = MP > 16 ? MP / 16 : 1;  // column tiles
  static constexpr int kRows = 16 * T;              // weight rows per wave
  static constexpr int kRpi = 8 / S;                // weight rows per 1 KB block
  static constexpr int kSwz = 2 * S - 1;            // weight column swizzle mask
  static constexpr int kCi = 2 * T * S;             // weight loads per chunk
  static constexpr int kWst = kCi * 1024;           // wave weight buffer
  static constexpr int kRpa = 4 / S;                // activation rows per 1 KB block
  static constexpr int kACols = 16 * S;             // 16-byte columns per activation row
  static constexpr int kAi = MP / kRpa;             // activation loads per chunk
  static constexpr int kApw = (kAi + WR - 1) / WR;  // activation loads per wave
  static constexpr int kNab = WR > 1 ? 2 : 1;       // activation buffers per slice
  static constexpr int kAst = kAi * 1024;
  static constexpr int kActBase = kWaves * kWst;
  static constexpr int kLds = kActBase + KS * kNab * kAst;
  static_assert(S == 1 || S == 2 || S == 4, "chunk steps");
  static_assert(MP == 4 || MP == 8 || (MP % 16 == 0 && MP <= 96), "padded activation rows");
  static_assert(kWaves * T * kMT * kWave * 16 <= kLds, "reduction buffer");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};
template <int T, int S, int APW>
struct Chunk {
  uint4_t c[2 * T * S];
  uint4_t a[APW];
};
}  // namespace f8

// (No __restrict__ on the inputs: the issue fence below must be able to
// order their loads.)
//
// A grid with gridDim.y > 1 splits the activation rows into groups of MP:
// workgroup row y takes rows [MP y, MP y + MP).  Workgroups past the last
// tile (the launcher may round the grid's width up) exit at once.
template <int T, int WR, int KS, int S, int MP>
__global__ __launch_bounds__(64 * WR * KS) void gemv_fp8_mfma_kernel(
    const uint8_t *w, const float *cs, int N, int K, const uint16_t *x, int M, uint16_t *y) {
  using C = f8::Cfg<T, WR, KS, S, MP>;
  using R = f8::Chunk<T, S, C::kApw>;
  constexpr int MT = C::kMT;
  if ((int)blockIdx.x * (C::kRows * WR) >= N) return;        // whole workgroup
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
  const int n0 = blockIdx.x * (C::kRows * WR) + C::kRows * wr;
  uint8_t *ws = smem + wave * C::kWst;
  uint8_t *abuf = smem + C::kActBase + ks * C::kNab * C::kAst;

  const int nct = K / (128 * S);
  const int cps = (nct + KS - 1) / KS;
  const int cb = ks * cps, ce = min(nct, cb + cps);

  const uint8_t *wsrc[C::kCi];
#pragma unroll
  for (int q = 0; q < C::kCi; ++q) {
    const int r = q * C::kRpi + (lane % C::kRpi);
    const int j = (lane / C::kRpi) ^ (q & C::kSwz);
    wsrc[q] = w + (size_t)min(n0 + r, N - 1) * (size_t)K + 16 * j;
  }
  // activation pieces of this wave: p = wr, wr + WR, ... (the last repeated)
  const uint16_t *asrc[C::kApw];
  int apiece[C::kApw];
#pragma unroll
  for (int u = 0; u < C::kApw; ++u) {
    const int p = min(wr + WR * u, C::kAi - 1);
    apiece[u] = p;
    const int r = min(p * C::kRpa + (lane % C::kRpa), M - 1);
    const int j = (lane / C::kRpa) ^ (p & (C::kACols - 1));
    asrc[u] = x + (size_t)r * K + 8 * j;
  }
  auto load = [&](int c, R &rg) {
#pragma unroll
    for (int q = 0; q < C::kCi; ++q) rg.c[q] = load16_nt(wsrc[q] + (size_t)c * (128 * S));
#pragma unroll
    for (int u = 0; u < C::kApw; ++u) rg.a[u] = load16(asrc[u] + (size_t)c * (128 * S));
    issue_fence();   // keep each chunk's loads together and ahead of later work
  };
  auto store = [&](const R &rg, uint8_t *ab) {
#pragma unroll
    for (int q = 0; q < C::kCi; ++q) *reinterpret_cast<uint4_t *>(ws + 1024 * q + 16 * lane) = rg.c[q];
#pragma unroll
    for (int u = 0; u < C::kApw; ++u)
      *reinterpret_cast<uint4_t *>(ab + 1024 * apiece[u] + 16 * lane) = rg.a[u];
  };

  float4_t acc[T][MT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < MT; ++c) acc[t][c] = float4_t{0.f, 0.f, 0.f, 0.f};

  // activation row of column tile c for this lane (columns >= MP wrap when
  // MP < 16)
  auto arow = [&](int c) { return MP >= 16 ? 16 * c + i : (i & (MP - 1)); };
  auto decode = [&](int st, int t, half8_t (&a)[4]) {
    const int r = 16 * t + i, q = r / C::kRpi;
    uint4_t wq[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = 8 * st + 2 * grp + h;
      wq[h] = *reinterpret_cast<const uint4_t *>(
          ws + 1024 * q + 16 * (C::kRpi * (j ^ (q & C::kSwz)) + r % C::kRpi));
    }
    fp8_decode(wq, a);
  };
  auto act = [&](const uint8_t *ab, int st, int c, uint4_t (&xv)[4]) {
    const int ar = arow(c), aa = ar / C::kRpa;
    const uint8_t *ap = ab + 1024 * aa + 16 * (ar % C::kRpa);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 16 * st + 4 * grp + u;
      xv[u] = *reinterpret_cast<const uint4_t *>(ap + 16 * C::kRpa * (j ^ (aa & (C::kACols - 1))));
    }
  };
  auto consume = [&](const uint8_t *ab) {
#pragma unroll
    for (int st = 0; st < S; ++st) {
      if constexpr (MT == 1) {
        // one column tile: decode each weight tile just before its products
        uint4_t xv[4];
        act(ab, st, 0, xv);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          half8_t a[4];
          decode(st, t, a);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            acc[t][0] = mfma_16x16x32_f16(a[u], __builtin_bit_cast(half8_t, xv[u]), acc[t][0]);
        }
      } else {
        // several column tiles: decode every weight tile once, reuse it MT times
        half8_t a[T][4];
#pragma unroll
        for (int t = 0; t < T; ++t) decode(st, t, a[t]);
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

  // A lone wave walks its own slice.  Waves that share activations run cps
  // steps in lockstep (the barrier); steps past a slice's end load its last
  // chunk again and compute nothing, so every path issues the same loads
  // (the load past the last step likewise re-reads into registers that are
  // never stored).
  const int steps = WR > 1 ? cps : ce - cb;
  if (steps > 0) {
    const int cl = max(ce - 1, 0);                       // a valid chunk to re-read
    R r0;
    load(min(cb, cl), r0);
    for (int k = 0; k < steps; ++k) {
      const int c = cb + k;
      uint8_t *ab = abuf + (k & (C::kNab - 1)) * C::kAst;
      store(r0, ab);
      if constexpr (WR > 1) wg_barrier();
      load(min(c + 1, cl), r0);
      if (c < ce) consume(ab);
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
          for (int v = 1; v < KS; ++v) acc[t][c] += red[(((v * WR + wr) * T + t) * MT + c) * kWave + lane];
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
            const int n = n0 + 16 * t + 4 * grp + r;
            if (n < N) y[(size_t)m * N + n] = f32_to_f16_bits(acc[t][c][r] * cs[n]);
          }
        }
      }
    }
  }
}

// groups > 1: M > MP rows in groups of MP, one grid row per group.  The grid
// width is then a multiple of 8, so the groups of one tile land on one XCD
// (workgroups are dealt to the 8 XCDs in turn) and re-read its weights from
// that XCD's L2.
template <int T, int WR, int KS, int S, int MP>
static hipError_t launch_mfma_cfg(const uint8_t *w, const float *cs, int N, int K,
                                  const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  using C = f8::Cfg<T, WR, KS, S, MP>;
  if (K % (128 * S) != 0) return hipErrorInvalidValue;   // chunks must tile K
  const hipError_t lds_ok =
      allow_lds((const void *)gemv_fp8_mfma_kernel<T, WR, KS, S, MP>, C::kLds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int rows = C::kRows * WR;
  const int groups = (M + MP - 1) / MP;
  int blocks = (N + rows - 1) / rows;
  if (groups > 1) blocks = (blocks + 7) / 8 * 8;
  hipLaunchKernelGGL((gemv_fp8_mfma_kernel<T, WR, KS, S, MP>), dim3(blocks, groups),
                     dim3(64 * C::kWaves), C::kLds, stream, w, cs, N, K, x, M, y);
  return hipGetLastError();
}

// Tiles per wave, K split and chunk length, measured on MI355X at M = 3, 4
// and 8 over K 5120..17408, N 5120..34816.  Up to 256 tiles (N <= 4096) one
// tile per wave with a four-way K split (eight-way of 2-step chunks when
// K % 512 != 0) keeps enough waves streaming (measured at M = 8 over K
// 2048..16384, N 1024..4096: 14336 x 4096 19.3 -> 14.6 us, 8192 x 2048
// 12.4 -> 8.7 us, 11008 x 4096 18.6 -> 13.0 us).
template <int MP>
static hipError_t launch_mfma_mp(const uint8_t *w, const float *cs, int N, int K,
                                 const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
#define SKINNY_F8(T, KS, S) return launch_mfma_cfg<T, 1, KS, S, MP>(w, cs, N, K, x, M, y, stream)
  if (tiles >= 1536) {
    if (M <= 4) SKINNY_F8(1, 1, 2);
    SKINNY_F8(2, 1, 2);
  }
  if (tiles >= 512) {
    if (s4) SKINNY_F8(1, 1, 4);
    SKINNY_F8(1, 1, 2);
  }
  if (tiles <= 256) {
    if (s4) SKINNY_F8(1, 4, 4);
    SKINNY_F8(1, 8, 2);
  }
  if (s4 && K >= 8192 && M > 4) SKINNY_F8(2, 4, 4);
  if (s4) SKINNY_F8(1, 2, 4);
  SKINNY_F8(1, 2, 2);
#undef SKINNY_F8
}

// 9 <= M <= 16: sixteen activation rows per chunk, twice the activation
// bytes per weight byte of M <= 8; measured on MI355X at M = 12 and 16, K
// 5120..17408, N 5120..34816: wide matrices take four tiles per wave (each
// activation chunk feeds four tiles), mid-width ones one, narrow ones split
// K four ways.  Measured again over every configuration on N 2048..8192:
// 512-599 tiles split K (8192 x 8192 at M = 12 20.9 -> 17.8 us), and up to
// 256 tiles one tile per wave with a two- or four-way split (28672 x 4096
// 39.9 -> 29.5 us, 4096 x 4096 11.4 -> 8.5 us).
static hipError_t launch_mfma_wide(const uint8_t *w, const float *cs, int N, int K,
                                   const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
#define SKINNY_F8(T, KS, S) return launch_mfma_cfg<T, 1, KS, S, 16>(w, cs, N, K, x, M, y, stream)
  if (tiles >= 1536) SKINNY_F8(4, 1, 2);
  if (tiles >= 600) {
    if (s4) SKINNY_F8(1, 1, 4);
    SKINNY_F8(1, 2, 2);
  }
  if (tiles >= 512) {
    if (K >= 8192) SKINNY_F8(2, 4, 2);
    if (s4) SKINNY_F8(1, 2, 4);
    SKINNY_F8(1, 2, 2);
  }
  if (tiles > 256) {
    if (s4 && K >= 8192) SKINNY_F8(2, 4, 4);
    SKINNY_F8(2, 4, 2);
  }
  if (s4) {
    if (K >= 16384) SKINNY_F8(1, 4, 4);
    SKINNY_F8(1, 2, 4);
  }
  SKINNY_F8(1, 4, 2);
#undef SKINNY_F8
}

// 17 <= M <= 96: MP / 16 column tiles per decoded weight operand.  The
// activation chunk (MP rows) outweighs the weights, so two to eight waves
// share it through LDS, and LDS then leaves room for a K split only with
// short chunks.  Measured on MI355X at M = 32, 64, 96 over K 5120..17408, N
// 5120..34816: wide matrices favour more sharing waves, narrow ones a K
// split.  (Narrow matrices, and mid-width ones above M = 48, now go to
// launch_mfma_grouped: in one pass they were limited by their few
// workgroups, 0.6 TB/s on 17408 x 5120 at M = 96.)
template <int MP>
static hipError_t launch_mfma_chunked_mp(const uint8_t *w, const float *cs, int N, int K,
                                         const uint16_t *x, int M, uint16_t *y,
                                         hipStream_t stream) {
  const int tiles = (N + 15) / 16;
#define SKINNY_F8(T, WR, KS, S) \
  return launch_mfma_cfg<T, WR, KS, S, MP>(w, cs, N, K, x, M, y, stream)
  if constexpr (MP <= 48) {
    if (tiles >= 1536) SKINNY_F8(2, 2, 1, 2);
    SKINNY_F8(1, 4, 2, 2);
  } else if constexpr (MP == 64) {
    if (tiles >= 1536) SKINNY_F8(1, 4, 1, 2);
    SKINNY_F8(1, 2, 1, 2);
  } else {
    if (tiles >= 1536) SKINNY_F8(1, 8, 1, 1);
    if (tiles >= 512) SKINNY_F8(1, 4, 1, 2);
    SKINNY_F8(1, 2, 2, 1);
  }
#undef SKINNY_F8
}

// 17 <= M <= 96 on narrow and mid-width matrices: the rows in groups of 16
// or 32, one grid row per group (launch_mfma_cfg), so that a narrow matrix
// still fills the chip; the groups of a tile re-read its weights from one
// L2.  Measured on MI355X at M = 32, 48, 64, 96: 5120 x 5120 at M = 96 50.1
// -> 24.1 us, 17408 x 5120 149.6 -> 68.4 us, 5120 x 10240 54.5 -> 35.8 us;
// wide matrices keep one pass over all rows.
static hipError_t launch_mfma_grouped(const uint8_t *w, const float *cs, int N, int K,
                                      const uint16_t *x, int M, uint16_t *y,
                                      hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
  if (tiles <= 256 && s4) {
    // up to 4096 rows: groups of 16 with a K split (measured over every
    // configuration at M = 32, 64, 96 on N 2048..4096, K 4096..28672:
    // 8192 x 2048 at M = 64 35.0 -> 16.2 us, 28672 x 4096 109.6 -> 64.7 us,
    // 14336 x 4096 at M = 32 29.5 -> 24.8 us, at M = 96 57.4 -> 52.9 us)
    if (M <= 32) {
      if (K >= 12288) return launch_mfma_cfg<2, 1, 4, 4, 16>(w, cs, N, K, x, M, y, stream);
      return launch_mfma_cfg<1, 1, 2, 4, 16>(w, cs, N, K, x, M, y, stream);
    }
    if (M <= 64) {
      if (tiles <= 128) return launch_mfma_cfg<2, 1, 4, 4, 16>(w, cs, N, K, x, M, y, stream);
      return launch_mfma_cfg<1, 4, 2, 4, 16>(w, cs, N, K, x, M, y, stream);
    }
    if (K >= 12288) return launch_mfma_cfg<2, 1, 1, 4, 16>(w, cs, N, K, x, M, y, stream);
    if (K >= 8192) return launch_mfma_cfg<1, 4, 2, 4, 16>(w, cs, N, K, x, M, y, stream);
    return launch_mfma_cfg<1, 4, 1, 4, 16>(w, cs, N, K, x, M, y, stream);
  }
  if (tiles < 512) {
    if (M <= 32) {
      if (s4) return launch_mfma_cfg<1, 1, 1, 4, 16>(w, cs, N, K, x, M, y, stream);
      return launch_mfma_cfg<1, 1, 1, 2, 16>(w, cs, N, K, x, M, y, stream);
    }
    if (M <= 48) {
      if (s4) return launch_mfma_cfg<2, 1, 2, 4, 16>(w, cs, N, K, x, M, y, stream);
      return launch_mfma_cfg<2, 1, 2, 2, 16>(w, cs, N, K, x, M, y, stream);
    }
    return launch_mfma_cfg<1, 4, 2, 2, 32>(w, cs, N, K, x, M, y, stream);
  }
  return launch_mfma_cfg<1, 4, 1, 2, 32>(w, cs, N, K, x, M, y, stream);
}

static hipError_t launch_mfma(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                              int M, uint16_t *y, hipStream_t stream) {
  if (M <= 4) return launch_mfma_mp<4>(w, cs, N, K, x, M, y, stream);
  if (M <= 8) return launch_mfma_mp<8>(w, cs, N, K, x, M, y, stream);
  if (M <= 16) return launch_mfma_wide(w, cs, N, K, x, M, y, stream);
  const int tiles = (N + 15) / 16;
  if (tiles < 512 || (tiles < 1536 && M > 48))
    return launch_mfma_grouped(w, cs, N, K, x, M, y, stream);
  switch ((M + 15) / 16) {
    case 2: return launch_mfma_chunked_mp<32>(w, cs, N, K, x, M, y, stream);
    case 3: return launch_mfma_chunked_mp<48>(w, cs, N, K, x, M, y, stream);
    case 4: return launch_mfma_chunked_mp<64>(w, cs, N, K, x, M, y, stream);
    case 5: return launch_mfma_chunked_mp<80>(w, cs, N, K, x, M, y, stream);
    default: return launch_mfma_chunked_mp<96>(w, cs, N, K, x, M, y, stream);
  }
}

// Vector kernel with the activation rows staged in LDS (M <= 6, M K <= 80 K
// elements).  The plain vector kernel reads each lane's activation bytes
// through the vector memory path once per wave, M bytes per weight byte at
// two rows per wave, and that path bounds it before HBM does.  Here a
// workgroup of W waves loads the rows once (issued ahead of the first
// weight loads), stores them as swizzled 16-byte pieces, one barrier, and
// every lane reads its chunk's activations from LDS.  Each wave takes R
// rows, one 16-element chunk per lane per round, the next round's weights
// in flight under the current one's arithmetic.  Decode and dot order per
// row are the plain kernel's.
template <int M, int R, int W, int A>
__global__ __launch_bounds__(64 * W) void gemv_fp8_lds_kernel(
    const uint8_t *w, const float *cs, int N, int K, const uint16_t *x, uint16_t *y) {
  extern __shared__ uint4_t xs[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // row addresses stay scalar
  const int n0 = (blockIdx.x * W + wave) * R;
  const int nc = K >> 4;                    // 16-element chunks per row
  const int np = K >> 3;                    // 16-byte activation pieces per row
  const int tot = M * np;
  uint4_t av[A];
  act_issue<A, 64 * W>(x, tot, av);

  const uint8_t *wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wrow[r] = w + (size_t)min(n0 + r, N - 1) * (size_t)K;
  struct Round {
    uint4_t wq[R];
  };
  auto load = [&](int c, Round &rd) {
#pragma unroll
    for (int r = 0; r < R; ++r) rd.wq[r] = load16_nt(wrow[r] + 16 * c);
  };
  Round r0, r1;
  load(min(lane, nc - 1), r0);
  issue_fence();
  act_stage<2, A, 64 * W>(x, tot, np, xs, av);
  wg_barrier();
  if (n0 >= N) return;

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
  auto compute = [&](int c, const Round &rd) {
    uint4_t xv[M][2];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int q = 0; q < 2; ++q) xv[m][q] = xs[m * np + act_slot<2>(c, q)];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // word i holds elements 4i..4i+3: pair (4i, 4i+1) and (4i+2, 4i+3)
      uint32_t wh[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wh[2 * i + 0] = __builtin_bit_cast(uint32_t, e4m3x2_to_h2<false>(rd.wq[r][i]));
        wh[2 * i + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_h2<true>(rd.wq[r][i]));
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a = acc[r][m];
#pragma unroll
        for (int p = 0; p < 8; ++p) a = dot2_f16(wh[p], xv[m][p >> 2][p & 3], a);
        acc[r][m] = a;
      }
    }
  };
  // chunks c = lane, lane + 64, ...: the two round buffers alternate
  for (int c = lane; c < nc; c += 2 * kWave) {
    if (c + kWave < nc) load(c + kWave, r1);
    issue_fence();
    compute(c, r0);
    if (c + kWave >= nc) break;
    if (c + 2 * kWave < nc) load(c + 2 * kWave, r0);
    issue_fence();
    compute(c + kWave, r1);
  }

  constexpr int V = next_pow2_f(R * M);
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = (i < R * M) ? acc[i / M][i % M] : 0.0f;
  const float total = wave_reduce_transpose<V>(v, lane);
  constexpr int SHIFT = 6 - Log2<V>::value;
  const int idx = lane >> SHIFT;
  if ((lane & ((1 << SHIFT) - 1)) == 0 && idx < R * M) {
    const int r = idx / M, m = idx % M;
    const int n = n0 + r;
    if (n < N) y[(size_t)m * N + n] = f32_to_f16_bits(total * cs[n]);
  }
}

template <int M, int R, int U>
static hipError_t launch_mru(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                             uint16_t *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((gemv_fp8_kernel<M, R, U>), dim3(blocks), dim3(256), 0, stream,
                     w, cs, N, K, x, y);
  return hipGetLastError();
}

// Plain vector kernel shape: two rows per wave measured best on MI355X at M <= 2
// for every shape tried (K 4096 to 17408, N 4096 to 34816).  Each lane
// loads up to U = 6 chunks of a row per round (one memory round trip per
// round: 5.9 -> 6.2 TB/s on a 5120 x 34816 matrix), U fitted to the chunks
// per lane.  Wider M (only for K % 256 != 0) takes four rows per wave.
template <int M>
static hipError_t launch_m(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                           uint16_t *y, hipStream_t stream) {
  if constexpr (M <= 2) {
    const int per_lane = ((K >> 4) + kWave - 1) / kWave;
    if (per_lane <= 2) return launch_mru<M, 2, 2>(w, cs, N, K, x, y, stream);
    if (per_lane <= 3) return launch_mru<M, 2, 3>(w, cs, N, K, x, y, stream);
    if (per_lane <= 4) return launch_mru<M, 2, 4>(w, cs, N, K, x, y, stream);
    return launch_mru<M, 2, 6>(w, cs, N, K, x, y, stream);
  } else {
    return launch_mru<M, 4, 1>(w, cs, N, K, x, y, stream);
  }
}

// Staged-activation vector kernel (M <= 5, and M = 6 up to 8192 rows):
// three rows per wave, eight waves per workgroup (two rows and four waves on
// small matrices: at M = 1 with N and K up to 8192, at M = 2 up to 2^24
// weights, below; measured on MI355X over K
// 5120 and 17408, N 5120 to 34816: 17408 x 5120 at M = 1 18.3 -> 16.0 us,
// 5120 x 34816 at M = 2 33.6 -> 28.3 us; at M = 3 and 4 on par with or ahead
// of the matrix cores; at M = 5 5120 x 5120 9.9 -> 8.4 us, 5120 x 10240 13.5
// -> 12.9 us, 5120 x 34816 37.0 -> 36.3 us; at M = 6 only 5120 x 5120 gains,
// 9.8 -> 8.4 us, and at M = 8 none).
constexpr int kF8LdsMaxM = 6;
constexpr int kF8LdsNarrowN = 8192;         // M = 6: staged only up to this N
constexpr int kF8LdsMaxMK = 80 * 1024;      // M K binary16 activations in LDS
// Narrow matrices (N <= 4096) with rows of K >= 8192 take the matrix cores'
// narrow table from M = 3 (measured on MI355X: 14336 x 4096 at M = 4
// 15.6 -> 12.7 us, 12288 x 1024 at M = 5 14.5 -> 9.9 us, 8192 x 2048 at M = 3
// 8.2 -> 7.3 us); shorter rows stay staged (4096 x 4096 at M = 3..5 and
// 2048 x 2048 5-8% faster staged).
constexpr int kF8NarrowN = 4096;
constexpr int kF8NarrowMinK = 8192;

template <int M, int A, int R = 3, int W = 8>
static hipError_t launch_lds_a(const uint8_t *w, const float *cs, int N, int K,
                               const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const int lds = M * K * 2;
  const hipError_t lds_ok =
      allow_lds((const void *)gemv_fp8_lds_kernel<M, R, W, A>, 2 * kF8LdsMaxMK);
  if (lds_ok != hipSuccess) return lds_ok;
  const int rows = R * W;
  hipLaunchKernelGGL((gemv_fp8_lds_kernel<M, R, W, A>), dim3((N + rows - 1) / rows),
                     dim3(64 * W), lds, stream, w, cs, N, K, x, y);
  return hipGetLastError();
}

template <int M, int R, int W>
static hipError_t launch_lds_rw(const uint8_t *w, const float *cs, int N, int K,
                                const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const int per_thread = (M * (K >> 3) + 64 * W - 1) / (64 * W);   // first staging batch
  if (per_thread <= 2) return launch_lds_a<M, 2, R, W>(w, cs, N, K, x, y, stream);
  if (per_thread <= 4) return launch_lds_a<M, 4, R, W>(w, cs, N, K, x, y, stream);
  if (per_thread <= 8) return launch_lds_a<M, 8, R, W>(w, cs, N, K, x, y, stream);
  return launch_lds_a<M, 12, R, W>(w, cs, N, K, x, y, stream);
}

// One activation row on a small matrix (N and K up to 8192) takes two rows
// per wave and four waves per workgroup: more, smaller workgroups.  Measured
// at M = 1: 2048 x 5120 5.3 -> 4.3 us, 4096 x 4096 5.35 -> 4.85 us, 4096 x
// 8192 7.8 -> 7.4 us; rows of K = 17408 lose with it (16.0 -> 16.6 us).
constexpr int kF8SmallMaxNK = 8192;
// At M = 2 the same shape wins only on matrices of up to 2^24 weights
// (5120 x 2048 5.7 -> 4.6 us, 4096 x 4096 5.6 -> 5.0 us; 5120 x 5120 and
// larger lose with it).
constexpr long long kF8SmallMaxWeights = 1LL << 24;

template <int M>
static hipError_t launch_lds(const uint8_t *w, const float *cs, int N, int K,
                             const uint16_t *x, uint16_t *y, hipStream_t stream) {
  if constexpr (M == 1) {
    if (N <= kF8SmallMaxNK && K <= kF8SmallMaxNK)
      return launch_lds_rw<M, 2, 4>(w, cs, N, K, x, y, stream);
  } else if constexpr (M == 2) {
    if ((long long)N * K <= kF8SmallMaxWeights)
      return launch_lds_rw<M, 2, 4>(w, cs, N, K, x, y, stream);
  }
  return launch_lds_rw<M, 3, 8>(w, cs, N, K, x, y, stream);
}

// Vector kernel for 1 <= M <= 8 rows.
static hipError_t launch_vector(const uint8_t *w, const float *cs, int N, int K,
                                const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  switch (M) {
    case 1: return launch_m<1>(w, cs, N, K, x, y, stream);
    case 2: return launch_m<2>(w, cs, N, K, x, y, stream);
    case 3: return launch_m<3>(w, cs, N, K, x, y, stream);
    case 4: return launch_m<4>(w, cs, N, K, x, y, stream);
    case 5: return launch_m<5>(w, cs, N, K, x, y, stream);
    case 6: return launch_m<6>(w, cs, N, K, x, y, stream);
    case 7: return launch_m<7>(w, cs, N, K, x, y, stream);
    default: return launch_m<8>(w, cs, N, K, x, y, stream);
  }
}

// M <= 5 (M = 6 up to N = 8192) takes the staged-activation vector kernel
// while the rows fit in LDS, except, from M = 3, matrices of at most 4096
// rows with K >= 8192.  The matrix-core kernel takes every other M >= 3 in
// one weight pass when K is a whole number of 256-element chunks.
// Otherwise the plain vector kernel serves up to 8 rows per pass over the
// weights: rows 1..8, 9..16, ...
hipError_t launch_gemv_fp8(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                           int M, uint16_t *y, hipStream_t stream) {
  const bool narrow_long = M >= 3 && N <= kF8NarrowN && K >= kF8NarrowMinK && K % 256 == 0;
  if (M <= kF8LdsMaxM && M * K <= kF8LdsMaxMK && (M < 6 || N <= kF8LdsNarrowN) && !narrow_long) {
    switch (M) {
      case 1: return launch_lds<1>(w, cs, N, K, x, y, stream);
      case 2: return launch_lds<2>(w, cs, N, K, x, y, stream);
      case 3: return launch_lds<3>(w, cs, N, K, x, y, stream);
      case 4: return launch_lds<4>(w, cs, N, K, x, y, stream);
      case 5: return launch_lds<5>(w, cs, N, K, x, y, stream);
      default: return launch_lds<6>(w, cs, N, K, x, y, stream);
    }
  }
  if (M >= kFp8MfmaMinM && K % 256 == 0) return launch_mfma(w, cs, N, K, x, M, y, stream);
  for (int m0 = 0; m0 < M; m0 += 8) {
    const hipError_t e = launch_vector(w, cs, N, K, x + (size_t)m0 * K, min(8, M - m0),
                                       y + (size_t)m0 * N, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace skinny
