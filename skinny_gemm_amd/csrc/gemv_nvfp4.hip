// gemv_nvfp4.hip -- NVFP4 weights (E2M1 codes, E4M3 scale per 16 elements,
// float32 per-tensor scale) x binary16 activations, M = 1..16 rows.
//
// "v100-skinny README", "How QPN works": packed codes stay compressed in
// memory and are decoded only in registers where they are consumed; the
// global scale is folded into the group scales and every 16-element group
// is flushed into a float32 accumulator, which keeps activation outliers
// from overflowing binary16.  Here each group's dot is accumulated in
// float32 by v_dot2_f32_f16 (binary16 products are exact in float32) and
// flushed with acc += p * (e4m3(scale) * g).
//
// Mapping (one wave = R weight rows, full K):
//   * lane l takes 32-element chunks c = l, l + 64, ...: 16 code bytes (one
//     128-bit load) and the two group scales of the chunk (one 16-bit load);
//   * codes decode two at a time with v_cvt_scalef32_pk_f16_fp4 (scale 1.0,
//     exact), once per row, reused for all M activation rows;
//   * the chunk's binary16 activations (M x 64 B) are loaded once per lane
//     and reused for all R rows;
//   * a transposing butterfly reduces the R*M partial sums per lane.
// At M <= 2 the same mapping runs with the activation rows staged in LDS
// once per workgroup (gemv_nvfp4_lds_kernel, and gemv_nvfp4_flat_kernel,
// which spreads a wave's rows evenly over its lanes); M >= 3 takes the
// matrix cores (M = 3 on 4097..5120 rows the staged kernel).
// Bytes per call: N*K*(1/2 + 1/16) weights + 2*M*K activations + 2*M*N out.
#include "device.h"
#include "launch.h"
#include "nvfp4.h"

namespace skinny {

// Activation rows from which the matrix-core kernel is used.
constexpr int kNvfp4MfmaMinM = 3;

constexpr int next_pow2_n(int v) { return v <= 1 ? 1 : 2 * next_pow2_n((v + 1) / 2); }

// (No __restrict__ on the inputs: the issue barrier below must be able to
// keep a round's loads ahead of its arithmetic.)
template <int M, int R, int U>
__global__ __launch_bounds__(256) void gemv_nvfp4_kernel(
    const uint8_t *codes, const uint8_t *scales, float g, int N, int K, const uint16_t *x,
    uint16_t *y) {
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6)) * R;
  if (n0 >= N) return;
  const int nc = K >> 5;                    // 32-element chunks per row

  const uint8_t *crow[R];
  const uint16_t *srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(n0 + r, N - 1);
    crow[r] = codes + (size_t)n * (size_t)(K >> 1);
    srow[r] = reinterpret_cast<const uint16_t *>(scales + (size_t)n * (size_t)(K >> 4));
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
    uint32_t sc2[UU][R];
    uint4_t xv[UU][M][4];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      const int c = min(c0 + u * kWave, nc - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wq[u][r] = load16_nt(crow[r] + 16 * c);
        sc2[u][r] = load_u16_nt(srow[r] + c);
      }
      // activations of the chunk: 32 binary16 = 16 pairs per row m
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint16_t *xp = x + (size_t)m * K + 32 * c;
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[u][m][q] = load16(xp + 8 * q);
      }
    }
    if constexpr (U > 0) issue_all();
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      const bool live = c0 + u * kWave < nc;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // decode: word i, byte j -> elements 8i+2j (low nibble), 8i+2j+1
        uint32_t wh[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wh[4 * i + 0] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<0>(wq[u][r][i]));
          wh[4 * i + 1] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<1>(wq[u][r][i]));
          wh[4 * i + 2] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<2>(wq[u][r][i]));
          wh[4 * i + 3] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<3>(wq[u][r][i]));
        }
        const float s0 = e4m3_to_f32<0>(sc2[u][r]) * g;
        const float s1 = e4m3_to_f32<1>(sc2[u][r]) * g;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          // pair p (0..15) of the chunk is dword p%4 of xv[u][m][p/4]
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int p = 0; p < 8; ++p) p0 = dot2_f16(wh[p], xv[u][m][p >> 2][p & 3], p0);
#pragma unroll
          for (int p = 8; p < 16; ++p) p1 = dot2_f16(wh[p], xv[u][m][p >> 2][p & 3], p1);
          float a = fmaf(p0, s0, acc[r][m]);
          a = fmaf(p1, s1, a);
          acc[r][m] = live ? a : acc[r][m];
        }
      }
    }
  }

  constexpr int V = next_pow2_n(R * M);
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = (i < R * M) ? acc[i / M][i % M] : 0.0f;
  const float total = wave_reduce_transpose<V>(v, lane);
  constexpr int SHIFT = 6 - Log2<V>::value;
  const int idx = lane >> SHIFT;
  if ((lane & ((1 << SHIFT) - 1)) == 0 && idx < R * M) {
    const int r = idx / M, m = idx % M;
    const int n = n0 + r;
    if (n < N) y[(size_t)m * N + n] = f32_to_f16_bits(total);
  }
}

// Vector kernel with the activation rows staged in LDS (M <= 2, M K <= 80 K
// elements).  The plain vector kernel reads each lane's 64 activation bytes
// per chunk through the vector memory path once per wave, 1.8 bytes per
// weight byte at two rows per wave, and that path, not HBM, bounds it on
// wide matrices.  Here a workgroup of W waves loads the rows once (issued
// ahead of the first weight loads), stores them as swizzled 16-byte pieces,
// one barrier, and every lane reads its chunk's activations from LDS.  Each
// wave takes R rows, one 32-element chunk per lane per round, the next
// round's weights in flight under the current one's arithmetic.  Decode,
// group dots and flushes are the plain kernel's, in the same order per row.
template <int M, int R, int W, int A>
__global__ __launch_bounds__(64 * W) void gemv_nvfp4_lds_kernel(
    const uint8_t *codes, const uint8_t *scales, float g, int N, int K, const uint16_t *x,
    uint16_t *y) {
  extern __shared__ uint4_t xs[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // row addresses stay scalar
  const int n0 = (blockIdx.x * W + wave) * R;
  const int nc = K >> 5;                    // 32-element chunks per row
  const int np = K >> 3;                    // 16-byte activation pieces per row
  const int tot = M * np;
  uint4_t av[A];
  act_issue<A, 64 * W>(x, tot, av);

  const uint8_t *crow[R];
  const uint16_t *srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(n0 + r, N - 1);
    crow[r] = codes + (size_t)n * (size_t)(K >> 1);
    srow[r] = reinterpret_cast<const uint16_t *>(scales + (size_t)n * (size_t)(K >> 4));
  }
  struct Round {
    uint4_t wq[R];
    uint32_t sc[R];
  };
  auto load = [&](int c, Round &rd) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      rd.wq[r] = load16_nt(crow[r] + 16 * c);
      rd.sc[r] = load_u16_nt(srow[r] + c);
    }
  };
  Round r0, r1;
  load(min(lane, nc - 1), r0);
  issue_fence();
  act_stage<4, A, 64 * W>(x, tot, np, xs, av);
  wg_barrier();
  if (n0 >= N) return;

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
  auto compute = [&](int c, const Round &rd) {
    uint4_t xv[M][4];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[m][q] = xs[m * np + act_slot<4>(c, q)];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // the two 16-element groups in turn (words 0-1, then 2-3), each decoded
      // just before its dots: fewer registers live, more waves resident
      float p[2][M];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t wh[8];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t w = rd.wq[r][2 * h + i];
          wh[4 * i + 0] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<0>(w));
          wh[4 * i + 1] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<1>(w));
          wh[4 * i + 2] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<2>(w));
          wh[4 * i + 3] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<3>(w));
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float t = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; ++q) t = dot2_f16(wh[q], xv[m][2 * h + (q >> 2)][q & 3], t);
          p[h][m] = t;
        }
      }
      const float s0 = e4m3_to_f32<0>(rd.sc[r]) * g;
      const float s1 = e4m3_to_f32<1>(rd.sc[r]) * g;
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = fmaf(p[1][m], s1, fmaf(p[0][m], s0, acc[r][m]));
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

  constexpr int V = next_pow2_n(R * M);
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = (i < R * M) ? acc[i / M][i % M] : 0.0f;
  const float total = wave_reduce_transpose<V>(v, lane);
  constexpr int SHIFT = 6 - Log2<V>::value;
  const int idx = lane >> SHIFT;
  if ((lane & ((1 << SHIFT) - 1)) == 0 && idx < R * M) {
    const int r = idx / M, m = idx % M;
    const int n = n0 + r;
    if (n < N) y[(size_t)m * N + n] = f32_to_f16_bits(total);
  }
}

// Flat variant of the staged kernel for one activation row (M = 1) when a
// row holds an odd number of half-waves of chunks (K = 3072 or 5120): the
// round mapping above then leaves half the lanes idle in its last round.
// A wave's R rows are adjacent in memory, one span of R * nc chunks (16 code
// bytes and 2 scale bytes each), and lane l takes chunks f = l + 64 i of the
// span, i < L = R nc / 64: every lane busy, all L loads issued before the
// activation staging, one memory round trip.  Chunk f belongs to row f / nc
// at position f % nc; since nc >= 64, stepping f by 64 wraps into the next
// row at most once.  Decode, group dots and flushes are the staged kernel's,
// one chunk at a time.
template <int R, int L, int W, int A>
__global__ __launch_bounds__(64 * W) void gemv_nvfp4_flat_kernel(
    const uint8_t *codes, const uint8_t *scales, float g, int N, int K, const uint16_t *x,
    uint16_t *y) {
  extern __shared__ uint4_t xs[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // span address stays scalar
  const int n0 = (blockIdx.x * W + wave) * R;
  const int nc = K >> 5;                    // 32-element chunks per row
  const int np = K >> 3;                    // 16-byte activation pieces
  uint4_t av[A];
  act_issue<A, 64 * W>(x, np, av);

  // waves past N read row N - 1 and store nothing
  const int nw = min(n0, N - 1);
  const int span = min(R, N - nw) * nc;     // chunks of the rows that exist
  const uint8_t *cspan = codes + (size_t)nw * (size_t)(K >> 1);
  const uint16_t *sspan = reinterpret_cast<const uint16_t *>(scales + (size_t)nw * (size_t)(K >> 4));
  uint4_t wq[L];
  uint32_t sc[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int f = min(lane + kWave * i, span - 1);
    wq[i] = load16_nt(cspan + 16 * (size_t)f);
    sc[i] = load_u16_nt(sspan + f);
  }
  issue_fence();
  act_stage<4, A, 64 * W>(x, np, np, xs, av);
  wg_barrier();
  if (n0 >= N) return;

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  int c = lane, row = 0;                    // position and row of chunk i
  uint4_t xn[4];                            // its activations, read one chunk ahead
#pragma unroll
  for (int q = 0; q < 4; ++q) xn[q] = xs[act_slot<4>(c, q)];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    __builtin_amdgcn_sched_barrier(0);      // one chunk at a time: few registers live
    uint4_t xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = xn[q];
    const int ri = row;
    const bool live = lane + kWave * i < span;
    if (i + 1 < L) {
      c += kWave;
      if (c >= nc) { c -= nc; ++row; }
#pragma unroll
      for (int q = 0; q < 4; ++q) xn[q] = xs[act_slot<4>(c, q)];
    }
    float p[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t wh[8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w = wq[i][2 * h + j];
        wh[4 * j + 0] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<0>(w));
        wh[4 * j + 1] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<1>(w));
        wh[4 * j + 2] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<2>(w));
        wh[4 * j + 3] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<3>(w));
      }
      float t = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) t = dot2_f16(wh[q], xv[2 * h + (q >> 2)][q & 3], t);
      p[h] = t;
    }
    const float s0 = e4m3_to_f32<0>(sc[i]) * g;
    const float s1 = e4m3_to_f32<1>(sc[i]) * g;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float a = fmaf(p[1], s1, fmaf(p[0], s0, acc[r]));
      acc[r] = (live && ri == r) ? a : acc[r];
    }
  }

  constexpr int V = next_pow2_n(R);
  float v[V];
#pragma unroll
  for (int k = 0; k < V; ++k) v[k] = k < R ? acc[k] : 0.0f;
  const float total = wave_reduce_transpose<V>(v, lane);
  constexpr int SHIFT = 6 - Log2<V>::value;
  const int r = lane >> SHIFT;
  if ((lane & ((1 << SHIFT) - 1)) == 0 && r < R && n0 + r < N)
    y[n0 + r] = f32_to_f16_bits(total);
}

// Matrix-core variant (3 <= M <= 16, K % 256 == 0).
//
// Tile: 16 weight rows.  Lane l = (i = l % 16, g = l / 16) of a wave feeds
// row 16t + i of the A operand of four v_mfma_f32_16x16x32_f16 per 128-K
// step: its 16 code bytes (elements k0 .. k0+31, k0 = 128 s + 32 g) decode
// two at a time to binary16 times the binary16 group scale -- exact, as an
// E2M1 value times an E4M3 value has at most 5 significant bits and lies in
// [2^-10, 2688].  The B operands are the activations x[i][k0 + 8t .. +8]
// (columns i >= M are computed and dropped).  The matrix core accumulates
// in float32 across all of K, so no binary16 partial sum exists anywhere;
// the per-tensor scale multiplies the finished sum.
//
// Data movement.  A workgroup is WR x KS waves: WR waves own different
// tiles (T each) and share one K slice, KS slices split K.  K is walked in
// chunks of S steps.  Every wave reads its own codes and group scales, and
// a 1/WR share of the slice's activation chunk (MP rows; rows past M repeat
// row M - 1), with 128-bit loads in row-contiguous order (each 1 KB load
// instruction covers whole 128-byte lines) into registers one chunk ahead
// of its use; registers, not LDS, hold the bytes in flight.  When a chunk's
// turn comes its weights are written to a wave-private LDS buffer and its
// activation share to the slice's activation buffer (double-buffered when
// WR > 1, with one barrier per chunk; a lone wave needs neither), then read
// back in the operand layout while the registers refill with the next
// chunk.  Sharing cuts the activation bytes each wave pulls from L2 WR-fold;
// at M = 8 a tile's chunk holds fewer weight bytes than activation bytes,
// and the two streams share the vector memory path.  Loads are issued in
// the order they are consumed, so each wait covers exactly one chunk.
// LDS layout: 1 KB blocks as written by one store instruction (lane l ->
// bytes 16 l); the 16-byte columns of each block are XOR-swizzled so the
// operand-layout reads (16 rows at one column) hit distinct banks.  The KS
// partial tiles are summed in LDS.
namespace nv {
template <int T, int WR, int KS, int S, int MP>
struct Cfg {
  static constexpr int kWaves = WR * KS;
  static constexpr int kRows = 16 * T;              // weight rows per wave
  static constexpr int kRpi = 16 / S;               // code rows per 1 KB block
  static constexpr int kCi = T * S;                 // code loads per chunk
  static constexpr int kSclB = kRows * 8 * S;       // scale bytes per chunk
  static constexpr int kWst = kCi * 1024 + kSclB;   // wave weight buffer
  static constexpr int kRpa = 4 / S;                // activation rows per 1 KB block
  static constexpr int kAi = MP / kRpa;             // activation loads per chunk
  static constexpr int kApw = (kAi + WR - 1) / WR;  // activation loads per wave
  static constexpr int kNab = WR > 1 ? 2 : 1;       // activation buffers per slice
  static constexpr int kAst = kAi * 1024;           // one activation buffer
  static constexpr int kActBase = kWaves * kWst;
  static constexpr int kLds = kActBase + KS * kNab * kAst;
  static_assert(S == 2 || S == 4, "chunk steps");
  static_assert(MP == 4 || MP == 8 || MP == 16, "padded activation rows");
  static_assert(kSclB <= 1024, "one scale load per chunk");
  static_assert(kWaves * T * kWave * 16 <= kLds, "reduction buffer");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};
}  // namespace nv

template <int T, int S, int APW>
struct NvChunk {
  uint4_t c[T * S];
  uint4_t s;
  uint4_t a[APW];
};

// (No __restrict__ on the inputs: the issue fences below must be able to
// order their loads.)
template <int T, int WR, int KS, int S, int MP>
__global__ __launch_bounds__(64 * WR * KS) void gemv_nvfp4_mfma_kernel(
    const uint8_t *codes, const uint8_t *scales, float g,
    int N, int K, const uint16_t *x, int M, uint16_t *y) {
  using C = nv::Cfg<T, WR, KS, S, MP>;
  using R = NvChunk<T, S, C::kApw>;
  extern __shared__ uint4_t smem4[];
  uint8_t *smem = reinterpret_cast<uint8_t *>(smem4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wr = wave % WR, ks = wave / WR;
  const int i = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * (C::kRows * WR) + C::kRows * wr;
  uint8_t *ws = smem + wave * C::kWst;
  uint8_t *abuf = smem + C::kActBase + ks * C::kNab * C::kAst;

  const size_t rowc = (size_t)(K >> 1), rows_ = (size_t)(K >> 4);
  const int nct = K / (128 * S);
  const int cps = (nct + KS - 1) / KS;
  const int cb = ks * cps, ce = min(nct, cb + cps);

  // per-lane sources (chunk 0)
  const uint8_t *csrc[C::kCi];
#pragma unroll
  for (int q = 0; q < C::kCi; ++q) {
    const int r = q * C::kRpi + (lane % C::kRpi);
    const int j = (lane / C::kRpi) ^ (q & (S - 1));
    csrc[q] = codes + (size_t)min(n0 + r, N - 1) * rowc + 16 * j;
  }
  const bool sact = lane < C::kSclB / 16;
  const int sl = lane % (C::kSclB / 16);       // lanes past the scale bytes repeat one
  const uint8_t *ssrc = scales + (size_t)min(n0 + sl % C::kRows, N - 1) * rows_ +
                        16 * (sl / C::kRows);
  // activation pieces of this wave: p = wr, wr + WR, ... (the last repeated)
  const uint16_t *asrc[C::kApw];
  int apiece[C::kApw];
#pragma unroll
  for (int u = 0; u < C::kApw; ++u) {
    const int p = min(wr + WR * u, C::kAi - 1);
    apiece[u] = p;
    const int r = min(p * C::kRpa + (lane % C::kRpa), M - 1);
    const int j = (lane / C::kRpa) ^ p;
    asrc[u] = x + (size_t)r * K + 8 * j;
  }
  auto load = [&](int c, R &rg) {
#pragma unroll
    for (int q = 0; q < C::kCi; ++q) rg.c[q] = load16_nt(csrc[q] + (size_t)c * (64 * S));
    // a chunk takes 8 S bytes of each row's scales, part of a 128-byte line:
    // the default cache policy keeps the rest of the line for the next chunks
    rg.s = load16(ssrc + (size_t)c * (8 * S));
#pragma unroll
    for (int u = 0; u < C::kApw; ++u) rg.a[u] = load16(asrc[u] + (size_t)c * (128 * S));
    issue_fence();   // keep each chunk's loads together and ahead of later work
  };
  auto store = [&](const R &rg, uint8_t *ab) {
#pragma unroll
    for (int q = 0; q < C::kCi; ++q) *reinterpret_cast<uint4_t *>(ws + 1024 * q + 16 * lane) = rg.c[q];
    if (sact) *reinterpret_cast<uint4_t *>(ws + C::kCi * 1024 + 16 * lane) = rg.s;
#pragma unroll
    for (int u = 0; u < C::kApw; ++u)
      *reinterpret_cast<uint4_t *>(ab + 1024 * apiece[u] + 16 * lane) = rg.a[u];
  };

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int ar = i & (MP - 1), aa = ar / C::kRpa;   // activation row (columns >= MP wrap)
  const int aoff = 1024 * aa + 16 * (ar % C::kRpa);
  auto consume = [&](const uint8_t *ab) {
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
        const int r = 16 * t + i, q = r / C::kRpi;
        const int j = 4 * st + grp;
        const uint4_t wq = *reinterpret_cast<const uint4_t *>(
            ws + 1024 * q + 16 * (C::kRpi * (j ^ (q & (S - 1))) + r % C::kRpi));
        const uint32_t sc = *reinterpret_cast<const uint16_t *>(
            ws + C::kCi * 1024 + 16 * ((st >> 1) * C::kRows + r) + 8 * (st & 1) + 2 * grp);
        nvfp4_step(wq, sc, xv, acc[t]);
      }
    }
  };

  // A lone wave walks its own slice.  Waves that share activations run
  // cps steps in lockstep (the barrier); steps past a slice's end load its
  // last chunk again and compute nothing, so every path issues the same
  // loads (the load past the last step likewise re-reads into registers
  // that are never stored).
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
        const int n = n0 + 16 * t + 4 * grp + r;
        if (n < N) y[(size_t)i * N + n] = f32_to_f16_bits(acc[t][r] * g);
      }
    }
  }
}

template <int T, int WR, int KS, int S, int MP>
static hipError_t launch_mfma_cfg(const uint8_t *codes, const uint8_t *scales, float g, int N,
                                  int K, const uint16_t *x, int M, uint16_t *y,
                                  hipStream_t stream) {
  using C = nv::Cfg<T, WR, KS, S, MP>;
  if (K % (128 * S) != 0) return hipErrorInvalidValue;   // chunks must tile K
  const hipError_t lds_ok =
      allow_lds((const void *)gemv_nvfp4_mfma_kernel<T, WR, KS, S, MP>, C::kLds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int rows = C::kRows * WR;
  const int blocks = (N + rows - 1) / rows;
  hipLaunchKernelGGL((gemv_nvfp4_mfma_kernel<T, WR, KS, S, MP>), dim3(blocks),
                     dim3(64 * C::kWaves), C::kLds, stream, codes, scales, g, N, K, x, M, y);
  return hipGetLastError();
}

// Tiles per wave, K split and chunk length, measured on MI355X at M = 4 and
// 8 over K 5120..17408, N 5120..34816: wide matrices want two tiles per
// wave and no split; mid-width ones one tile; narrow ones (few tiles, long
// K) a four-way split to keep enough waves streaming.  Up to 256 tiles
// (N <= 4096) one tile per wave with the four-way split keeps twice the
// waves (measured at M = 4 and 8 over K 2048..16384, N 1024..4096:
// 14336 x 4096 at M = 4 14.7 -> 10.2 us, 8192 x 2048 9.9 -> 6.8 us,
// 4096 x 4096 6.7 -> 5.3 us; K % 512 != 0 an eight-way split of 2-step
// chunks, 11008 x 4096 12.5 -> 9.0 us).
template <int MP>
static hipError_t launch_mfma_mp(const uint8_t *codes, const uint8_t *scales, float g, int N,
                                 int K, const uint16_t *x, int M, uint16_t *y,
                                 hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const bool s4 = K % 512 == 0;
#define SKINNY_NV(T, KS, S) return launch_mfma_cfg<T, 1, KS, S, MP>(codes, scales, g, N, K, x, M, y, stream)
  if (tiles >= 1536) {
    if (s4) SKINNY_NV(2, 1, 4);
    SKINNY_NV(2, 1, 2);
  }
  if (tiles >= 512) {
    if (s4) { if (M <= 4) SKINNY_NV(1, 2, 4); SKINNY_NV(1, 1, 4); }
    SKINNY_NV(1, 1, 2);
  }
  if (tiles <= 256) {
    if (s4) SKINNY_NV(1, 4, 4);
    SKINNY_NV(1, 8, 2);
  }
  if (s4 && K >= 8192) SKINNY_NV(2, 4, 4);
  SKINNY_NV(2, 4, 2);
#undef SKINNY_NV
}

// 9 <= M <= 16: sixteen activation rows per chunk, twice the activation
// bytes per weight byte of M <= 8, so here four waves sharing each
// activation chunk pays on matrices wide enough to fill the chip with
// 4-wave workgroups (measured on MI355X at M = 12 and 16, K 5120..17408,
// N 5120..34816: 2.45 -> 2.70 TB/s on 5120 x 34816); narrower ones split
// K, with one tile per wave up to 256 tiles (measured over every
// configuration on N 2048..8192: 8192 x 8192 at M = 12 23.5 -> 13.9 us with
// the split from 512 tiles, 28672 x 4096 36.2 -> 26.9 us, 4096 x 4096
// 8.4 -> 6.9 us with one tile per wave).
static hipError_t launch_mfma_wide(const uint8_t *codes, const uint8_t *scales, float g, int N,
                                   int K, const uint16_t *x, int M, uint16_t *y,
                                   hipStream_t stream) {
  const int tiles = (N + 15) / 16;
#define SKINNY_NV(T, WR, KS, S) \
  return launch_mfma_cfg<T, WR, KS, S, 16>(codes, scales, g, N, K, x, M, y, stream)
  if (tiles >= 600) {
    if (K % 512 == 0) SKINNY_NV(1, 4, 1, 4);
    SKINNY_NV(2, 2, 1, 2);
  }
  if (tiles > 256) SKINNY_NV(2, 1, 4, 2);
  SKINNY_NV(1, 1, 4, 2);
#undef SKINNY_NV
}

static hipError_t launch_mfma(const uint8_t *codes, const uint8_t *scales, float g, int N,
                              int K, const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  if (M <= 4) return launch_mfma_mp<4>(codes, scales, g, N, K, x, M, y, stream);
  if (M <= 8) return launch_mfma_mp<8>(codes, scales, g, N, K, x, M, y, stream);
  return launch_mfma_wide(codes, scales, g, N, K, x, M, y, stream);
}

template <int M, int R, int U>
static hipError_t launch_mru(const uint8_t *codes, const uint8_t *scales, float g, int N,
                             int K, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((gemv_nvfp4_kernel<M, R, U>), dim3(blocks), dim3(256), 0, stream,
                     codes, scales, g, N, K, x, y);
  return hipGetLastError();
}

// Plain vector kernel shape: two rows per wave measured best on MI355X at M <= 2
// for every shape tried (K 4096 to 17408, N 4096 to 34816).  A row of up to
// 4 chunks per lane is loaded in one round (one memory round trip: 3.9 ->
// 4.7 TB/s on a 5120 x 34816 matrix); longer rows keep the pipelined loop,
// faster there than several rounds.  Wider M (only for K % 256 != 0) takes
// four rows per wave.
template <int M>
static hipError_t launch_m(const uint8_t *codes, const uint8_t *scales, float g, int N, int K,
                           const uint16_t *x, uint16_t *y, hipStream_t stream) {
  if constexpr (M <= 2) {
    const int per_lane = ((K >> 5) + kWave - 1) / kWave;
    if (per_lane <= 2) return launch_mru<M, 2, 2>(codes, scales, g, N, K, x, y, stream);
    if (per_lane <= 3) return launch_mru<M, 2, 3>(codes, scales, g, N, K, x, y, stream);
    if (per_lane <= 4) return launch_mru<M, 2, 4>(codes, scales, g, N, K, x, y, stream);
    return launch_mru<M, 2, 0>(codes, scales, g, N, K, x, y, stream);
  } else {
    return launch_mru<M, 4, 1>(codes, scales, g, N, K, x, y, stream);
  }
}

// Staged-activation vector kernel (M <= 2, and M = 3 on 4097..5120 rows): three
// rows per wave, four waves per workgroup at M = 1 and eight at M = 2 and 3
// (measured on MI355X over K 5120 and 17408, N 5120 to 34816: 5120 x 34816 at
// M = 1 24.7 -> 19.0 us, at M = 2 28.3 -> 24.9 us against the matrix cores;
// 17408 x 5120 at M = 2 17.3 -> 14.1 us).  Small matrices take two rows and
// four waves instead: at M = 1 with N and K up to 8192, at M = 2 up to 2^24
// weights (below).
constexpr int kNvLdsMaxMK = 80 * 1024;      // M K binary16 activations in LDS

template <int M, int W, int A, int R = 3>
static hipError_t launch_lds_a(const uint8_t *codes, const uint8_t *scales, float g, int N,
                               int K, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const int lds = M * K * 2;
  const hipError_t lds_ok =
      allow_lds((const void *)gemv_nvfp4_lds_kernel<M, R, W, A>, 2 * kNvLdsMaxMK);
  if (lds_ok != hipSuccess) return lds_ok;
  const int rows = R * W;
  hipLaunchKernelGGL((gemv_nvfp4_lds_kernel<M, R, W, A>), dim3((N + rows - 1) / rows),
                     dim3(64 * W), lds, stream, codes, scales, g, N, K, x, y);
  return hipGetLastError();
}

// At M = 3 it also beats the matrix cores on matrices from N = 4097 up to
// N = 5120 (5120 x 5120 7.6 -> 6.8 us, 17408 x 5120 17.2 -> 16.4 us; wider
// matrices and M = 4 stay on the matrix cores).  Up to N = 4096 the matrix
// cores' narrow table (one tile per wave, K split) is as fast or faster
// (14336 x 4096 12.5 -> 9.9 us, 8192 x 2048 7.6 -> 6.7 us; 4096 x 4096 and
// 2048 x 2048 equal).
constexpr int kNvLdsM3MaxN = 5120;
constexpr int kNvNarrowN = 4096;

// One activation row on a small matrix (N and K up to 8192) takes two rows
// per wave: more, smaller workgroups.  Measured at M = 1: 4096 x 4096 4.0 ->
// 3.65 us, 8192 x 4096 5.9 -> 5.4 us, 5120 x 5120 5.0 -> 4.9 us; rows of
// K = 17408 lose with it (11.0 -> 11.8 us).
constexpr int kNvSmallMaxNK = 8192;
// At M = 2 the same shape wins only on matrices of up to 2^24 weights
// (5120 x 2048 5.4 -> 4.0 us, 4096 x 4096 4.6 -> 4.1 us; 5120 x 5120 and
// larger lose with it).
constexpr long long kSmallMaxWeights = 1LL << 24;

template <int M, int R, int W>
static hipError_t launch_lds_r(const uint8_t *codes, const uint8_t *scales, float g, int N,
                               int K, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const int per_thread = (M * (K >> 3) + 64 * W - 1) / (64 * W);   // first staging batch
  if (per_thread <= 2) return launch_lds_a<M, W, 2, R>(codes, scales, g, N, K, x, y, stream);
  if (per_thread <= 4) return launch_lds_a<M, W, 4, R>(codes, scales, g, N, K, x, y, stream);
  if (per_thread <= 8) return launch_lds_a<M, W, 8, R>(codes, scales, g, N, K, x, y, stream);
  return launch_lds_a<M, W, 12, R>(codes, scales, g, N, K, x, y, stream);
}

template <int M>
static hipError_t launch_lds(const uint8_t *codes, const uint8_t *scales, float g, int N, int K,
                             const uint16_t *x, uint16_t *y, hipStream_t stream) {
  if constexpr (M == 1) {
    if (N <= kNvSmallMaxNK && K <= kNvSmallMaxNK)
      return launch_lds_r<M, 2, 4>(codes, scales, g, N, K, x, y, stream);
    return launch_lds_r<M, 3, 4>(codes, scales, g, N, K, x, y, stream);
  } else {
    if (M == 2 && (long long)N * K <= kSmallMaxWeights)
      return launch_lds_r<M, 2, 4>(codes, scales, g, N, K, x, y, stream);
    return launch_lds_r<M, 3, 8>(codes, scales, g, N, K, x, y, stream);
  }
}

// Flat kernel (M = 1, nc = K / 32 in {96, 160}): two rows per wave, L = nc / 32
// chunks per lane; four waves per workgroup, eight on wide matrices
// (measured on MI355X at M = 1: 5120 x 10240 8.2 -> 7.3 us with four waves,
// 5120 x 34816 18.2 -> 17.9 us with eight; 5120 x 5120 is as fast on the
// round mapping and keeps it).
template <int L, int W>
static hipError_t launch_flat_lw(const uint8_t *codes, const uint8_t *scales, float g, int N,
                                 int K, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  constexpr int R = 2;
  const int rows = R * W;
  const int lds = 2 * K;
  if ((K >> 3) <= 2 * 64 * W)
    hipLaunchKernelGGL((gemv_nvfp4_flat_kernel<R, L, W, 2>), dim3((N + rows - 1) / rows),
                       dim3(64 * W), lds, stream, codes, scales, g, N, K, x, y);
  else
    hipLaunchKernelGGL((gemv_nvfp4_flat_kernel<R, L, W, 4>), dim3((N + rows - 1) / rows),
                       dim3(64 * W), lds, stream, codes, scales, g, N, K, x, y);
  return hipGetLastError();
}

static bool flat_fits(int N, int K) {
  const int nc = K >> 5;
  return N >= 8192 && (nc == 96 || nc == 160);
}

static hipError_t launch_flat(const uint8_t *codes, const uint8_t *scales, float g, int N, int K,
                              const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const bool wide = N >= 16384;
  if ((K >> 5) == 96)
    return wide ? launch_flat_lw<3, 8>(codes, scales, g, N, K, x, y, stream)
                : launch_flat_lw<3, 4>(codes, scales, g, N, K, x, y, stream);
  return wide ? launch_flat_lw<5, 8>(codes, scales, g, N, K, x, y, stream)
              : launch_flat_lw<5, 4>(codes, scales, g, N, K, x, y, stream);
}

// Vector kernel for 1 <= M <= 8 rows.
static hipError_t launch_vector(const uint8_t *codes, const uint8_t *scales, float g, int N,
                                int K, const uint16_t *x, int M, uint16_t *y,
                                hipStream_t stream) {
  switch (M) {
    case 1: return launch_m<1>(codes, scales, g, N, K, x, y, stream);
    case 2: return launch_m<2>(codes, scales, g, N, K, x, y, stream);
    case 3: return launch_m<3>(codes, scales, g, N, K, x, y, stream);
    case 4: return launch_m<4>(codes, scales, g, N, K, x, y, stream);
    case 5: return launch_m<5>(codes, scales, g, N, K, x, y, stream);
    case 6: return launch_m<6>(codes, scales, g, N, K, x, y, stream);
    case 7: return launch_m<7>(codes, scales, g, N, K, x, y, stream);
    default: return launch_m<8>(codes, scales, g, N, K, x, y, stream);
  }
}

// M <= 2 takes the staged-activation vector kernel while the rows fit in
// LDS (its flat variant at M = 1 on wide matrices with K = 3072 or 5120),
// and so does M = 3 on matrices of 4097 to 5120 rows.
// The matrix-core kernel takes every M >= 3 in one weight pass when K is a
// whole number of 256-element chunks.  Otherwise the plain vector kernel
// serves up to 8 rows per pass: rows 9..M take a second pass.
hipError_t launch_gemv_nvfp4(const uint8_t *codes, const uint8_t *scales, float g, int N, int K,
                             const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  if (M == 3 && N <= kNvLdsM3MaxN && M * K <= kNvLdsMaxMK && (N > kNvNarrowN || K % 256 != 0))
    return launch_lds<3>(codes, scales, g, N, K, x, y, stream);
  if (M <= 2 && M * K <= kNvLdsMaxMK) {
    if (M == 1 && flat_fits(N, K)) return launch_flat(codes, scales, g, N, K, x, y, stream);
    if (M == 1) return launch_lds<1>(codes, scales, g, N, K, x, y, stream);
    return launch_lds<2>(codes, scales, g, N, K, x, y, stream);
  }
  if (M >= kNvfp4MfmaMinM && K % 256 == 0)
    return launch_mfma(codes, scales, g, N, K, x, M, y, stream);
  if (M <= 8) return launch_vector(codes, scales, g, N, K, x, M, y, stream);
  const hipError_t e = launch_vector(codes, scales, g, N, K, x, 8, y, stream);
  if (e != hipSuccess) return e;
  return launch_vector(codes, scales, g, N, K, x + (size_t)8 * K, M - 8, y + (size_t)8 * N,
                       stream);
}

}  // namespace skinny
