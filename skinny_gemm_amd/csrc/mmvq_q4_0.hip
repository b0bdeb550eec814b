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
#include "device.h"
#include "launch.h"

namespace skinny {

// Activation rows from which the matrix-core kernel is used.
constexpr int kQ4MfmaMinM = 5;

constexpr int next_pow2(int v) { return v <= 1 ? 1 : 2 * next_pow2((v + 1) / 2); }

template <int M, int R, bool NT>
__global__ __launch_bounds__(256) void mmvq_q4_0_kernel(
    const uint8_t *__restrict__ w_qs, const uint16_t *__restrict__ w_d, int N, int K,
    const int8_t *__restrict__ a_qs, const uint16_t *__restrict__ a_d,
    const uint16_t *__restrict__ a_s, float *__restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6)) * R;
  if (n0 >= N) return;
  const int nb = K >> 5;

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

#pragma unroll 2
  for (int b = lane; b < nb; b += kWave) {
    uint4_t wq[R];
    float d4[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wq[r] = NT ? load16_nt(wrow[r] + 16 * b) : load16(wrow[r] + 16 * b);
      d4[r] = f16_bits_to_f32(NT ? load_u16_nt(drow[r] + b) : drow[r][b]);
    }
    uint4_t aq0[M], aq1[M];
    float d8[M], s8x8[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int8_t *ap = a_qs + (size_t)m * K + 32 * b;
      aq0[m] = load16(ap);
      aq1[m] = load16(ap + 16);
      d8[m] = f16_bits_to_f32(a_d[(size_t)m * nb + b]);
      s8x8[m] = 8.0f * f16_bits_to_f32(a_s[(size_t)m * nb + b]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // low nibbles = codes 0..15 of the block, high nibbles = codes 16..31
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = wq[r][i] & 0x0F0F0F0Fu;
        hi[i] = (wq[r][i] >> 4) & 0x0F0F0F0Fu;
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        int32_t isum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          isum = dot4_i8(lo[i], aq0[m][i], isum);
          isum = dot4_i8(hi[i], aq1[m][i], isum);
        }
        const float t = fmaf(d8[m], (float)isum, -s8x8[m]);
        acc[r][m] = fmaf(d4[r], t, acc[r][m]);
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

// Matrix-core variant for wider M.  One v_mfma_i32_16x16x64_i8 computes the
// exact int32 block sums of 16 weight rows x 2 blocks x 8 activation rows.
// K slot g (lane group l / 16) of a step covers block b + g/2, bytes
// 8(g%2) .. 8(g%2)+7 of its 16 code bytes, i.e. elements 8(g%2) + 0..7
// (low nibbles) and 16 + 8(g%2) + 0..7 (high nibbles):
//   * B operand (columns = weight rows): lane (j = l % 16, g) takes those 8
//     bytes of row n0 + j and splits them into 16 codes with two ANDs and
//     two shift+ANDs;
//   * A operand (rows a = 8h + m): block-diagonal, so a row only meets the
//     K slots of its own block h -- lane (j, g) holds the matching 16 Q8_1
//     codes of row m = j % 8 when j / 8 == g / 2 and m < M, else zeros; it
//     is shared by the T weight tiles and kept four steps ahead in a ring;
//   * lane l then owns isum for weight row n0 + l%16, block b + g/2 and
//     activation rows 4(g%2) .. 4(g%2)+3, and applies the float32 block
//     epilogue acc += d4 * (d8 * isum - 8 * s8).
// Each wave takes a contiguous range of K and stages it in chunks of 32
// blocks in wave-private LDS: weight codes and scales are read
// row-contiguously (a 128-bit load per lane covering 512 bytes of each of
// two rows per instruction), the chunk's activation scales as (d8, 8 s8)
// pairs; the next chunk is in flight while the current one is consumed,
// and the last chunk may be partial.  Lanes l and l^32 (even and odd
// blocks) and then the waves are summed at the end.
namespace q4 {
constexpr int kCh = 16;                // block pairs per staged chunk
constexpr int kBlk = 2 * kCh;          // blocks per chunk (32)
constexpr int kRowB = kBlk * 16;       // code bytes per row per chunk (512)
constexpr int kSclB = kBlk * 2;        // weight-scale bytes per row per chunk (64)
constexpr int kRowP = kRowB + 16;      // padded LDS pitches
constexpr int kSclP = kSclB + 16;
constexpr int kActB = kBlk * 8 * 8;    // (d8, 8 s8) for 8 rows m per block (2 KB)
constexpr int kXr = 4;                 // activation steps kept in flight
template <int T>
constexpr int wave_lds() { return 16 * T * (kRowP + kSclP) + kActB; }
}  // namespace q4

__device__ __forceinline__ void q4_mfma_step(const uint2_t &wq, const int4_t &aop, float d4,
                                             const float4_t &sa, const float4_t &sb,
                                             float (&acc)[4]) {
  int4_t bop;
  bop[0] = (int)(wq.x & 0x0F0F0F0Fu);
  bop[1] = (int)(wq.y & 0x0F0F0F0Fu);
  bop[2] = (int)((wq.x >> 4) & 0x0F0F0F0Fu);
  bop[3] = (int)((wq.y >> 4) & 0x0F0F0F0Fu);
  const int4_t zero = {0, 0, 0, 0};
  const int4_t isum = mfma_16x16x64_i8(aop, bop, zero);
  acc[0] = fmaf(d4, fmaf(sa[0], (float)isum[0], -sa[1]), acc[0]);
  acc[1] = fmaf(d4, fmaf(sa[2], (float)isum[1], -sa[3]), acc[1]);
  acc[2] = fmaf(d4, fmaf(sb[0], (float)isum[2], -sb[1]), acc[2]);
  acc[3] = fmaf(d4, fmaf(sb[2], (float)isum[3], -sb[3]), acc[3]);
}

// The 16 activation codes a lane contributes to the A operand of block
// pair p (the caller zeroes them off the diagonal or past K).
__device__ __forceinline__ int4_t q4_aop(const int8_t *arow, int p) {
  const uint2_t lo = load8(arow + 64 * p);
  const uint2_t hi = load8(arow + 64 * p + 16);
  return int4_t{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
}

__device__ __forceinline__ int4_t keep_if(bool keep, const int4_t &v) {
  return int4_t{keep ? v[0] : 0, keep ? v[1] : 0, keep ? v[2] : 0, keep ? v[3] : 0};
}

__device__ __forceinline__ uint4_t keep_if(bool keep, const uint4_t &v) {
  return uint4_t{keep ? v[0] : 0u, keep ? v[1] : 0u, keep ? v[2] : 0u, keep ? v[3] : 0u};
}

template <int W, int T>
__global__ __launch_bounds__(64 * W) void mmvq_q4_0_mfma_kernel(
    const uint8_t *__restrict__ w_qs, const uint16_t *__restrict__ w_d, int N, int K,
    const int8_t *__restrict__ a_qs, const uint16_t *__restrict__ a_d,
    const uint16_t *__restrict__ a_s, int M, float *__restrict__ y) {
  using namespace q4;
  constexpr int ROWS = 16 * T;
  constexpr int CLD = ROWS / 2;        // code loads per chunk (2 rows of 512 B each)
  extern __shared__ uint4_t smem4[];
  uint8_t *smem = reinterpret_cast<uint8_t *>(smem4);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, grp = lane >> 4;
  const int hb = grp >> 1, bh = grp & 1, q0 = 2 * bh;
  const int n0 = blockIdx.x * ROWS;
  const int nb = K >> 5;
  uint8_t *cl = smem + wave * wave_lds<T>();
  uint8_t *sl = cl + ROWS * kRowP;
  float4_t *al = reinterpret_cast<float4_t *>(sl + ROWS * kSclP);   // [32 blocks][4]
  float4_t *red = reinterpret_cast<float4_t *>(smem + W * wave_lds<T>());

  const size_t rowc = (size_t)(K >> 1);
  const uint8_t *cg[CLD];
  const uint8_t *sg[T];
#pragma unroll
  for (int q = 0; q < CLD; ++q)
    cg[q] = w_qs + (size_t)min(n0 + 2 * q + (lane >> 5), N - 1) * rowc + 16 * (lane & 31);
#pragma unroll
  for (int q = 0; q < T; ++q)
    sg[q] = reinterpret_cast<const uint8_t *>(w_d + (size_t)min(n0 + 16 * q + (lane >> 2), N - 1) * nb) +
            16 * (lane & 3);
  // activation-scale staging: lane -> block (lane & 31), rows m = 4 (lane >> 5) .. +3
  const int ab = lane & 31, am0 = 4 * (lane >> 5);

  const bool aact = ((j >> 3) == hb) && (j & 7) < M;
  const int8_t *arow = a_qs + (size_t)(aact ? (j & 7) : 0) * (size_t)K + 32 * hb + 8 * bh;
  // Staged chunks of 32 blocks need 16-byte aligned weight-scale rows
  // (K % 256 == 0, so nb % 8 == 0); the last chunk may be partial, its
  // missing pieces staged as zeros (zero codes and zero scales add nothing).
  const bool staged = (K % 256) == 0;
  const int nchunks = staged ? (nb + kBlk - 1) / kBlk : 0;
  const int per = (nchunks + W - 1) / W;
  const int c0 = min(nchunks, wave * per), c1 = min(nchunks, c0 + per);

  float acc[T][4];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] = 0.f;

  // Every prefetch below is unconditional, from an address clamped into the
  // arrays, so that no branch separates a load from its use; what lies past
  // K (or off the diagonal) is zeroed by a select when it is consumed.
  // Staged chunks imply nb >= 8, so the clamps below stay in range.
  const int pmax = (nb - 1 - hb) >> 1;             // last pair with this lane's block < nb
  int4_t ar[kXr];
#pragma unroll
  for (int d = 0; d < kXr; ++d) ar[d] = q4_aop(arow, min(c0 * kCh + d, pmax));

  uint4_t cr[CLD], sr[T];
  uint32_t avr[8];                     // raw binary16 bits of d8, s8 for 4 rows m
  auto fetch = [&](int c) {
    const int cb = min(c * kBlk + (lane & 31), nb - 1);
#pragma unroll
    for (int q = 0; q < CLD; ++q) cr[q] = load16_nt(cg[q] + (size_t)(cb - (lane & 31)) * 16);
    const int sb = min(c * kBlk + 8 * (lane & 3), nb - 8);
#pragma unroll
    for (int q = 0; q < T; ++q) sr[q] = load16_nt(sg[q] + (size_t)(sb - 8 * (lane & 3)) * 2);
    const int abk = min(c * kBlk + ab, nb - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = min(am0 + r, M - 1);
      avr[2 * r] = a_d[(size_t)m * nb + abk];
      avr[2 * r + 1] = a_s[(size_t)m * nb + abk];
    }
  };
  if (c0 < c1) fetch(c0);
  for (int c = c0; c < c1; ++c) {
    {
      const bool cv = c * kBlk + (lane & 31) < nb;
      const bool sv = c * kBlk + 8 * (lane & 3) < nb;
      const bool av = c * kBlk + ab < nb;
#pragma unroll
      for (int q = 0; q < CLD; ++q)
        *reinterpret_cast<uint4_t *>(cl + (2 * q + (lane >> 5)) * kRowP + 16 * (lane & 31)) =
            keep_if(cv, cr[q]);
#pragma unroll
      for (int q = 0; q < T; ++q)
        *reinterpret_cast<uint4_t *>(sl + (16 * q + (lane >> 2)) * kSclP + 16 * (lane & 3)) =
            keep_if(sv, sr[q]);
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[2 * r] = av ? f16_bits_to_f32((uint16_t)avr[2 * r]) : 0.f;
        v[2 * r + 1] = av ? 8.0f * f16_bits_to_f32((uint16_t)avr[2 * r + 1]) : 0.f;
      }
      al[4 * ab + 2 * (lane >> 5)] = float4_t{v[0], v[1], v[2], v[3]};
      al[4 * ab + 2 * (lane >> 5) + 1] = float4_t{v[4], v[5], v[6], v[7]};
    }
    if (c + 1 < c1) fetch(c + 1);
#pragma unroll
    for (int st = 0; st < kCh; ++st) {
      const int slot = st % kXr;
      const int bl = 2 * st + hb;                  // this lane's block within the chunk
      const bool live = aact && c * kBlk + bl < nb;
      const int4_t aop = keep_if(live, ar[slot]);
      const float4_t sa = al[4 * bl + q0], sb = al[4 * bl + q0 + 1];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint2_t wq = *reinterpret_cast<const uint2_t *>(cl + (16 * t + j) * kRowP + 16 * bl + 8 * bh);
        const float d4 = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(sl + (16 * t + j) * kSclP + 2 * bl));
        q4_mfma_step(wq, aop, d4, sa, sb, acc[t]);
      }
      ar[slot] = q4_aop(arow, min(c * kCh + st + kXr, pmax));
    }
  }
  // without staging (K % 256 != 0) the last wave reads every block directly
  if (!staged && wave == W - 1) {
    for (int p = 0; 2 * p < nb; ++p) {
      const int b = 2 * p + hb;                    // this lane's block
      const bool bact = b < nb;
      int4_t aop = {0, 0, 0, 0};
      float4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
      if (bact) {
        aop = keep_if(aact, q4_aop(arow, p));
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = min(4 * bh + r, M - 1);
          v[2 * r] = f16_bits_to_f32(a_d[(size_t)m * nb + b]);
          v[2 * r + 1] = 8.0f * f16_bits_to_f32(a_s[(size_t)m * nb + b]);
        }
        sa = float4_t{v[0], v[1], v[2], v[3]};
        sb = float4_t{v[4], v[5], v[6], v[7]};
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int nrow = min(n0 + 16 * t + j, N - 1);
        uint2_t wq = {0u, 0u};
        float d4 = 0.f;
        if (bact) {
          wq = load8_nt(w_qs + (size_t)nrow * rowc + 16 * b + 8 * bh);
          d4 = f16_bits_to_f32(load_u16_nt(w_d + (size_t)nrow * nb + b));
        }
        q4_mfma_step(wq, aop, d4, sa, sb, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] = add_swap32(acc[t][r]);
    if (lane < 32)
      red[(wave * T + t) * 32 + lane] = float4_t{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
  }
  __syncthreads();
  if (wave == 0 && lane < 32) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float4_t tot = red[t * 32 + lane];
#pragma unroll
      for (int v = 1; v < W; ++v) tot += red[(v * T + t) * 32 + lane];
      const int n = n0 + 16 * t + j;
      if (n < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * bh + r;
          if (m < M) y[(size_t)m * N + n] = tot[r];
        }
      }
    }
  }
}

template <int W, int T>
static hipError_t launch_mfma_wt(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                                 const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                 int M, float *y, hipStream_t stream) {
  const int blocks = (N + 16 * T - 1) / (16 * T);
  const size_t shmem = (size_t)W * q4::wave_lds<T>() + sizeof(float4_t) * 32 * W * T;
  hipLaunchKernelGGL((mmvq_q4_0_mfma_kernel<W, T>), dim3(blocks), dim3(64 * W), shmem,
                     stream, w_qs, w_d, N, K, a_qs, a_d, a_s, M, y);
  return hipGetLastError();
}

// Tiles per wave T (weight rows sharing one activation operand) and waves
// per workgroup W (K split), W * T <= 4 so the staging buffers fit in 64 KB
// of LDS.  Measured on MI355X at M = 8: wide matrices prefer two tiles and
// few K splits, narrow ones four K splits to fill the machine.
static void pick_tw(int N, int K, int &T, int &W) {
  (void)K;
  const int tiles = (N + 15) / 16;
  if (tiles >= 1024) { T = 2; W = tiles >= 2000 ? 1 : 2; }
  else if (tiles >= 512) { T = 1; W = 2; }
  else { T = 1; W = 4; }
}

static hipError_t launch_mfma(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                              const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                              int M, float *y, hipStream_t stream) {
  int T, W;
  pick_tw(N, K, T, W);
#define SKINNY_Q4_CASE(TT, WW)                                                              \
  if (T == TT && W == WW)                                                                  \
    return launch_mfma_wt<WW, TT>(w_qs, w_d, N, K, a_qs, a_d, a_s, M, y, stream);
  SKINNY_Q4_CASE(1, 1) SKINNY_Q4_CASE(1, 2) SKINNY_Q4_CASE(1, 4)
  SKINNY_Q4_CASE(2, 1) SKINNY_Q4_CASE(2, 2)
#undef SKINNY_Q4_CASE
  return hipErrorInvalidValue;
}

template <int M, int R, bool NT = true>
static hipError_t launch_mr(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                            const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                            float *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((mmvq_q4_0_kernel<M, R, NT>), dim3(blocks), dim3(256), 0, stream,
                     w_qs, w_d, N, K, a_qs, a_d, a_s, y);
  return hipGetLastError();
}

// Rows per wave for the vector kernel: two rows (a handful of 128-bit
// weight loads in flight per lane, many waves) measured best on MI355X at
// M <= 4 on every Llama-2-7B shape; four at wider M, where the activation
// block is reused across more rows.
static int rows_per_wave(int N, int M) {
  (void)N;
  return M <= 4 ? 2 : 4;
}

template <int M>
static hipError_t launch_m(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                           const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                           float *y, hipStream_t stream) {
  switch (rows_per_wave(N, M)) {
    case 2: return launch_mr<M, 2>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    case 4: return launch_mr<M, 4>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
    default: return launch_mr<M, 8>(w_qs, w_d, N, K, a_qs, a_d, a_s, y, stream);
  }
}

hipError_t launch_mmvq_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                            const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                            int M, float *y, hipStream_t stream) {
  if (M >= kQ4MfmaMinM) return launch_mfma(w_qs, w_d, N, K, a_qs, a_d, a_s, M, y, stream);
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

}  // namespace skinny
