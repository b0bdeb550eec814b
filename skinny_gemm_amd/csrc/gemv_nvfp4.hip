// gemv_nvfp4.hip -- NVFP4 weights (E2M1 codes, E4M3 scale per 16 elements,
// float32 per-tensor scale) x binary16 activations, M = 1..8 rows.
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
// Bytes per call: N*K*(1/2 + 1/16) weights + 2*M*K activations + 2*M*N out.
#include "device.h"
#include "launch.h"

namespace skinny {

// Activation rows from which the matrix-core kernel is used.
constexpr int kNvfp4MfmaMinM = 3;

constexpr int next_pow2_n(int v) { return v <= 1 ? 1 : 2 * next_pow2_n((v + 1) / 2); }

template <int M, int R>
__global__ __launch_bounds__(256) void gemv_nvfp4_kernel(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, float g,
    int N, int K, const uint16_t *__restrict__ x, uint16_t *__restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6)) * R;
  if (n0 >= N) return;
  const int nc = K >> 5;                    // 32-element chunks per row

  const uint8_t *crow[R];
  const uint8_t *srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(n0 + r, N - 1);
    crow[r] = codes + (size_t)n * (size_t)(K >> 1);
    srow[r] = scales + (size_t)n * (size_t)(K >> 4);
  }

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

#pragma unroll 2
  for (int c = lane; c < nc; c += kWave) {
    uint4_t wq[R];
    uint32_t sc2[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wq[r] = load16(crow[r] + 16 * c);
      sc2[r] = *reinterpret_cast<const uint16_t *>(srow[r] + 2 * c);
    }
    // activations of the chunk: 32 binary16 = 16 pairs per row m
    uint4_t xv[M][4];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint16_t *xp = x + (size_t)m * K + 32 * c;
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[m][q] = load16(xp + 8 * q);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // decode: word i, byte j -> elements 8i+2j (low nibble), 8i+2j+1
      uint32_t wh[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wh[4 * i + 0] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<0>(wq[r][i]));
        wh[4 * i + 1] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<1>(wq[r][i]));
        wh[4 * i + 2] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<2>(wq[r][i]));
        wh[4 * i + 3] = __builtin_bit_cast(uint32_t, e2m1x2_to_h2<3>(wq[r][i]));
      }
      const float s0 = e4m3_to_f32<0>(sc2[r]) * g;
      const float s1 = e4m3_to_f32<1>(sc2[r]) * g;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        // pair p (0..15) of the chunk is dword p%4 of xv[m][p/4]
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int p = 0; p < 8; ++p) p0 = dot2_f16(wh[p], xv[m][p >> 2][p & 3], p0);
#pragma unroll
        for (int p = 8; p < 16; ++p) p1 = dot2_f16(wh[p], xv[m][p >> 2][p & 3], p1);
        acc[r][m] = fmaf(p0, s0, acc[r][m]);
        acc[r][m] = fmaf(p1, s1, acc[r][m]);
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

// Matrix-core variant (any M <= 8).
//
// A workgroup of W waves owns T tiles of 16 weight rows; each wave takes a
// contiguous range of K.  The weight stream is read row-contiguously -- one
// 128-bit load per lane, 64 lanes covering 1 KB of a single row per
// instruction, which the memory system serves at close to streaming rate --
// into registers, then written to a wave-private LDS buffer (rows padded
// against bank conflicts) and read back in the matrix-core operand layout:
// lane l = (i = l % 16, g = l / 16) takes 16 code bytes of row 16t + i
// (elements k0 .. k0+31, k0 = 128 s + 32 g) and the two group scales, and
// decodes them two at a time to binary16 times the binary16 group scale --
// exact, as an E2M1 value times an E4M3 value has at most 5 significant
// bits and lies in [2^-10, 2688] -- giving the A operands of four
// v_mfma_f32_16x16x32_f16.  The B operands are the activations
// x[i][k0 + 8t .. +8], loaded four steps ahead into a register ring by the
// lanes with i < M (the other lanes' columns are never stored).  The matrix core accumulates in
// float32 across all of K, so no binary16 partial sum exists anywhere; the
// per-tensor scale is applied to the finished float32 sum.  The next chunk
// of weights is in flight while the current one is consumed.  Steps past
// the last whole chunk are read directly in the operand layout.  The W
// partial tiles are summed through LDS.
__device__ __forceinline__ void nvfp4_step(const uint4_t &wq, uint32_t sc, const uint4_t (&xv)[4],
                                           float4_t &acc) {
  const half2_t s0 = h2_bcast(e4m3_to_f32<0>(sc));
  const half2_t s1 = h2_bcast(e4m3_to_f32<1>(sc));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const half2_t st = t < 2 ? s0 : s1;
    const half2_t h0 = e2m1x2_to_h2<0>(wq[t]) * st;
    const half2_t h1 = e2m1x2_to_h2<1>(wq[t]) * st;
    const half2_t h2 = e2m1x2_to_h2<2>(wq[t]) * st;
    const half2_t h3 = e2m1x2_to_h2<3>(wq[t]) * st;
    const half8_t a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
    acc = mfma_16x16x32_f16(a, __builtin_bit_cast(half8_t, xv[t]), acc);
  }
}

namespace nv {
constexpr int kCh = 8;                 // 128-element steps per staged chunk
constexpr int kRowB = kCh * 64;        // code bytes per row per chunk (512)
constexpr int kSclB = kCh * 8;         // scale bytes per row per chunk (64)
constexpr int kRowP = kRowB + 16;      // padded LDS pitches
constexpr int kSclP = kSclB + 16;
constexpr int kXr = 4;                 // activation steps kept in flight
template <int T>
constexpr int wave_lds() { return 16 * T * (kRowP + kSclP); }
}  // namespace nv

template <int W, int T>
__global__ __launch_bounds__(64 * W) void gemv_nvfp4_mfma_kernel(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, float g,
    int N, int K, const uint16_t *__restrict__ x, int M, uint16_t *__restrict__ y) {
  using namespace nv;
  constexpr int ROWS = 16 * T;
  constexpr int CLD = ROWS / 2;        // 1 KB code loads per chunk (2 rows each)
  constexpr int SLD = T;               // 1 KB scale loads per chunk (16 rows each)
  extern __shared__ uint4_t smem4[];
  uint8_t *smem = reinterpret_cast<uint8_t *>(smem4);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * ROWS;
  uint8_t *cl = smem + wave * wave_lds<T>();
  uint8_t *sl = cl + ROWS * kRowP;
  float4_t *red = reinterpret_cast<float4_t *>(smem + W * wave_lds<T>());

  const size_t rowc = (size_t)(K >> 1), rows_ = (size_t)(K >> 4);
  // row-contiguous load mapping: codes, lane -> (row 2q + lane/32, bytes 16 (lane%32));
  // scales, lane -> (row 16q + lane/4, bytes 16 (lane%4))
  const uint8_t *cg[CLD];
  const uint8_t *sg[SLD];
#pragma unroll
  for (int q = 0; q < CLD; ++q)
    cg[q] = codes + (size_t)min(n0 + 2 * q + (lane >> 5), N - 1) * rowc + 16 * (lane & 31);
#pragma unroll
  for (int q = 0; q < SLD; ++q)
    sg[q] = scales + (size_t)min(n0 + 16 * q + (lane >> 2), N - 1) * rows_ + 16 * (lane & 3);

  const bool xact = i < M;
  const uint16_t *xrow = x + (size_t)(xact ? i : 0) * (size_t)K + 32 * grp;
  const int nsteps = (K + 127) >> 7;
  // staged chunks need 16-byte aligned scale rows (K % 256 == 0)
  const int nchunks = (K % 256 == 0) ? K / (128 * kCh) : 0;
  const int per = (nchunks + W - 1) / W;
  const int c0 = min(nchunks, wave * per), c1 = min(nchunks, c0 + per);

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  // activations for the next kXr steps, kept in a ring of registers
  uint4_t xr[kXr][4];
#pragma unroll
  for (int d = 0; d < kXr; ++d) {
#pragma unroll
    for (int q = 0; q < 4; ++q) xr[d][q] = uint4_t{0u, 0u, 0u, 0u};
    if (xact && c0 * kCh + d < c1 * kCh) {
#pragma unroll
      for (int q = 0; q < 4; ++q) xr[d][q] = load16(xrow + 128 * (c0 * kCh + d) + 8 * q);
    }
  }
  uint4_t cr[CLD], sr[SLD];
  if (c0 < c1) {
#pragma unroll
    for (int q = 0; q < CLD; ++q) cr[q] = load16_nt(cg[q] + (size_t)c0 * kRowB);
#pragma unroll
    for (int q = 0; q < SLD; ++q) sr[q] = load16_nt(sg[q] + (size_t)c0 * kSclB);
  }
  for (int c = c0; c < c1; ++c) {
#pragma unroll
    for (int q = 0; q < CLD; ++q)
      *reinterpret_cast<uint4_t *>(cl + (2 * q + (lane >> 5)) * kRowP + 16 * (lane & 31)) = cr[q];
#pragma unroll
    for (int q = 0; q < SLD; ++q)
      *reinterpret_cast<uint4_t *>(sl + (16 * q + (lane >> 2)) * kSclP + 16 * (lane & 3)) = sr[q];
    if (c + 1 < c1) {
#pragma unroll
      for (int q = 0; q < CLD; ++q) cr[q] = load16_nt(cg[q] + (size_t)(c + 1) * kRowB);
#pragma unroll
      for (int q = 0; q < SLD; ++q) sr[q] = load16_nt(sg[q] + (size_t)(c + 1) * kSclB);
    }
#pragma unroll
    for (int st = 0; st < kCh; ++st) {
      const int slot = st % kXr;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint4_t wq = *reinterpret_cast<const uint4_t *>(cl + (16 * t + i) * kRowP + 64 * st + 16 * grp);
        const uint32_t sc = *reinterpret_cast<const uint16_t *>(sl + (16 * t + i) * kSclP + 8 * st + 2 * grp);
        nvfp4_step(wq, sc, xr[slot], acc[t]);
      }
      // refill this slot with the activations kXr steps ahead
      const int ahead = c * kCh + st + kXr;
      if (xact && ahead < c1 * kCh) {
#pragma unroll
        for (int q = 0; q < 4; ++q) xr[slot][q] = load16(xrow + 128 * ahead + 8 * q);
      }
    }
  }
  // steps past the last whole chunk, read in the operand layout (last wave)
  if (wave == W - 1) {
    for (int s = nchunks * kCh; s < nsteps; ++s) {
      const bool kact = 128 * s + 32 * grp < K;
      uint4_t xv[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
      if (kact && xact) {
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[q] = load16(xrow + 128 * s + 8 * q);
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int nrow = min(n0 + 16 * t + i, N - 1);
        uint4_t wq = {0u, 0u, 0u, 0u};
        uint32_t sc = 0;
        if (kact) {
          wq = load16_nt(codes + (size_t)nrow * rowc + 64 * s + 16 * grp);
          sc = load_u16_nt(reinterpret_cast<const uint16_t *>(scales + (size_t)nrow * rows_) +
                           4 * s + grp);
        }
        nvfp4_step(wq, sc, xv, acc[t]);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < T; ++t) red[(wave * T + t) * kWave + lane] = acc[t];
  __syncthreads();
  if (wave == 0 && xact) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float4_t tot = red[t * kWave + lane];
#pragma unroll
      for (int v = 1; v < W; ++v) tot += red[(v * T + t) * kWave + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 16 * t + 4 * grp + r;
        if (n < N) y[(size_t)i * N + n] = f32_to_f16_bits(tot[r] * g);
      }
    }
  }
}

template <int W, int T>
static hipError_t launch_mfma_wt(const uint8_t *codes, const uint8_t *scales, float g, int N,
                                 int K, const uint16_t *x, int M, uint16_t *y,
                                 hipStream_t stream) {
  const int blocks = (N + 16 * T - 1) / (16 * T);
  const size_t shmem = (size_t)W * nv::wave_lds<T>() + sizeof(float4_t) * W * T * kWave;
  hipLaunchKernelGGL((gemv_nvfp4_mfma_kernel<W, T>), dim3(blocks), dim3(64 * W), shmem, stream,
                     codes, scales, g, N, K, x, M, y);
  return hipGetLastError();
}

// Tiles per wave T (weight rows sharing one activation operand) and waves
// per workgroup W (K split), W * T <= 4 so the staging buffers fit in 64 KB
// of LDS.  Measured on MI355X at M = 4 and 8: wide matrices prefer two
// tiles and few K splits, narrow ones four K splits.
static void pick_tw(int N, int K, int &T, int &W) {
  (void)K;
  const int tiles = (N + 15) / 16;
  if (tiles >= 2000) { T = 2; W = 1; }
  else if (tiles >= 1024) { T = 2; W = 2; }
  else { T = 1; W = 4; }
}

static hipError_t launch_mfma(const uint8_t *codes, const uint8_t *scales, float g, int N,
                              int K, const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  int T, W;
  pick_tw(N, K, T, W);
#define SKINNY_NV_CASE(TT, WW) \
  if (T == TT && W == WW) return launch_mfma_wt<WW, TT>(codes, scales, g, N, K, x, M, y, stream);
  SKINNY_NV_CASE(1, 1) SKINNY_NV_CASE(1, 2) SKINNY_NV_CASE(1, 4)
  SKINNY_NV_CASE(2, 1) SKINNY_NV_CASE(2, 2)
#undef SKINNY_NV_CASE
  return hipErrorInvalidValue;
}

template <int M, int R>
static hipError_t launch_mr(const uint8_t *codes, const uint8_t *scales, float g, int N, int K,
                            const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((gemv_nvfp4_kernel<M, R>), dim3(blocks), dim3(256), 0, stream,
                     codes, scales, g, N, K, x, y);
  return hipGetLastError();
}

static int rows_per_wave(int N) {
  int r = 2;
  while (r < 8 && N / (2 * r) >= 2048) r *= 2;
  return r;
}

template <int M>
static hipError_t launch_m(const uint8_t *codes, const uint8_t *scales, float g, int N, int K,
                           const uint16_t *x, uint16_t *y, hipStream_t stream) {
  switch (rows_per_wave(N)) {
    case 2: return launch_mr<M, 2>(codes, scales, g, N, K, x, y, stream);
    case 4: return launch_mr<M, 4>(codes, scales, g, N, K, x, y, stream);
    default: return launch_mr<M, 8>(codes, scales, g, N, K, x, y, stream);
  }
}

hipError_t launch_gemv_nvfp4(const uint8_t *codes, const uint8_t *scales, float g, int N, int K,
                             const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  if (M >= kNvfp4MfmaMinM) return launch_mfma(codes, scales, g, N, K, x, M, y, stream);
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

}  // namespace skinny
