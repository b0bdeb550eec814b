// gemv_fp8.hip -- FP8 E4M3 weights x binary16 activations, M = 1..8 rows,
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
// transposing butterfly for the R*M partial sums at the end.
// Bytes per call: N*K + 4*N weights and scales + 2*M*K + 2*M*N.
#include "device.h"
#include "launch.h"

namespace skinny {

// Activation rows from which the matrix-core kernel is used.
constexpr int kFp8MfmaMinM = 3;

constexpr int next_pow2_f(int v) { return v <= 1 ? 1 : 2 * next_pow2_f((v + 1) / 2); }

template <int M, int R>
__global__ __launch_bounds__(256) void gemv_fp8_kernel(
    const uint8_t *__restrict__ w, const float *__restrict__ cs, int N, int K,
    const uint16_t *__restrict__ x, uint16_t *__restrict__ y) {
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

#pragma unroll 2
  for (int c = lane; c < nc; c += kWave) {
    uint4_t wq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wq[r] = load16_nt(wrow[r] + 16 * c);
    uint4_t xv[M][2];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint16_t *xp = x + (size_t)m * K + 16 * c;
      xv[m][0] = load16(xp);
      xv[m][1] = load16(xp + 8);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // word i holds elements 4i..4i+3: pair (4i, 4i+1) and (4i+2, 4i+3)
      uint32_t wh[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wh[2 * i + 0] = __builtin_bit_cast(uint32_t, e4m3x2_to_h2<false>(wq[r][i]));
        wh[2 * i + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_h2<true>(wq[r][i]));
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a = acc[r][m];
#pragma unroll
        for (int p = 0; p < 8; ++p) a = dot2_f16(wh[p], xv[m][p >> 2][p & 3], a);
        acc[r][m] = a;
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

// Matrix-core variant (any M <= 8).
//
// A workgroup of W waves owns T tiles of 16 weight rows; each wave takes a
// contiguous range of K.  The weights are read row-contiguously (64 lanes x
// 16 bytes covering 512 bytes of each of two rows per instruction) into
// registers, written to a wave-private LDS buffer and read back in the
// matrix-core operand layout: lane l = (i = l % 16, g = l / 16) takes 32
// bytes of row 16t + i (elements k0 .. k0+31, k0 = 128 s + 32 g), decodes
// them exactly to binary16 and feeds four v_mfma_f32_16x16x32_f16 whose B
// operands are x[i][k0 + 8t .. +8], kept four steps ahead in a register
// ring by the lanes with i < M.  Float32 accumulation across K; the channel
// scale multiplies the finished sum.  The next chunk of weights is in
// flight while the current one is consumed; steps past the last whole chunk
// (the final one possibly partial, K being a multiple of 16 only) are read
// directly in the operand layout.  The W partial tiles are summed in LDS.
__device__ __forceinline__ void fp8_step(const uint4_t (&wq)[2], const uint4_t (&xv)[4],
                                         float4_t &acc) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t w0 = wq[t >> 1][2 * (t & 1)];
    const uint32_t w1 = wq[t >> 1][2 * (t & 1) + 1];
    const half2_t h0 = e4m3x2_to_h2<false>(w0);
    const half2_t h1 = e4m3x2_to_h2<true>(w0);
    const half2_t h2 = e4m3x2_to_h2<false>(w1);
    const half2_t h3 = e4m3x2_to_h2<true>(w1);
    const half8_t a = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
    acc = mfma_16x16x32_f16(a, __builtin_bit_cast(half8_t, xv[t]), acc);
  }
}

namespace f8 {
constexpr int kCh = 4;                 // 128-element steps per staged chunk
constexpr int kRowB = kCh * 128;       // weight bytes per row per chunk (512)
constexpr int kRowP = kRowB + 16;      // padded LDS pitch
constexpr int kXr = 4;                 // activation steps kept in flight
template <int T>
constexpr int wave_lds() { return 16 * T * kRowP; }
}  // namespace f8

template <int W, int T>
__global__ __launch_bounds__(64 * W) void gemv_fp8_mfma_kernel(
    const uint8_t *__restrict__ w, const float *__restrict__ cs, int N, int K,
    const uint16_t *__restrict__ x, int M, uint16_t *__restrict__ y) {
  using namespace f8;
  constexpr int ROWS = 16 * T;
  constexpr int CLD = ROWS / 2;        // 1 KB loads per chunk (2 rows each)
  extern __shared__ uint4_t smem4[];
  uint8_t *smem = reinterpret_cast<uint8_t *>(smem4);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * ROWS;
  uint8_t *wl = smem + wave * wave_lds<T>();
  float4_t *red = reinterpret_cast<float4_t *>(smem + W * wave_lds<T>());

  const uint8_t *wg[CLD];
#pragma unroll
  for (int q = 0; q < CLD; ++q)
    wg[q] = w + (size_t)min(n0 + 2 * q + (lane >> 5), N - 1) * (size_t)K + 16 * (lane & 31);

  const bool xact = i < M;
  const uint16_t *xrow = x + (size_t)(xact ? i : 0) * (size_t)K + 32 * grp;
  const int nsteps = (K + 127) >> 7;
  const int nchunks = K / kRowB;
  const int per = (nchunks + W - 1) / W;
  const int c0 = min(nchunks, wave * per), c1 = min(nchunks, c0 + per);

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

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
  uint4_t cr[CLD];
  if (c0 < c1) {
#pragma unroll
    for (int q = 0; q < CLD; ++q) cr[q] = load16_nt(wg[q] + (size_t)c0 * kRowB);
  }
  for (int c = c0; c < c1; ++c) {
#pragma unroll
    for (int q = 0; q < CLD; ++q)
      *reinterpret_cast<uint4_t *>(wl + (2 * q + (lane >> 5)) * kRowP + 16 * (lane & 31)) = cr[q];
    if (c + 1 < c1) {
#pragma unroll
      for (int q = 0; q < CLD; ++q) cr[q] = load16_nt(wg[q] + (size_t)(c + 1) * kRowB);
    }
#pragma unroll
    for (int st = 0; st < kCh; ++st) {
      const int slot = st % kXr;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint8_t *src = wl + (16 * t + i) * kRowP + 128 * st + 32 * grp;
        const uint4_t wq[2] = {*reinterpret_cast<const uint4_t *>(src),
                               *reinterpret_cast<const uint4_t *>(src + 16)};
        fp8_step(wq, xr[slot], acc[t]);
      }
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
      uint4_t xv[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
      bool hact[2];
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        hact[hlf] = 128 * s + 32 * grp + 16 * hlf < K;
        if (hact[hlf] && xact) {
          xv[2 * hlf] = load16(xrow + 128 * s + 16 * hlf);
          xv[2 * hlf + 1] = load16(xrow + 128 * s + 16 * hlf + 8);
        }
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint8_t *row = w + (size_t)min(n0 + 16 * t + i, N - 1) * (size_t)K + 32 * grp;
        uint4_t wq[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf)
          if (hact[hlf]) wq[hlf] = load16_nt(row + 128 * s + 16 * hlf);
        fp8_step(wq, xv, acc[t]);
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
        if (n < N) y[(size_t)i * N + n] = f32_to_f16_bits(tot[r] * cs[n]);
      }
    }
  }
}

template <int W, int T>
static hipError_t launch_mfma_wt(const uint8_t *w, const float *cs, int N, int K,
                                 const uint16_t *x, int M, uint16_t *y, hipStream_t stream) {
  const int blocks = (N + 16 * T - 1) / (16 * T);
  const size_t shmem = (size_t)W * f8::wave_lds<T>() + sizeof(float4_t) * W * T * kWave;
  hipLaunchKernelGGL((gemv_fp8_mfma_kernel<W, T>), dim3(blocks), dim3(64 * W), shmem, stream,
                     w, cs, N, K, x, M, y);
  return hipGetLastError();
}

// Tiles per wave T (weight rows sharing one activation operand) and waves
// per workgroup W (K split), W * T <= 4 so the staging buffers fit in 64 KB
// of LDS.  Measured on MI355X at M = 4 and 8: two tiles without K split for
// wide matrices, one tile and two K splits otherwise.
static void pick_tw(int N, int K, int &T, int &W) {
  (void)K;
  const int tiles = (N + 15) / 16;
  if (tiles >= 2000) { T = 2; W = 1; }
  else { T = 1; W = 2; }
}

static hipError_t launch_mfma(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                              int M, uint16_t *y, hipStream_t stream) {
  int T, W;
  pick_tw(N, K, T, W);
#define SKINNY_F8_CASE(TT, WW) \
  if (T == TT && W == WW) return launch_mfma_wt<WW, TT>(w, cs, N, K, x, M, y, stream);
  SKINNY_F8_CASE(1, 1) SKINNY_F8_CASE(1, 2) SKINNY_F8_CASE(1, 4)
  SKINNY_F8_CASE(2, 1) SKINNY_F8_CASE(2, 2)
#undef SKINNY_F8_CASE
  return hipErrorInvalidValue;
}

template <int M, int R>
static hipError_t launch_mr(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                            uint16_t *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((gemv_fp8_kernel<M, R>), dim3(blocks), dim3(256), 0, stream,
                     w, cs, N, K, x, y);
  return hipGetLastError();
}

// Two rows per wave: few 128-bit weight loads in flight per lane and many
// waves measured best on MI355X at M <= 2 for every shape tried (K 4096 to
// 17408, N 4096 to 34816); four or eight rows only pay once the activation
// block is reused across more rows, which is where the matrix-core kernel
// takes over.
static int rows_per_wave(int N, int M) {
  (void)N;
  return M <= 2 ? 2 : 4;
}

template <int M>
static hipError_t launch_m(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                           uint16_t *y, hipStream_t stream) {
  switch (rows_per_wave(N, M)) {
    case 2: return launch_mr<M, 2>(w, cs, N, K, x, y, stream);
    case 4: return launch_mr<M, 4>(w, cs, N, K, x, y, stream);
    default: return launch_mr<M, 8>(w, cs, N, K, x, y, stream);
  }
}

hipError_t launch_gemv_fp8(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                           int M, uint16_t *y, hipStream_t stream) {
  if (M >= kFp8MfmaMinM) return launch_mfma(w, cs, N, K, x, M, y, stream);
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

}  // namespace skinny
