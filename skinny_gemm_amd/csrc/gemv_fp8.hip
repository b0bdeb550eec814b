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
    for (int r = 0; r < R; ++r) wq[r] = load16(wrow[r] + 16 * c);
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

template <int M, int R>
static hipError_t launch_mr(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                            uint16_t *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((gemv_fp8_kernel<M, R>), dim3(blocks), dim3(256), 0, stream,
                     w, cs, N, K, x, y);
  return hipGetLastError();
}

static int rows_per_wave(int N) {
  int r = 2;
  while (r < 8 && N / (2 * r) >= 2048) r *= 2;
  return r;
}

template <int M>
static hipError_t launch_m(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                           uint16_t *y, hipStream_t stream) {
  switch (rows_per_wave(N)) {
    case 2: return launch_mr<M, 2>(w, cs, N, K, x, y, stream);
    case 4: return launch_mr<M, 4>(w, cs, N, K, x, y, stream);
    default: return launch_mr<M, 8>(w, cs, N, K, x, y, stream);
  }
}

hipError_t launch_gemv_fp8(const uint8_t *w, const float *cs, int N, int K, const uint16_t *x,
                           int M, uint16_t *y, hipStream_t stream) {
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
