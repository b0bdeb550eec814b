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
