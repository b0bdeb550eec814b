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

constexpr int next_pow2(int v) { return v <= 1 ? 1 : 2 * next_pow2((v + 1) / 2); }

template <int M, int R>
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
      wq[r] = load16(wrow[r] + 16 * b);
      d4[r] = f16_bits_to_f32(drow[r][b]);
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

template <int M, int R>
static hipError_t launch_mr(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                            const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                            float *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((mmvq_q4_0_kernel<M, R>), dim3(blocks), dim3(256), 0, stream,
                     w_qs, w_d, N, K, a_qs, a_d, a_s, y);
  return hipGetLastError();
}

// Rows per wave: enough waves to fill 256 CUs several times over, and at
// most 64 partial sums per lane.
static int rows_per_wave(int N, int M) {
  const int rmax = M <= 4 ? 8 : (M <= 8 ? 8 : 4);
  int r = 2;
  while (r < rmax && N / (2 * r) >= 2048) r *= 2;
  return r;
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
