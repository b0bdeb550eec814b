// mmvq_iq4_xs.hip -- IQ4_XS weights x Q8_1 activations, M = 1..8 rows.
//
// "Machine Learning on NVIDIA CMP" ("llama.cpp results", model table): an
// IQ4_XS model (Qwen3-8B) decodes through the same MMVQ 4-way int8 dot as
// Q4_0.  The pages do not define the format; the arithmetic is the published
// GGUF IQ4_XS one, in a planar byte layout at the same 4.25 bits per weight:
//
//   qs  [N][K/2]       4-bit table indices, Q4_0 nibble order per block of 32
//   hdr [N][K/256][8]  binary16 d; a 16-bit word H holding the high two bits
//                      of the 6-bit scale ls_j of sub-block j at bits
//                      2j..2j+1; a 32-bit word L holding its low four bits
//                      at bits 4j..4j+3
//   weight = d * (ls_j - 32) * T[q],  T the fixed 16-entry IQ4_NL table
//
// Per block b of 32 (one Q8_1 block, sub-block j = b % 8 of its super-block):
//   acc += d (ls_j - 32) d8 isum,  isum = sum T[q] q8  (exact int32)
// T is signed, so no Q8_1 sum term enters.
//
// Decode (iq4.h): a word of four indices becomes four int8 table values
// with three byte permutes.
//
// Large matrices at M >= 6 take the Q4_0 matrix-core kernel instead, with
// the indices decoded through the table into its int8 operands.
//
// Mapping, as the Q4_K vector kernel: one wave = R weight rows over the full
// K; lane l takes blocks l, l + 64, ... in rounds of U blocks, all loaded
// before any is used; the lane's Q8_1 block is loaded once for all R rows; a
// transposing butterfly leaves one output per lane.  A lane always sees
// sub-block j = l % 8, so its scale bits sit at fixed positions; the eight
// lanes of a super-block read its 8-byte header, so one header load
// instruction covers 64 contiguous bytes.
// Bytes per call: N*K*(1/2 + 1/32) weights, M*K*(1 + 2/32) activations (codes
// and d8), 4*M*N output.
#include "device.h"
#include "iq4.h"
#include "launch.h"

namespace skinny {

constexpr int iq4_pow2(int v) { return v <= 1 ? 1 : 2 * iq4_pow2((v + 1) / 2); }

// Leaves one finished output per lane: y[m][n0 + r] for the lane's index.
template <int R, int M>
__device__ __forceinline__ void iq4_store(float (&acc)[R][M], int lane, int n0, int N, float *y) {
  constexpr int V = iq4_pow2(R * M);
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

// (No __restrict__ on the inputs: the issue barrier must be able to keep a
// round's loads ahead of its arithmetic.)
template <int M, int R, int U>
__global__ __launch_bounds__(256) void mmvq_iq4_xs_kernel(
    const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, const int8_t *a_qs,
    const uint16_t *a_d, float *y) {
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6)) * R;
  if (n0 >= N) return;
  const int nb = K >> 5;
  const int j = lane & 7;
  const Iq4Regs kr;

  const uint8_t *wrow[R];
  const uint8_t *hrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(n0 + r, N - 1);          // ragged tail: recompute the last row
    wrow[r] = w_qs + (size_t)n * (size_t)(K >> 1);
    hrow[r] = w_hdr + (size_t)n * (size_t)(K >> 8) * 8;
  }

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  // blocks past the row end load block nb - 1 again and are not accumulated
  for (int b0 = lane; b0 < nb; b0 += U * kWave) {
    uint4_t wq[U][R];
    uint2_t hd[U][R];
    uint4_t aq0[U][M], aq1[U][M];
    uint16_t d8h[U][M];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = min(b0 + u * kWave, nb - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wq[u][r] = load16_nt(wrow[r] + 16 * b);
        hd[u][r] = load8_nt(hrow[r] + 8 * (b >> 3));
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int8_t *ap = a_qs + (size_t)m * K + 32 * b;
        aq0[u][m] = load16(ap);
        aq1[u][m] = load16(ap + 16);
        d8h[u][m] = a_d[(size_t)m * nb + b];
      }
    }
    issue_all();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = b0 + u * kWave < nb;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float dls = iq4_scale(hd[u][r], j);
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) iq4_decode(wq[u][r][i], lo[i], hi[i], kr);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          int32_t isum = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            isum = dot4_i8(lo[i], aq0[u][m][i], isum);
            isum = dot4_i8(hi[i], aq1[u][m][i], isum);
          }
          const float a = fmaf(dls * f16_bits_to_f32(d8h[u][m]), (float)isum, acc[r][m]);
          acc[r][m] = live ? a : acc[r][m];
        }
      }
    }
  }
  iq4_store<R, M>(acc, lane, n0, N, y);
}

// The Q8_1 activation rows staged in LDS once per workgroup (M >= 3): codes
// int8 [M][K], then d8 float [M][K/32].  The plain kernel re-reads each
// lane's activation blocks from L2 for every R rows; here a workgroup of W
// waves loads them once.  Activation loads are issued first, then the
// wave's first round of weights; the first staging batch is stored while
// the weights are in flight, one barrier, then rounds of one block per lane
// with the next round's weights in flight.  Per block the arithmetic is the
// plain kernel's, in the same order.
template <int M, int R, int W, int A>
__global__ __launch_bounds__(64 * W) void mmvq_iq4_xs_lds_kernel(
    const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, const int8_t *a_qs,
    const uint16_t *a_d, float *y) {
  extern __shared__ uint4_t smem4[];
  int8_t *lq = reinterpret_cast<int8_t *>(smem4);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // row addresses stay scalar
  const int nb = K >> 5;
  const int j = lane & 7;
  const Iq4Regs kr;
  float *ld8 = reinterpret_cast<float *>(lq + M * K);
  const int n0 = (blockIdx.x * W + wave) * R;
  // 16-byte pieces: codes (M K / 16), then d8 (M nb / 8, eight blocks each)
  const int ncode = M * K / 16, npieces = ncode + M * nb / 8;
  auto piece = [&](int p) {
    return p < ncode ? reinterpret_cast<const uint8_t *>(a_qs) + 16 * (size_t)p
                     : reinterpret_cast<const uint8_t *>(a_d) + 16 * (size_t)(p - ncode);
  };
  uint4_t av[A];
#pragma unroll
  for (int a = 0; a < A; ++a) av[a] = load16(piece(min(tid + a * W * kWave, npieces - 1)));
  issue_fence();

  const int nw = min(n0, N - 1);            // waves past N read row N - 1 and store nothing
  const uint8_t *wrow[R];
  const uint8_t *hrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(nw + r, N - 1);
    wrow[r] = w_qs + (size_t)n * (size_t)(K >> 1);
    hrow[r] = w_hdr + (size_t)n * (size_t)(K >> 8) * 8;
  }
  struct Round {
    uint4_t wq[R];
    uint2_t hd[R];
  };
  auto load = [&](int b0, Round &rd) {
    const int b = min(b0, nb - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      rd.wq[r] = load16_nt(wrow[r] + 16 * b);
      rd.hd[r] = load8_nt(hrow[r] + 8 * (b >> 3));
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
        float *dst = ld8 + 8 * (p - ncode);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dst[e] = f16_bits_to_f32((uint16_t)(av[a][e >> 1] >> (16 * (e & 1))));
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
  auto compute = [&](int b0, const Round &rd) {
    const int b = min(b0, nb - 1);
    const bool live = b0 < nb;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float dls = iq4_scale(rd.hd[r], j);
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) iq4_decode(rd.wq[r][i], lo[i], hi[i], kr);
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
        const float a = fmaf(dls * ld8[m * nb + b], (float)isum, acc[r][m]);
        acc[r][m] = live ? a : acc[r][m];
      }
    }
  };
  // rounds b0 = lane, lane + 64, ...: the two round buffers alternate
  for (int b0 = lane; b0 < nb; b0 += 2 * kWave) {
    if (b0 + kWave < nb) load(b0 + kWave, r1);
    issue_fence();
    compute(b0, r0);
    if (b0 + kWave >= nb) break;
    if (b0 + 2 * kWave < nb) load(b0 + 2 * kWave, r0);
    issue_fence();
    compute(b0 + kWave, r1);
  }
  iq4_store<R, M>(acc, lane, n0, N, y);
}

template <int M, int R, int U>
static hipError_t launch_iq4_mru(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                          const int8_t *a_qs, const uint16_t *a_d, float *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  hipLaunchKernelGGL((mmvq_iq4_xs_kernel<M, R, U>), dim3((waves + 3) / 4), dim3(256), 0, stream,
                     w_qs, w_hdr, N, K, a_qs, a_d, y);
  return hipGetLastError();
}

// Launch shapes measured on MI355X over the Qwen3-8B projections (K x N
// 4096 x 6144, 4096 x 4096, 4096 x 24576, 12288 x 4096) at M = 1, 2, 4, 8
// with weights rotating over > 1 GiB.  At M = 1 a lane takes its whole share
// of a row in one round up to 8 blocks (K <= 16384; longer rows take rounds
// of 6), but wide matrices with short rows one block per round (4096 x
// 24576: 12.3 -> 11.4 us against two blocks and four rows per wave); at M = 2
// rounds of two blocks up to K = 12288 (12288 x 4096 8.8 -> 8.4 us against
// one round of six), four rows per wave on wide matrices; wider M one block
// per round, four rows per wave on wide matrices.
template <int M>
static hipError_t launch_iq4_m(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                        const int8_t *a_qs, const uint16_t *a_d, float *y, hipStream_t stream) {
  const int per_lane = ((K >> 5) + kWave - 1) / kWave;
#define SKINNY_IQ4(R, U) return launch_iq4_mru<M, R, U>(w_qs, w_hdr, N, K, a_qs, a_d, y, stream)
  if constexpr (M == 1) {
    // one round of exactly the lane's share of the row: a padding slot in
    // the round would cost a block's decode for nothing (K = 5120 and 13824
    // had a quarter and an eighth of their rounds padded with rounds of 4
    // and 8)
    switch (per_lane) {
      case 1:
      case 2:
        if (N >= 16384) SKINNY_IQ4(2, 1);
        SKINNY_IQ4(2, 2);
      case 3: SKINNY_IQ4(2, 3);
      case 4: SKINNY_IQ4(2, 4);
      case 5: SKINNY_IQ4(2, 5);
      case 6: SKINNY_IQ4(2, 6);
      case 7: SKINNY_IQ4(2, 7);
      case 8: SKINNY_IQ4(2, 8);
      default: SKINNY_IQ4(2, 6);
    }
  } else if constexpr (M == 2) {
    if (per_lane <= 2 && N >= 16384) SKINNY_IQ4(4, 2);
    if (per_lane <= 6) SKINNY_IQ4(2, 2);
    if (per_lane > 8) SKINNY_IQ4(2, 6);
    SKINNY_IQ4(2, 8);
  } else {
    if (N >= 16384) SKINNY_IQ4(4, 1);
    SKINNY_IQ4(2, 1);
  }
#undef SKINNY_IQ4
}

constexpr int kIq4LdsMaxBytes = 160 * 1024;

static int iq4_lds_bytes(int M, int K) { return M * K + 4 * M * (K >> 5); }

template <int M, int R, int W, int A>
static hipError_t launch_iq4_lds_a(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                            const int8_t *a_qs, const uint16_t *a_d, float *y,
                            hipStream_t stream) {
  const int lds = iq4_lds_bytes(M, K);
  const hipError_t lds_ok = allow_lds((const void *)mmvq_iq4_xs_lds_kernel<M, R, W, A>, lds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int rows = R * W;
  hipLaunchKernelGGL((mmvq_iq4_xs_lds_kernel<M, R, W, A>), dim3((N + rows - 1) / rows),
                     dim3(64 * W), lds, stream, w_qs, w_hdr, N, K, a_qs, a_d, y);
  return hipGetLastError();
}

template <int M, int R, int W>
static hipError_t launch_iq4_lds_rw(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                             const int8_t *a_qs, const uint16_t *a_d, float *y,
                             hipStream_t stream) {
  const int pieces = M * K / 16 + M * (K >> 5) / 8;
  const int per_thread = (pieces + 64 * W - 1) / (64 * W);   // first staging batch
#define SKINNY_IQ4L(A) \
  return launch_iq4_lds_a<M, R, W, A>(w_qs, w_hdr, N, K, a_qs, a_d, y, stream)
  if (per_thread <= 4) SKINNY_IQ4L(4);
  if (per_thread <= 8) SKINNY_IQ4L(8);
  SKINNY_IQ4L(16);
#undef SKINNY_IQ4L
}

template <int M>
static hipError_t launch_iq4_lds(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                          const int8_t *a_qs, const uint16_t *a_d, float *y, hipStream_t stream) {
  return launch_iq4_lds_rw<M, 2, 8>(w_qs, w_hdr, N, K, a_qs, a_d, y, stream);
}

hipError_t launch_mmvq_iq4_xs(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                              const int8_t *a_qs, const uint16_t *a_d, int M, float *y,
                              hipStream_t stream) {
  // From M = 6 large matrices take the matrix cores (the Q4_0 kernel with
  // table-decoded operands; measured on MI355X at M = 8: 4096 x 24576
  // 22.2 -> 18.6 us, 5120 x 13824 21.9 -> 15.4 us, 13824 x 5120 27.0 -> 20.1
  // us, 8192 x 8192 16.9 -> 14.4 us, 12288 x 4096 12.5 -> 11.9 us; below 48M
  // weights the vector and staged kernels stay ahead at every M, 4096 x 6144
  // 7.9 against 8.3 us)
  if (M >= 6 && (long long)N * K >= (48ll << 20))
    return launch_mmvq_iq4_xs_mfma(w_qs, w_hdr, N, K, a_qs, a_d, M, y, stream);
  // From M = 3 the staged kernel where the activation re-reads weigh most:
  // long rows (12288 x 4096 at M = 4: 10.2 -> 9.4 us, at M = 8: 15.7 -> 12.6
  // us) and, from M = 6, narrow matrices (4096 x 4096 at M = 8); the vector
  // kernel elsewhere (4096 x 6144 at M = 8: 9.4 -> 7.8 us, 4096 x 24576:
  // 23.4 -> 22.4 us against staging).
  if (M >= 3 && (K >= 8192 || (M >= 6 && N <= 4096)) &&
      iq4_lds_bytes(M, K) <= kIq4LdsMaxBytes) {
    switch (M) {
#define SKINNY_IQ4L(MM) \
  case MM: return launch_iq4_lds<MM>(w_qs, w_hdr, N, K, a_qs, a_d, y, stream);
      SKINNY_IQ4L(3) SKINNY_IQ4L(4) SKINNY_IQ4L(5) SKINNY_IQ4L(6) SKINNY_IQ4L(7)
#undef SKINNY_IQ4L
      default: return launch_iq4_lds<8>(w_qs, w_hdr, N, K, a_qs, a_d, y, stream);
    }
  }
  switch (M) {
#define SKINNY_IQ4(MM) \
  case MM: return launch_iq4_m<MM>(w_qs, w_hdr, N, K, a_qs, a_d, y, stream);
    SKINNY_IQ4(1) SKINNY_IQ4(2) SKINNY_IQ4(3) SKINNY_IQ4(4)
    SKINNY_IQ4(5) SKINNY_IQ4(6) SKINNY_IQ4(7)
#undef SKINNY_IQ4
    default: return launch_iq4_m<8>(w_qs, w_hdr, N, K, a_qs, a_d, y, stream);
  }
}

}  // namespace skinny
