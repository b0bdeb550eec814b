// mmvq_kquant.hip -- K-quant weights (Q4_K, Q6_K) x Q8_1 activations,
// M = 1..8 rows.
//
// "Machine Learning on NVIDIA CMP" ("llama.cpp results", model table):
// Q4_K and Q6_K models decode through the same MMVQ 4-way int8 dot as Q4_0.
// The pages do not define these formats; the arithmetic is the published
// GGUF K-quant one (super-blocks of 256 weights with per-sub-block integer
// scales), in planar byte layouts at the same bits per weight:
//
//   Q4_K  qs  [N][K/2]        4-bit codes, Q4_0 nibble order per block of 32
//         hdr [N][K/256][16]  binary16 d, binary16 dmin, then 12 bytes p
//                             holding sc_j = p[j] & 63 and
//                             m_j = (p[j] >> 6) | (nibble j of p[8..11]) << 2
//         weight = d * sc_j * q - dmin * m_j      (sub-block j of 32)
//   Q6_K  ql [N][K/2]   low 4 bits, Q4_0 nibble order per block of 32
//         qh [N][K/4]   high 2 bits: 8 bytes per block, byte 4h + t bits
//                       2c..2c+1 belong to element 16h + 4c + t
//         sc [N][K/16]  int8 scale per sub-block of 16;  d [N][K/256] binary16
//         weight = d * sc_j * (q - 32)
//
// Per block b of 32 (one Q8_1 block, exact int32 block sums):
//   Q4_K: acc += d sc d8 isum - dmin m s8      (the min through the sum term)
//   Q6_K: acc += d d8 (sc_2b isum_lo + sc_2b+1 isum_hi), codes q - 32 formed
//         in registers ((q | 0x80) - 0x20) ^ 0x80 per byte, no borrow.
//
// Mapping, as the Q4_0 vector kernel: one wave = R weight rows over the
// full K; lane l takes blocks b = l, l + 64, ... in rounds of U blocks, all
// loaded before any is used; the lane's Q8_1 block is loaded once and reused
// for all R rows; a transposing butterfly leaves one output per lane.  Since
// 64 is a multiple of 8, a lane always sees sub-block j = l % 8 of a Q4_K
// super-block, so its scale/min bit positions are fixed per lane.
// Bytes per call: Q4_K N*K*(1/2 + 1/16) + Q6_K N*K*(1/2 + 1/4 + 1/16 + 1/128),
// plus M*K*(1 + 4/32) (Q4_K) or M*K*(1 + 2/32) (Q6_K) activations and
// 4*M*N output.
#include "device.h"
#include "launch.h"

namespace skinny {

constexpr int kq_pow2(int v) { return v <= 1 ? 1 : 2 * kq_pow2((v + 1) / 2); }

// Leaves one finished output per lane: y[m][n0 + r] for the lane's index.
template <int R, int M>
__device__ __forceinline__ void kq_store(float (&acc)[R][M], int lane, int n0, int N, float *y) {
  constexpr int V = kq_pow2(R * M);
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

// Value of v held by lane Q of the caller's group of four lanes.
template <int Q>
__device__ __forceinline__ uint32_t quad_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Q * 0x55, 0xF, 0xF, false);
}

// (No __restrict__ on the inputs: the issue barrier below must be able to
// keep a round's loads ahead of its arithmetic.)
//
// The eight lanes of a super-block share its 16-byte header, of which each
// lane uses three dwords: 0 (d, dmin), 1 or 2 (its scale/min byte) and 3
// (the high min bits).  Each lane loads one dword -- quad lane 0 dword 0,
// lane 1 dword 1 (first quad of the eight) or 2 (second), lane 2 dword 3 --
// and takes the other two from its quad (a quarter of the bytes of loading
// the whole header per lane).  Rounds start on a multiple of 8 blocks and
// K / 32 is a multiple of 8, so a quad is always entirely in or out of the
// loop.
template <int M, int R, int U>
__global__ __launch_bounds__(256) void mmvq_q4_k_kernel(
    const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, const int8_t *a_qs,
    const uint16_t *a_d, const uint16_t *a_s, float *y) {
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6)) * R;
  if (n0 >= N) return;
  const int nb = K >> 5;

  const uint8_t *wrow[R];
  const uint8_t *hrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(n0 + r, N - 1);          // ragged tail: recompute the last row
    wrow[r] = w_qs + (size_t)n * (size_t)(K >> 1);
    hrow[r] = w_hdr + (size_t)n * (size_t)(K >> 8) * 16;
  }
  // sub-block j = lane % 8: scale/min byte p[j] is header byte 4 + j (dword
  // 1 + j / 4), the high min bits nibble j % 2 of p[8 + j / 2] (dword 3)
  const int j = lane & 7;
  const int s_sh = 8 * (j & 3);
  const int h_sh = 8 * (j >> 1) + 4 * (j & 1);
  const int hq = (lane & 3) == 0 ? 0 : (lane & 3) == 1 ? 1 + (j >> 2) : 3;   // dword loaded

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  // blocks past the row end load block nb - 1 again and are not accumulated
  for (int b0 = lane; b0 < nb; b0 += U * kWave) {
    uint4_t wq[U][R];
    uint32_t hw[U][R];
    uint4_t aq0[U][M], aq1[U][M];
    uint16_t d8h[U][M], s8h[U][M];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = min(b0 + u * kWave, nb - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wq[u][r] = load16_nt(wrow[r] + 16 * b);
        hw[u][r] = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t *>(hrow[r] + 16 * (b >> 3)) + hq);
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
      const bool live = b0 + u * kWave < nb;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t h0 = quad_lane<0>(hw[u][r]);
        const uint32_t pb = quad_lane<1>(hw[u][r]) >> s_sh;
        const uint32_t h3 = quad_lane<2>(hw[u][r]);
        const uint32_t sc = pb & 63u;
        const uint32_t mn = ((pb >> 6) & 3u) | (((h3 >> h_sh) & 15u) << 2);
        const float dsc = f16_bits_to_f32((uint16_t)(h0 & 0xFFFFu)) * (float)sc;
        const float dmm = f16_bits_to_f32((uint16_t)(h0 >> 16)) * (float)mn;
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo[i] = wq[u][r][i] & 0x0F0F0F0Fu;
          hi[i] = (wq[u][r][i] >> 4) & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
          int32_t isum = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            isum = dot4_i8(lo[i], aq0[u][m][i], isum);
            isum = dot4_i8(hi[i], aq1[u][m][i], isum);
          }
          const float t = fmaf(dsc * f16_bits_to_f32(d8h[u][m]), (float)isum,
                               -(dmm * f16_bits_to_f32(s8h[u][m])));
          const float a = acc[r][m] + t;
          acc[r][m] = live ? a : acc[r][m];
        }
      }
    }
  }
  kq_store<R, M>(acc, lane, n0, N, y);
}

// High bits of the four elements of low-nibble word i (byte t <- bits 2i,
// 2i+1 of byte t of h), placed at bits 4..5 of each byte.
__device__ __forceinline__ uint32_t q6_high(uint32_t h, int i) {
  const uint32_t v = i == 0 ? h << 4 : i == 1 ? h << 2 : i == 2 ? h : h >> 2;
  return v & 0x30303030u;
}

// Four 6-bit codes q -> four int8 values q - 32: setting bit 7 first keeps
// the byte-wise subtraction from borrowing across bytes.
__device__ __forceinline__ uint32_t q6_centre(uint32_t q) {
  return ((q | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
}

template <int M, int R, int U>
__global__ __launch_bounds__(256) void mmvq_q6_k_kernel(
    const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc, const uint16_t *w_d, int N,
    int K, const int8_t *a_qs, const uint16_t *a_d, float *y) {
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6)) * R;
  if (n0 >= N) return;
  const int nb = K >> 5;

  const uint8_t *lrow[R];
  const uint8_t *hrow[R];
  const uint16_t *srow[R];
  const uint16_t *drow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(n0 + r, N - 1);
    lrow[r] = w_ql + (size_t)n * (size_t)(K >> 1);
    hrow[r] = w_qh + (size_t)n * (size_t)(K >> 2);
    srow[r] = reinterpret_cast<const uint16_t *>(w_sc + (size_t)n * (size_t)(K >> 4));
    drow[r] = w_d + (size_t)n * (size_t)(K >> 8);
  }

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  for (int b0 = lane; b0 < nb; b0 += U * kWave) {
    uint4_t wl[U][R];
    uint2_t wh[U][R];
    uint16_t scw[U][R], dh[U][R];
    uint4_t aq0[U][M], aq1[U][M];
    uint16_t d8h[U][M];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = min(b0 + u * kWave, nb - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wl[u][r] = load16_nt(lrow[r] + 16 * b);
        wh[u][r] = load8_nt(hrow[r] + 8 * b);
        scw[u][r] = load_u16_nt(srow[r] + b);
        dh[u][r] = load_u16_nt(drow[r] + (b >> 3));
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
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo[i] = q6_centre((wl[u][r][i] & 0x0F0F0F0Fu) | q6_high(wh[u][r].x, i));
          hi[i] = q6_centre(((wl[u][r][i] >> 4) & 0x0F0F0F0Fu) | q6_high(wh[u][r].y, i));
        }
        const int32_t sa = (int32_t)(int8_t)(scw[u][r] & 0xFFu);
        const int32_t sb = (int32_t)(int8_t)(scw[u][r] >> 8);
        const float d6 = f16_bits_to_f32(dh[u][r]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          int32_t ia = 0, ib = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ia = dot4_i8(lo[i], aq0[u][m][i], ia);
            ib = dot4_i8(hi[i], aq1[u][m][i], ib);
          }
          const int32_t itot = sa * ia + sb * ib;
          const float a = fmaf(d6 * f16_bits_to_f32(d8h[u][m]), (float)itot, acc[r][m]);
          acc[r][m] = live ? a : acc[r][m];
        }
      }
    }
  }
  kq_store<R, M>(acc, lane, n0, N, y);
}

// Q4_K with the Q8_1 activation rows staged in LDS once per workgroup
// (M >= 3, matrices up to N = 6144): codes int8 [M][K], then d8 and s8 as
// float [M][K/32] each.  The mapping, header sharing and per-block
// arithmetic are mmvq_q4_k_kernel's; as in the staged Q6_K kernel below,
// activations are loaded once per workgroup (issued first, first batch
// stored while the first weight round is in flight, one barrier) and the
// rounds of one block per lane alternate two register buffers.
template <int M, int R, int W, int A>
__global__ __launch_bounds__(64 * W) void mmvq_q4_k_lds_kernel(
    const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, const int8_t *a_qs,
    const uint16_t *a_d, const uint16_t *a_s, float *y) {
  extern __shared__ uint4_t smem4[];
  int8_t *lq = reinterpret_cast<int8_t *>(smem4);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // row addresses stay scalar
  const int nb = K >> 5;
  float *ld8 = reinterpret_cast<float *>(lq + M * K);
  float *ls8 = ld8 + M * nb;
  const int n0 = (blockIdx.x * W + wave) * R;
  // 16-byte pieces: codes (M K / 16), d8 (M nb / 8), s8 (M nb / 8)
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
  const uint8_t *hrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(nw + r, N - 1);
    wrow[r] = w_qs + (size_t)n * (size_t)(K >> 1);
    hrow[r] = w_hdr + (size_t)n * (size_t)(K >> 8) * 16;
  }
  const int j = lane & 7;                   // sub-block of the lane's blocks
  const int s_sh = 8 * (j & 3);
  const int h_sh = 8 * (j >> 1) + 4 * (j & 1);
  const int hq = (lane & 3) == 0 ? 0 : (lane & 3) == 1 ? 1 + (j >> 2) : 3;   // dword loaded
  struct Round {
    uint4_t wq[R];
    uint32_t hw[R];
  };
  auto load = [&](int b, Round &rd) {
    b = min(b, nb - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      rd.wq[r] = load16_nt(wrow[r] + 16 * b);
      rd.hw[r] = __builtin_nontemporal_load(
          reinterpret_cast<const uint32_t *>(hrow[r] + 16 * (b >> 3)) + hq);
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
        float *dst = p < ncode + nd ? ld8 + 8 * (p - ncode) : ls8 + 8 * (p - ncode - nd);
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
  auto compute = [&](int b, const Round &rd) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t h0 = quad_lane<0>(rd.hw[r]);
      const uint32_t pb = quad_lane<1>(rd.hw[r]) >> s_sh;
      const uint32_t h3 = quad_lane<2>(rd.hw[r]);
      const uint32_t sc = pb & 63u;
      const uint32_t mn = ((pb >> 6) & 3u) | (((h3 >> h_sh) & 15u) << 2);
      const float dsc = f16_bits_to_f32((uint16_t)(h0 & 0xFFFFu)) * (float)sc;
      const float dmm = f16_bits_to_f32((uint16_t)(h0 >> 16)) * (float)mn;
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = rd.wq[r][i] & 0x0F0F0F0Fu;
        hi[i] = (rd.wq[r][i] >> 4) & 0x0F0F0F0Fu;
      }
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
        const float t = fmaf(dsc * ld8[m * nb + b], (float)isum, -(dmm * ls8[m * nb + b]));
        acc[r][m] = acc[r][m] + t;
      }
    }
  };
  // blocks b = lane, lane + 64, ...: the two round buffers alternate (nb is a
  // multiple of 8, so a quad enters and leaves the loop together)
  for (int b = lane; b < nb; b += 2 * kWave) {
    if (b + kWave < nb) load(b + kWave, r1);
    issue_fence();
    compute(b, r0);
    if (b + kWave >= nb) break;
    if (b + 2 * kWave < nb) load(b + 2 * kWave, r0);
    issue_fence();
    compute(b + kWave, r1);
  }
  kq_store<R, M>(acc, lane, n0, N, y);
}

// Q6_K with the Q8_1 activation rows staged in LDS once per workgroup
// (3 <= M <= 8): codes int8 [M][K] then d8 float [M][K/32].  The plain
// kernel re-reads each lane's activation blocks from L2 for every R rows,
// M x 34 bytes per 26 weight bytes per row; here a workgroup of W waves
// loads them once.  Activation loads are issued first, then the wave's
// first round of weights; the first staging batch is stored while the
// weights are in flight, one barrier, then rounds of U blocks per lane with
// the next round's weights in flight.  Per block the arithmetic is the plain
// kernel's, in the same order.
template <int M, int R, int U, int W, int A>
__global__ __launch_bounds__(64 * W) void mmvq_q6_k_lds_kernel(
    const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc, const uint16_t *w_d, int N,
    int K, const int8_t *a_qs, const uint16_t *a_d, float *y) {
  extern __shared__ uint4_t smem4[];
  int8_t *lq = reinterpret_cast<int8_t *>(smem4);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // row addresses stay scalar
  const int nb = K >> 5;
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
  const uint8_t *lrow[R];
  const uint8_t *hrow[R];
  const uint16_t *srow[R];
  const uint16_t *drow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(nw + r, N - 1);
    lrow[r] = w_ql + (size_t)n * (size_t)(K >> 1);
    hrow[r] = w_qh + (size_t)n * (size_t)(K >> 2);
    srow[r] = reinterpret_cast<const uint16_t *>(w_sc + (size_t)n * (size_t)(K >> 4));
    drow[r] = w_d + (size_t)n * (size_t)(K >> 8);
  }
  struct Round {
    uint4_t wl[U][R];
    uint2_t wh[U][R];
    uint16_t scw[U][R], dh[U][R];
  };
  auto load = [&](int b0, Round &rd) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = min(b0 + u * kWave, nb - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        rd.wl[u][r] = load16_nt(lrow[r] + 16 * b);
        rd.wh[u][r] = load8_nt(hrow[r] + 8 * b);
        rd.scw[u][r] = load_u16_nt(srow[r] + b);
        rd.dh[u][r] = load_u16_nt(drow[r] + (b >> 3));
      }
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
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = min(b0 + u * kWave, nb - 1);
      const bool live = b0 + u * kWave < nb;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo[i] = q6_centre((rd.wl[u][r][i] & 0x0F0F0F0Fu) | q6_high(rd.wh[u][r].x, i));
          hi[i] = q6_centre(((rd.wl[u][r][i] >> 4) & 0x0F0F0F0Fu) | q6_high(rd.wh[u][r].y, i));
        }
        const int32_t sa = (int32_t)(int8_t)(rd.scw[u][r] & 0xFFu);
        const int32_t sb = (int32_t)(int8_t)(rd.scw[u][r] >> 8);
        const float d6 = f16_bits_to_f32(rd.dh[u][r]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const uint4_t aq0 = *reinterpret_cast<const uint4_t *>(lq + (size_t)m * K + 32 * b);
          const uint4_t aq1 = *reinterpret_cast<const uint4_t *>(lq + (size_t)m * K + 32 * b + 16);
          int32_t ia = 0, ib = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ia = dot4_i8(lo[i], aq0[i], ia);
            ib = dot4_i8(hi[i], aq1[i], ib);
          }
          const int32_t itot = sa * ia + sb * ib;
          const float a = fmaf(d6 * ld8[m * nb + b], (float)itot, acc[r][m]);
          acc[r][m] = live ? a : acc[r][m];
        }
      }
    }
  };
  // rounds b0 = lane, lane + 64 U, ...: the two round buffers alternate
  for (int b0 = lane; b0 < nb; b0 += 2 * U * kWave) {
    if (b0 + U * kWave < nb) load(b0 + U * kWave, r1);
    issue_fence();
    compute(b0, r0);
    if (b0 + U * kWave >= nb) break;
    if (b0 + 2 * U * kWave < nb) load(b0 + 2 * U * kWave, r0);
    issue_fence();
    compute(b0 + U * kWave, r1);
  }
  kq_store<R, M>(acc, lane, n0, N, y);
}

template <int M, int R, int U>
static hipError_t launch_q4k_mru(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                 const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                 float *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  hipLaunchKernelGGL((mmvq_q4_k_kernel<M, R, U>), dim3((waves + 3) / 4), dim3(256), 0, stream,
                     w_qs, w_hdr, N, K, a_qs, a_d, a_s, y);
  return hipGetLastError();
}

template <int M, int R, int U>
static hipError_t launch_q6k_mru(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                                 const uint16_t *w_d, int N, int K, const int8_t *a_qs,
                                 const uint16_t *a_d, float *y, hipStream_t stream) {
  const int waves = (N + R - 1) / R;
  hipLaunchKernelGGL((mmvq_q6_k_kernel<M, R, U>), dim3((waves + 3) / 4), dim3(256), 0, stream,
                     w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y);
  return hipGetLastError();
}

// Launch shapes measured on MI355X over the Qwen3-8B projections (K 4096 and
// 12288, N 4096 to 24576) at M = 1, 2, 4, 8.  At M <= 2 a lane takes its
// whole share of a row in one round of exactly that many blocks up to 8
// (K <= 16384; longer rows take rounds of 6), two rows per wave, four on
// wide matrices (rounds padded to 4 or 8 blocks had cost, measured against
// exact rounds on MI355X: Q4_K 5120 x 13824 at M = 1 10.2 -> 8.8 us, Q6_K at
// M = 2 17.1 -> 12.8 us, 5120 x 5120 8.6 -> 6.8 us).  Wider M takes one or two blocks per
// round (the activation registers grow with M) and four rows per wave on
// wide matrices (Q4_K at M = 4 on 12288 x 4096: 11.6 -> 10.1 us with two).
template <int M>
static hipError_t launch_q4k_m(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                               const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                               float *y, hipStream_t stream) {
  const int per_lane = ((K >> 5) + kWave - 1) / kWave;
#define SKINNY_Q4K(R, U) return launch_q4k_mru<M, R, U>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream)
  if constexpr (M <= 2) {
    // one round of exactly the lane's share of the row up to 8 blocks (a
    // padding slot costs a block's loads and dots for nothing)
    switch (per_lane) {
      case 1:
      case 2:
        if (N >= 16384) SKINNY_Q4K(4, 2);
        SKINNY_Q4K(2, 2);
      case 3: SKINNY_Q4K(2, 3);
      case 4: SKINNY_Q4K(2, 4);
      case 5: SKINNY_Q4K(2, 5);
      case 6: SKINNY_Q4K(2, 6);
      case 7: SKINNY_Q4K(2, 7);
      case 8: SKINNY_Q4K(2, 8);
      default: SKINNY_Q4K(2, 6);
    }
  } else {
    if (N >= 16384) SKINNY_Q4K(4, 1);
    SKINNY_Q4K(2, 1);
  }
#undef SKINNY_Q4K
}

template <int M>
static hipError_t launch_q6k_m(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                               const uint16_t *w_d, int N, int K, const int8_t *a_qs,
                               const uint16_t *a_d, float *y, hipStream_t stream) {
  const int per_lane = ((K >> 5) + kWave - 1) / kWave;
#define SKINNY_Q6K(R, U) \
  return launch_q6k_mru<M, R, U>(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y, stream)
  if constexpr (M <= 2) {
    switch (per_lane) {           // as Q4_K: one round of exactly the lane's share
      case 1:
      case 2:
        if (M == 2 && N >= 16384) SKINNY_Q6K(4, 2);
        SKINNY_Q6K(2, 2);
      case 3: SKINNY_Q6K(2, 3);
      case 4: SKINNY_Q6K(2, 4);
      case 5: SKINNY_Q6K(2, 5);
      case 6: SKINNY_Q6K(2, 6);
      case 7: SKINNY_Q6K(2, 7);
      case 8: SKINNY_Q6K(2, 8);
      default: SKINNY_Q6K(2, 6);
    }
  } else {
    if (N >= 16384) SKINNY_Q6K(4, 1);
    SKINNY_Q6K(2, 2);
  }
#undef SKINNY_Q6K
}

// Routing.  From M = 3 matrices of at most 6144 rows take the staged kernel
// (when the activation rows fit in LDS), and matrices of fewer than 1100
// tiles of 16 rows the Q4_0 matrix-core kernel (its header array has the
// geometry of the Q4_0 block scales).  Wider ones take the matrix cores from
// M = 5 (4096 x 24576 at M = 8 2.5 -> 3.5 TB/s there), and below that the
// plain vector kernel.
// Staged Q4_K (3 <= M <= 8, N <= 6144): three rows per wave on mid-width
// matrices, two otherwise, eight waves per workgroup (measured on MI355X over
// the Qwen3-8B projections at M = 3..8: 4096 x 4096 at M = 5 5.9 -> 4.9 us,
// 12288 x 4096 at M = 4 10.3 -> 8.9 us, 4096 x 6144 at M = 8 8.1 -> 7.3 us).
// From N = 7168 the matrix cores are faster at every M from 3 (measured over
// every configuration on nine shapes: 8192 x 8192 at M = 8 21.9 -> 14.1 us,
// 7168 x 7168 at M = 4 13.8 -> 10.7 us, 5120 x 13824 at M = 6 19.2 -> 14.0
// us; at M = 3 2560 x 10240 and 5120 x 13824 lose 2-4%).
constexpr int kQ4kLdsMaxN = 6144;
constexpr int kQ4kMfmaNarrowTiles = 1100;

static int q4k_lds_bytes(int M, int K) { return M * K + 8 * M * (K >> 5); }

template <int M, int R, int A>
static hipError_t launch_q4k_lds_a(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                   const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                   float *y, hipStream_t stream) {
  constexpr int W = 8;
  const int lds = q4k_lds_bytes(M, K);
  const hipError_t lds_ok = allow_lds((const void *)mmvq_q4_k_lds_kernel<M, R, W, A>, lds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int rows = R * W;
  hipLaunchKernelGGL((mmvq_q4_k_lds_kernel<M, R, W, A>), dim3((N + rows - 1) / rows),
                     dim3(64 * W), lds, stream, w_qs, w_hdr, N, K, a_qs, a_d, a_s, y);
  return hipGetLastError();
}

template <int M, int R>
static hipError_t launch_q4k_lds_r(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                   const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                   float *y, hipStream_t stream) {
  const int pieces = M * K / 16 + 2 * (M * (K >> 5) / 8);
  const int per_thread = (pieces + 511) / 512;   // first staging batch
#define SKINNY_Q4L(A) \
  return launch_q4k_lds_a<M, R, A>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream)
  if (per_thread <= 4) SKINNY_Q4L(4);
  if (per_thread <= 8) SKINNY_Q4L(8);
  SKINNY_Q4L(16);
#undef SKINNY_Q4L
}

template <int M>
static hipError_t launch_q4k_lds(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                                 const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
                                 float *y, hipStream_t stream) {
  if (N > 4096) return launch_q4k_lds_r<M, 3>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream);
  return launch_q4k_lds_r<M, 2>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream);
}

hipError_t launch_mmvq_q4_k(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                            const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s, int M,
                            float *y, hipStream_t stream) {
  // Rows past K = 12288 at M <= 2 on matrices of 4096 rows or more: the
  // staged kernel (measured on MI355X: 13824 x 5120 at M = 2 16.2 -> 10.3
  // us, 17408 x 5120 at M = 1 13.2 -> 11.0 us; 12288 x 4096 and N = 2048 lose)
  if (M <= 2 && K > 12288 && N >= 4096 && q4k_lds_bytes(M, K) <= 160 * 1024)
    return M == 1 ? launch_q4k_lds<1>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream)
                  : launch_q4k_lds<2>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream);
  if (M >= 3 && N <= kQ4kLdsMaxN && q4k_lds_bytes(M, K) <= 160 * 1024) {
    switch (M) {
#define SKINNY_Q4L(MM) \
  case MM: return launch_q4k_lds<MM>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream);
      SKINNY_Q4L(3) SKINNY_Q4L(4) SKINNY_Q4L(5) SKINNY_Q4L(6) SKINNY_Q4L(7)
#undef SKINNY_Q4L
      default: return launch_q4k_lds<8>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream);
    }
  }
  const int tiles = (N + 15) / 16;
  if (M >= 5 || (M >= 3 && tiles < kQ4kMfmaNarrowTiles))
    return launch_mmvq_q4_k_mfma(w_qs, w_hdr, N, K, a_qs, a_d, a_s, M, y, stream);
  switch (M) {
#define SKINNY_Q4K(MM) \
  case MM: return launch_q4k_m<MM>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream);
    SKINNY_Q4K(1) SKINNY_Q4K(2) SKINNY_Q4K(3) SKINNY_Q4K(4)
    SKINNY_Q4K(5) SKINNY_Q4K(6) SKINNY_Q4K(7)
#undef SKINNY_Q4K
    default: return launch_q4k_m<8>(w_qs, w_hdr, N, K, a_qs, a_d, a_s, y, stream);
  }
}

// Staged Q6_K (3 <= M <= 8): one block per lane per round; four rows per
// wave and four waves on wide matrices, eight waves of one to four rows on
// mid-width ones (below), two rows and eight waves otherwise (measured on MI355X over the Qwen3-8B
// projections at M = 4 and 8: at M = 8 4096 x 6144 9.9 -> 8.6 us, 4096 x 4096
// 7.1 -> 6.4 us, 12288 x 4096 16.9 -> 14.3 us, 4096 x 24576 27.4 -> 27.1 us
// against the plain kernel).
constexpr int kQ6LdsMaxBytes = 160 * 1024;

static int q6k_lds_bytes(int M, int K) { return M * K + 4 * M * (K >> 5); }

template <int M, int R, int W, int A>
static hipError_t launch_q6k_lds_a(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                                   const uint16_t *w_d, int N, int K, const int8_t *a_qs,
                                   const uint16_t *a_d, float *y, hipStream_t stream) {
  const int lds = q6k_lds_bytes(M, K);
  const hipError_t lds_ok = allow_lds((const void *)mmvq_q6_k_lds_kernel<M, R, 1, W, A>, lds);
  if (lds_ok != hipSuccess) return lds_ok;
  const int rows = R * W;
  hipLaunchKernelGGL((mmvq_q6_k_lds_kernel<M, R, 1, W, A>), dim3((N + rows - 1) / rows),
                     dim3(64 * W), lds, stream, w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y);
  return hipGetLastError();
}

template <int M, int R, int W>
static hipError_t launch_q6k_lds_rw(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                                    const uint16_t *w_d, int N, int K, const int8_t *a_qs,
                                    const uint16_t *a_d, float *y, hipStream_t stream) {
  const int pieces = M * K / 16 + M * (K >> 5) / 8;
  const int per_thread = (pieces + 64 * W - 1) / (64 * W);   // first staging batch
#define SKINNY_Q6L(A) \
  return launch_q6k_lds_a<M, R, W, A>(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y, stream)
  if (per_thread <= 4) SKINNY_Q6L(4);
  if (per_thread <= 8) SKINNY_Q6L(8);
  SKINNY_Q6L(16);
#undef SKINNY_Q6L
}

template <int M>
static hipError_t launch_q6k_lds(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                                 const uint16_t *w_d, int N, int K, const int8_t *a_qs,
                                 const uint16_t *a_d, float *y, hipStream_t stream) {
#define SKINNY_Q6RW(R, W) \
  return launch_q6k_lds_rw<M, R, W>(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y, stream)
  if (N >= 16384) SKINNY_Q6RW(4, 4);
  if (N > 4096) {
    // mid-width matrices: rows of K >= 7168 four rows per wave from M = 6,
    // two below; shorter rows one row per wave (measured on MI355X over
    // every R in 1..4 and W in 2, 4, 8 at M = 3, 4, 6, 8 on six shapes:
    // 8192 x 8192 at M = 8 24.8 -> 16.8 us, 7168 x 7168 at M = 4
    // 16.7 -> 12.0 us, 5120 x 13824 at M = 8 27.8 -> 22.0 us)
    if (K >= 7168) {
      if (M >= 6) SKINNY_Q6RW(4, 8);
      SKINNY_Q6RW(2, 8);
    }
    SKINNY_Q6RW(1, 8);
  }
  SKINNY_Q6RW(2, 8);
#undef SKINNY_Q6RW
}

hipError_t launch_mmvq_q6_k(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                            const uint16_t *w_d, int N, int K, const int8_t *a_qs,
                            const uint16_t *a_d, int M, float *y, hipStream_t stream) {
  // Long rows at M <= 2 on matrices of 4096 rows or more: the staged kernel
  // (measured on MI355X: at M = 2 past K = 12288, 14336 x 4096 14.7 -> 10.8
  // us, 13824 x 5120 20.5 -> 16.1 us; at M = 1 past K = 16384, 28672 x 4096
  // 20.9 -> 18.6 us; shorter rows, and N = 2048, stay on the vector kernel)
  if (M <= 2 && (M == 2 ? K > 12288 : K > 16384) && N >= 4096 &&
      q6k_lds_bytes(M, K) <= kQ6LdsMaxBytes)
    return M == 1 ? launch_q6k_lds<1>(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y, stream)
                  : launch_q6k_lds<2>(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y, stream);
  if (M >= 3 && q6k_lds_bytes(M, K) <= kQ6LdsMaxBytes) {
    switch (M) {
#define SKINNY_Q6L(MM) \
  case MM: return launch_q6k_lds<MM>(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y, stream);
      SKINNY_Q6L(3) SKINNY_Q6L(4) SKINNY_Q6L(5) SKINNY_Q6L(6) SKINNY_Q6L(7)
#undef SKINNY_Q6L
      default: return launch_q6k_lds<8>(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y, stream);
    }
  }
  switch (M) {
#define SKINNY_Q6K(MM) \
  case MM: return launch_q6k_m<MM>(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y, stream);
    SKINNY_Q6K(1) SKINNY_Q6K(2) SKINNY_Q6K(3) SKINNY_Q6K(4)
    SKINNY_Q6K(5) SKINNY_Q6K(6) SKINNY_Q6K(7)
#undef SKINNY_Q6K
    default: return launch_q6k_m<8>(w_ql, w_qh, w_sc, w_d, N, K, a_qs, a_d, y, stream);
  }
}

}  // namespace skinny
