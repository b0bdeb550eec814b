/*
 * skinny_gemm.h -- C ABI of libskinny_gemm.so: block-quantized matrix x
 * vector and skinny GEMM (M = 1..8 activation rows for the Q8_1 formats,
 * 1..16 for NVFP4, 1..96 for FP8) for LLM decode and speculative
 * verification on AMD Instinct MI355X (gfx950).
 *
 * Sources.  "Machine Learning on NVIDIA CMP" (sections "TL;DR", "llama.cpp
 * results", "The DP2A patch") describes decode as a quantized mat x vec
 * (MMVQ) over Q4_0 weights whose inner loop is a 4-way int8 dot with int32
 * accumulation, and requires any rewrite of that dot to stay bit-exact
 * integer arithmetic.  "v100-skinny README" (sections "Result", "How QPN
 * works", "Native mixed-precision checkpoint path") describes W4A16 NVFP4
 * and W8A16 FP8 skinny GEMMs at verification width M <= 8: packed weights
 * stay compressed in memory and are decoded only where consumed, the NVFP4
 * global scale is folded into the group-16 scales, and every 16-element
 * group is flushed into an FP32 accumulator so that binary16 cannot
 * overflow.  The pages leave the activation format, nibble order and FP8
 * scale granularity open; the readings taken are stated per function.
 *
 * Conventions shared by every entry point.
 *   - Every pointer is a device pointer on the current HIP device; `stream`
 *     is a hipStream_t passed as void* (NULL = the default stream).
 *   - The caller allocates and owns every buffer.  The library allocates
 *     no device memory and keeps no data between calls (only, per device,
 *     which kernels it has already allowed more than 64 KB of LDS), and is
 *     safe to call from several host threads.  Outputs must not overlap
 *     inputs.
 *   - A call validates its arguments on the host before any HIP call, then
 *     enqueues its kernel (several, for the split cases stated below) on
 *     `stream` and returns without synchronizing.
 *     Faults during execution surface at the caller's next synchronization.
 *   - binary16 values are passed as their 16-bit patterns (uint16_t).
 *   - A call with M == 0 or N == 0 has nothing to compute: it returns
 *     SKINNY_OK without touching memory (pointers may then be NULL).
 *   - There is exactly one code path per entry point; nothing falls back.
 *
 * Status codes (return values):
 */
#ifndef SKINNY_GEMM_H
#define SKINNY_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKINNY_OK               0
#define SKINNY_ERR_NULL        -1  /* a required pointer is NULL                    */
#define SKINNY_ERR_SHAPE       -2  /* K or N out of range, or K not a multiple of   */
                                   /* the format's block (see each function)        */
#define SKINNY_ERR_ALIGN       -3  /* a pointer is not aligned as required          */
#define SKINNY_ERR_M           -4  /* M outside the entry point's range             */
#define SKINNY_ERR_LAUNCH      -5  /* the HIP launch reported an error              */

/* Limits: 1 <= K <= SKINNY_MAX_K, 0 <= N <= SKINNY_MAX_N.  No kernel gives an
 * output row more than 32 threads, so N <= 2^24 keeps every grid near 2^29
 * work-items, well inside the 2^32 that one dispatch can hold. */
#define SKINNY_MAX_K  (1 << 20)
#define SKINNY_MAX_N  (1 << 24)
#define SKINNY_MAX_M_GEMV   8    /* mmvq_q4_0, mmvq_q4_k, mmvq_q6_k, mmvq_iq4_xs */
/* gemv_nvfp4_w4a16: two 8-row verification tiles. */
#define SKINNY_MAX_M_F16ACT 16
/* gemv_fp8_w8a16: also the "chunked" band up to 96 rows. */
#define SKINNY_MAX_M_FP8    96
#define SKINNY_MAX_M_QUANT  65536
/* quantize_act_q8_1: one thread per 8 elements, so M * K <= 2^32 keeps its grid
 * at 2^29 threads. */
#define SKINNY_MAX_MK_QUANT (1LL << 32)
/* mmvq_q4_0_f32act: decode widths only, one row of K in LDS per workgroup. */
#define SKINNY_MAX_M_F32ACT 2
#define SKINNY_MAX_K_F32ACT 12288

/* Static, human-readable text for a status code. */
const char *skinny_status_string(int status);

/*
 * quantize_act_q8_1 -- quantize activation rows to Q8_1.
 *
 * The activation side of the quantized mat x vec kernel ("Machine Learning
 * on NVIDIA CMP", "TL;DR" and "The DP2A patch": the dot consumes int8 codes).
 * For each row m and each block b of 32 consecutive elements:
 *   amax = max |x|;  if amax == 0 all outputs of the block are 0;
 *   d32  = amax / 127                         (binary32, correctly rounded)
 *   q_i  = round_half_away_from_zero(x_i / d32), clamped to [-127, 127]
 *   d    = binary16(d32),  s = binary16(d32 * sum_i q_i)   (round to nearest even)
 *
 *   x   float32 [M][K] row-major, 16-byte aligned.
 *   qs  int8    [M][K] row-major, 16-byte aligned.
 *   d   binary16 [M][K/32], 2-byte aligned.
 *   s   binary16 [M][K/32], 2-byte aligned.
 *   0 <= M <= SKINNY_MAX_M_QUANT; K % 32 == 0; M * K <= SKINNY_MAX_MK_QUANT
 *   (else SKINNY_ERR_SHAPE).
 * Results are bit-exact (one correct answer per input).  NaN or infinite
 * inputs give unspecified codes.
 */
int quantize_act_q8_1(const float *x, int M, int K,
                      int8_t *qs, uint16_t *d, uint16_t *s, void *stream);

/*
 * mmvq_q4_0 -- y = A * W^T for Q4_0 weights and Q8_1 activations.
 *
 * "Machine Learning on NVIDIA CMP", "llama.cpp results" and "The DP2A
 * patch": MMVQ with a 4-way int8 dot per 32-element block.
 * Weights, planar Q4_0: w_qs [N][K/2] bytes (byte j of block b holds code
 * 32b+j in its low nibble and code 32b+16+j in its high nibble), w_d
 * binary16 [N][K/32]; weight = (code - 8) * d.  Activations from
 * quantize_act_q8_1.  For each m, n:
 *   y[m][n] = sum_b d4[n][b] * (d8[m][b] * isum - 8 * s8[m][b]),
 *   isum    = sum_{i<32} code[n][32b+i] * q8[m][32b+i]   (exact int32),
 * i.e. the -8 of every weight is applied once per block through the Q8_1
 * sum term.  Accumulated in float32, output float32.
 *
 *   w_qs, w_d, a_qs, a_d, a_s 16-byte aligned (the scale arrays too are
 *   read with 128-bit loads); y float32 [M][N] row-major, 4-byte aligned.
 *   0 <= M <= SKINNY_MAX_M_GEMV; K % 32 == 0.
 * Block sums are exact integers; the float result matches the definition
 * to float32 summation-order rounding.
 */
int mmvq_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
              const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
              int M, float *y, void *stream);

/*
 * mmvq_q4_0_f32act -- quantize_act_q8_1 and mmvq_q4_0 in one launch, for
 * decode (M = 1 or 2).
 *
 * The same computation as quantize_act_q8_1(x) followed by mmvq_q4_0 on its
 * output ("Machine Learning on NVIDIA CMP", "TL;DR" and "The DP2A patch":
 * the activations are quantized to int8 blocks on the device before the
 * int8 dot), with the same block arithmetic, so y is bit-identical to the
 * two calls; the Q8_1 activations are kept in on-chip memory and never
 * written out, which saves the second launch and its round trip.
 *   w_qs, w_d  planar Q4_0 weights as for mmvq_q4_0.
 *   x          float32 [M][K] row-major, 16-byte aligned.
 *   y          float32 [M][N] row-major, 4-byte aligned.
 *   0 <= M <= SKINNY_MAX_M_F32ACT (else SKINNY_ERR_M; wider M: call the two
 *   entry points); K % 32 == 0 and K <= SKINNY_MAX_K_F32ACT (else
 *   SKINNY_ERR_SHAPE).
 */
int mmvq_q4_0_f32act(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                     const float *x, int M, float *y, void *stream);

/*
 * mmvq_q4_k -- y = A * W^T for Q4_K weights and Q8_1 activations.
 *
 * "Machine Learning on NVIDIA CMP", "llama.cpp results": Q4_K models decode
 * through the same MMVQ 4-way int8 dot as Q4_0.  The pages do not define the
 * format; this is the published GGUF K-quant arithmetic in a planar layout
 * of our own (4.5 bits per weight, as the original):
 *   w_qs  [N][K/2] bytes, 4-bit codes q in Q4_0 nibble order per block of
 *         32 (byte j: element j low nibble, element j+16 high nibble).
 *   w_hdr [N][K/256][16] bytes per super-block of 256: bytes 0-1 d and 2-3
 *         dmin (binary16), bytes 4..15 = p[0..11] with, for sub-block
 *         j = 0..7 of 32, sc_j = p[j] & 63 and
 *         m_j = (p[j] >> 6) | (((p[8 + j/2] >> (4 (j%2))) & 15) << 2).
 *   weight = d * sc_j * q - dmin * m_j.
 * For each m, n:  y = sum_b d sc d8 isum_b - dmin m s8_b,
 * isum_b = sum_{i<32} q * q8 (exact int32); the min enters through the Q8_1
 * sum term s8.  Accumulated in float32.
 *   w_qs, w_hdr, a_qs, a_d, a_s 16-byte aligned; y float32 [M][N], 4-byte
 *   aligned.  0 <= M <= SKINNY_MAX_M_GEMV; K % 256 == 0.
 */
int mmvq_q4_k(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
              const int8_t *a_qs, const uint16_t *a_d, const uint16_t *a_s,
              int M, float *y, void *stream);

/*
 * mmvq_q6_k -- y = A * W^T for Q6_K weights and Q8_1 activations.
 *
 * As mmvq_q4_k ("llama.cpp results": Q6_K models on the same int8 dot); the
 * published GGUF Q6_K arithmetic in a planar layout of our own (6.5625 bits
 * per weight, as the original):
 *   w_ql [N][K/2]  low 4 bits of the 6-bit codes, Q4_0 nibble order per
 *        block of 32.
 *   w_qh [N][K/4]  high 2 bits, 8 bytes per block of 32: byte 4h + t
 *        (h = 0, 1; t = 0..3), bits 2c..2c+1 = element 16h + 4c + t.
 *   w_sc [N][K/16] int8 scale of each sub-block of 16.
 *   w_d  [N][K/256] binary16.
 *   weight = d * sc_j * (q - 32), q = low | high << 4 in 0..63.
 * For each m, n:  y = sum_b d d8_b (sc_2b isum_lo + sc_2b+1 isum_hi), the
 * isums over the two 16-element halves of block b with codes q - 32 (exact
 * integers; the Q8_1 sum term is not used).  Accumulated in float32.
 *   w_ql, a_qs, a_d 16-byte aligned (a_d is read with 128-bit loads on
 *   some paths); w_qh 8-byte aligned; w_sc, w_d 2-byte aligned; y float32
 *   [M][N], 4-byte aligned.
 *   0 <= M <= SKINNY_MAX_M_GEMV; K % 256 == 0.
 */
int mmvq_q6_k(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
              const uint16_t *w_d, int N, int K, const int8_t *a_qs,
              const uint16_t *a_d, int M, float *y, void *stream);

/*
 * mmvq_iq4_xs -- y = A * W^T for IQ4_XS weights and Q8_1 activations.
 *
 * "Machine Learning on NVIDIA CMP", "llama.cpp results": an IQ4_XS model
 * decodes through the same MMVQ 4-way int8 dot as Q4_0.  The pages do not
 * define the format; this is the published GGUF IQ4_XS arithmetic in a
 * planar layout of our own (4.25 bits per weight, as the original):
 *   w_qs  [N][K/2] bytes, 4-bit indices q in Q4_0 nibble order per block of
 *         32 (byte j: element j low nibble, element j+16 high nibble).
 *   w_hdr [N][K/256][8] bytes per super-block of 256: bytes 0-1 d
 *         (binary16), bytes 2-3 a little-endian word H, bytes 4-7 a
 *         little-endian word L; sub-block j = 0..7 of 32 has the 6-bit scale
 *         ls_j = ((L >> 4j) & 15) | (((H >> 2j) & 3) << 4).
 *   weight = d * (ls_j - 32) * T[q], T = {-127, -104, -83, -65, -49, -35,
 *         -22, -10, 1, 13, 25, 38, 53, 69, 89, 113} (the IQ4_NL table).
 * For each m, n:  y = sum_b d (ls - 32) d8_b isum_b, isum_b = sum_{i<32}
 * T[q] q8 (exact int32; T is signed, so the Q8_1 sum term is not used).
 * Accumulated in float32.
 *   w_qs, w_hdr, a_qs, a_d 16-byte aligned (the headers are read with
 *   128-bit loads on some paths); y float32 [M][N], 4-byte aligned.
 *   0 <= M <= SKINNY_MAX_M_GEMV; K % 256 == 0.
 */
int mmvq_iq4_xs(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                const int8_t *a_qs, const uint16_t *a_d, int M, float *y,
                void *stream);

/*
 * gemv_nvfp4_w4a16 -- y = x * W^T for NVFP4 weights and binary16 activations.
 *
 * "v100-skinny README", "How QPN works": E2M1 codes with an E4M3 scale per
 * 16 elements and a per-tensor scale folded into the group scales; FP32
 * accumulation per 16-element group.
 *   w_codes  [N][K/2] bytes: element 2j of a row in the low nibble of byte
 *            j, element 2j+1 in the high nibble.  16-byte aligned.
 *   w_scales [N][K/16] OCP E4M3 ("FN") bytes, one per 16 elements.
 *            16-byte aligned.
 *   global_scale  per-tensor float32 multiplier.
 *   x        binary16 [M][K] row-major, 16-byte aligned.
 *   y        binary16 [M][N] row-major, 2-byte aligned:
 *            y = binary16( sum_j (sum_{i<16} e2m1 * x) * (e4m3(scale_j) * g) ),
 *            accumulated in float32, rounded to nearest even once.
 *   0 <= M <= SKINNY_MAX_M_F16ACT; K % 32 == 0.  Rows 9..16 serve the wide
 *   verification band of the same pages ("Native mixed-precision checkpoint
 *   path", dispatch table): one weight pass for all M rows whenever
 *   K % 256 == 0; otherwise rows 1..8 and 9..M take one pass each.
 */
int gemv_nvfp4_w4a16(const uint8_t *w_codes, const uint8_t *w_scales,
                     float global_scale, int N, int K,
                     const uint16_t *x, int M, uint16_t *y, void *stream);

/*
 * Q4_0 weights pre-permuted into matrix-core operand order.
 *
 * "v100-skinny README", "How QPN works": the weights are rearranged once, at
 * load time, into the order in which the matrix instructions consume them,
 * so the main loop does no shuffling.  The calls below give the same product
 * as mmvq_q4_0 from such a copy of the weights (same Q8_1 activations, same
 * exact int32 block sums).
 *
 * Packed layout (K % 256 == 0; U = ceil(N/16) tiles of 16 rows, P = K/128,
 * V = ceil(K/512); nb = K/32 blocks per row); lane l = 16 g + j with
 * g = 2 h + b (h, b < 2), j < 16:
 *   codes plane: U*P blocks of 1024 bytes, block (u, p) at byte 1024*(u*P + p);
 *     bytes 16l + 8e .. 16l + 8e + 7 (e < 2) of it =
 *     w_qs[16u + j][16*(4p + 2e + h) + 8b .. + 7];
 *   scale plane, after the codes plane: U*V blocks of 512 bytes, block (u, v)
 *     at byte 1024*U*P + 512*(u*V + v); the binary16 at bytes 256h + 16j + 2t
 *     (t < 8) = w_d[16u + j][16v + 2t + h];
 *   bytes for rows >= N or blocks >= nb are zero.
 */

/* prepack_q4_0_size -- bytes of the packed copy: 1024*U*P + 512*U*V.  Host
 * only.  0 <= N <= SKINNY_MAX_N; K % 256 == 0 (else SKINNY_ERR_SHAPE). */
int prepack_q4_0_size(int N, int K, size_t *bytes);

/*
 * prepack_q4_0 -- write the packed copy of planar Q4_0 weights.
 *   w_qs, w_d as for mmvq_q4_0 (w_qs 16-byte aligned, w_d 2-byte aligned);
 *   w_packed: prepack_q4_0_size bytes, 16-byte aligned, caller-owned, not
 *   overlapping the inputs.  Every byte of it is written.  K % 256 == 0.
 */
int prepack_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K, uint8_t *w_packed,
                 void *stream);

/*
 * mmvq_q4_0_packed -- mmvq_q4_0 on the packed copy.
 *   w_packed from prepack_q4_0 for the same N and K, 16-byte aligned;
 *   a_qs, a_d, a_s, y, M as for mmvq_q4_0 (0 <= M <= SKINNY_MAX_M_GEMV);
 *   K % 256 == 0.  Block sums are exact integers; the float result matches
 *   the definition to float32 summation-order rounding.
 */
int mmvq_q4_0_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                     const uint16_t *a_d, const uint16_t *a_s, int M, float *y, void *stream);

/*
 * Q4_K weights pre-permuted into matrix-core operand order: the codes plane
 * of the Q4_0 layout above (Q4_K codes have the Q4_0 nibble order), then a
 * header plane of U*(K/256) blocks of 256 bytes, block (u, q) at byte
 * 1024*U*P + 256*(u*(K/256) + q), whose bytes 16j .. 16j + 15 are
 * w_hdr[16u + j][16q .. 16q + 15] (the header of super-block q of that row);
 * bytes for rows >= N are zero.  The calls below give the same product as
 * mmvq_q4_k from such a copy.
 */

/* prepack_q4_k_size -- bytes of the packed copy: 1024*U*P + U*K.  Host only.
 * 0 <= N <= SKINNY_MAX_N; K % 256 == 0 (else SKINNY_ERR_SHAPE). */
int prepack_q4_k_size(int N, int K, size_t *bytes);

/*
 * prepack_q4_k -- write the packed copy of planar Q4_K weights.
 *   w_qs, w_hdr as for mmvq_q4_k (16-byte aligned); w_packed: prepack_q4_k_size
 *   bytes, 16-byte aligned, caller-owned, not overlapping the inputs.  Every
 *   byte of it is written.  K % 256 == 0.
 */
int prepack_q4_k(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, uint8_t *w_packed,
                 void *stream);

/*
 * mmvq_q4_k_packed -- mmvq_q4_k on the packed copy.
 *   w_packed from prepack_q4_k for the same N and K, 16-byte aligned;
 *   a_qs, a_d, a_s, y, M as for mmvq_q4_k (0 <= M <= SKINNY_MAX_M_GEMV).
 *   Block sums are exact integers; the float result matches the definition
 *   to float32 summation-order rounding.
 */
int mmvq_q4_k_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                     const uint16_t *a_d, const uint16_t *a_s, int M, float *y, void *stream);

/*
 * IQ4_XS weights pre-permuted into matrix-core operand order: the codes
 * plane of the Q4_0 layout above (IQ4_XS indices have the Q4_0 nibble
 * order), then a header plane of U*(K/256) blocks of 128 bytes, block (u, q)
 * at byte 1024*U*P + 128*(u*(K/256) + q), whose bytes 8j .. 8j + 7 are
 * w_hdr[16u + j][8q .. 8q + 7] (the header of super-block q of that row);
 * bytes for rows >= N are zero.  The calls below give the same product as
 * mmvq_iq4_xs from such a copy.
 */

/* prepack_iq4_xs_size -- bytes of the packed copy: 1024*U*P + U*K/2.  Host
 * only.  0 <= N <= SKINNY_MAX_N; K % 256 == 0 (else SKINNY_ERR_SHAPE). */
int prepack_iq4_xs_size(int N, int K, size_t *bytes);

/*
 * prepack_iq4_xs -- write the packed copy of planar IQ4_XS weights.
 *   w_qs, w_hdr as for mmvq_iq4_xs (16-byte aligned); w_packed:
 *   prepack_iq4_xs_size bytes, 16-byte aligned, caller-owned, not
 *   overlapping the inputs.  Every byte of it is written.  K % 256 == 0.
 */
int prepack_iq4_xs(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K, uint8_t *w_packed,
                   void *stream);

/*
 * mmvq_iq4_xs_packed -- mmvq_iq4_xs on the packed copy.
 *   w_packed from prepack_iq4_xs for the same N and K, 16-byte aligned;
 *   a_qs, a_d, y, M as for mmvq_iq4_xs (0 <= M <= SKINNY_MAX_M_GEMV).
 *   Block sums are exact integers; the float result matches the definition
 *   to float32 summation-order rounding.
 */
int mmvq_iq4_xs_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                       const uint16_t *a_d, int M, float *y, void *stream);

/*
 * Q6_K weights pre-permuted into matrix-core operand order.
 *
 * The matrix cores take one 16-element sub-block per K slot (lane
 * l = 16 g + j, g < 4: sub-block g of each 64-element step, row j of a
 * 16-row tile).  Packed layout (K % 256 == 0; U = ceil(N/16), P = K/128,
 * Q = K/256), four planes:
 *   L: U*P blocks of 1024 bytes, block (u, p) at byte 1024*(u*P + p); byte
 *      16l + 8e + c (e < 2, c < 8) = low(c) | low(8 + c) << 4, low(x) = the
 *      low 4 bits of element x of sub-block g of step 2p + e of row 16u + j;
 *   H: from 1024*U*P, U*Q blocks of 1024 bytes, block (u, q); bytes
 *      16l + 4t .. + 3 (t < 4) = w_qh[16u + j][8b + 4h .. + 3] with
 *      b = 2*(4q + t) + g/2, h = g % 2 (the high bits of that sub-block);
 *   C: from 1024*U*(P + Q), U*Q blocks of 256 bytes, block (u, q); byte
 *      4l + t = w_sc[16u + j][16q + 4t + g];
 *   D: from 1024*U*(P + Q) + 256*U*Q, U*Q blocks of 32 bytes, block (u, q);
 *      bytes 2j, 2j + 1 = w_d[16u + j][q];
 *   bytes for rows >= N are zero.
 */

/* prepack_q6_k_size -- bytes of the packed copy: 1024*U*P + 1312*U*Q.  Host
 * only.  0 <= N <= SKINNY_MAX_N; K % 256 == 0 (else SKINNY_ERR_SHAPE). */
int prepack_q6_k_size(int N, int K, size_t *bytes);

/*
 * prepack_q6_k -- write the packed copy of planar Q6_K weights.
 *   w_ql, w_qh, w_sc, w_d as for mmvq_q6_k (w_ql 16-byte, w_qh 8-byte, w_sc
 *   and w_d 2-byte aligned); w_packed: prepack_q6_k_size bytes, 16-byte
 *   aligned, caller-owned, not overlapping the inputs.  Every byte of it is
 *   written.  K % 256 == 0.
 */
int prepack_q6_k(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                 const uint16_t *w_d, int N, int K, uint8_t *w_packed, void *stream);

/*
 * mmvq_q6_k_packed -- mmvq_q6_k on the packed copy (matrix cores at every M).
 *   w_packed from prepack_q6_k for the same N and K, 16-byte aligned;
 *   a_qs, a_d (16-byte aligned), y, M as for mmvq_q6_k
 *   (0 <= M <= SKINNY_MAX_M_GEMV).  Sub-block sums are exact integers; the
 *   float result matches the definition to float32 summation-order rounding.
 */
int mmvq_q6_k_packed(const uint8_t *w_packed, int N, int K, const int8_t *a_qs,
                     const uint16_t *a_d, int M, float *y, void *stream);

/*
 * NVFP4 weights pre-permuted into matrix-core operand order.
 *
 * "v100-skinny README", "How QPN works": the weights are rearranged once, at
 * load time, into the order in which the matrix instructions consume them,
 * so the GEMV's main loop does no shuffling.  The three calls below give the
 * same product as gemv_nvfp4_w4a16 from such a copy of the weights.
 *
 * Packed layout (K % 256 == 0; U = ceil(N/16) tiles of 16 rows, S = K/128
 * steps of 128 elements, V = ceil(S/8)); lane l = 16 g + i, g < 4, i < 16:
 *   codes plane: U*S blocks of 1024 bytes, block (u, s) at byte 1024*(u*S + s);
 *     bytes 16l .. 16l+15 of it = w_codes[16u + i][64s + 16g .. 64s + 16g + 15]
 *     (elements 128s + 32g .. +31 of that row);
 *   scale plane, after the codes plane: U*V blocks of 1024 bytes, block (u, v)
 *     at byte 1024*(U*S + u*V + v); bytes 16l + 2t and 16l + 2t + 1 (t < 8) =
 *     w_scales[16u + i][8*(8v + t) + 2g] and [.. + 1];
 *   bytes for rows >= N or steps >= S are zero.
 */

/*
 * prepack_nvfp4_size -- bytes of the packed copy of an N x K NVFP4 matrix:
 * 1024 * U * (S + V).  Host only, no HIP call.
 *   0 <= N <= SKINNY_MAX_N; K % 256 == 0 (else SKINNY_ERR_SHAPE); bytes != NULL.
 */
int prepack_nvfp4_size(int N, int K, size_t *bytes);

/*
 * prepack_nvfp4 -- write the packed copy of canonical NVFP4 weights.
 *   w_codes, w_scales as for gemv_nvfp4_w4a16 (w_codes 16-byte aligned,
 *   w_scales 2-byte aligned); w_packed: prepack_nvfp4_size bytes, 16-byte
 *   aligned, caller-owned, not overlapping the inputs.  Every byte of it is
 *   written.  K % 256 == 0.
 */
int prepack_nvfp4(const uint8_t *w_codes, const uint8_t *w_scales, int N, int K,
                  uint8_t *w_packed, void *stream);

/*
 * gemv_nvfp4_w4a16_packed -- gemv_nvfp4_w4a16 on the packed copy.
 *   w_packed from prepack_nvfp4 for the same N and K, 16-byte aligned;
 *   global_scale, x, y, M as for gemv_nvfp4_w4a16 (0 <= M <= 16, one weight
 *   pass for all M rows); K % 256 == 0.  The result matches the definition
 *   to float32 summation-order rounding, as gemv_nvfp4_w4a16 does.
 */
int gemv_nvfp4_w4a16_packed(const uint8_t *w_packed, float global_scale, int N, int K,
                            const uint16_t *x, int M, uint16_t *y, void *stream);

/*
 * gemv_fp8_w8a16 -- y = x * W^T for FP8 E4M3 weights and binary16 activations.
 *
 * "v100-skinny README", "How QPN works": one contiguous E4M3 byte stream
 * per weight matrix.  The pages do not give the scale granularity; here it
 * is one float32 scale per output channel, applied after the dot.
 *   w   [N][K] OCP E4M3 ("FN") bytes, 16-byte aligned.
 *   channel_scale float32 [N], 4-byte aligned.
 *   x   binary16 [M][K] row-major, 16-byte aligned.
 *   y   binary16 [M][N] row-major, 2-byte aligned:
 *       y = binary16( channel_scale[n] * sum_k e4m3(w[n][k]) * x[m][k] ),
 *       accumulated in float32.
 *   0 <= M <= SKINNY_MAX_M_FP8; K % 16 == 0.  Rows 9..16 (the wide
 *   verification band, "How QPN works": two 8-row tiles against one weight
 *   pass) and 17..96 (the "chunked" FP8 band of the dispatch table in
 *   "Native mixed-precision checkpoint path") share one weight pass
 *   whenever K % 256 == 0; otherwise each group of up to 8 rows takes its
 *   own pass.  NaN weight codes (0x7F, 0xFF) give unspecified results.
 */
int gemv_fp8_w8a16(const uint8_t *w, const float *channel_scale, int N, int K,
                   const uint16_t *x, int M, uint16_t *y, void *stream);

/*
 * FP8 weights pre-permuted into matrix-core operand order.
 *
 * "v100-skinny README", "How QPN works": the weights are rearranged once, at
 * load time, into the order in which the matrix instructions consume them.
 * The calls below give the same product as gemv_fp8_w8a16 from such a copy.
 *
 * Packed layout (K % 256 == 0; U = ceil(N/16) tiles of 16 rows, S = K/128
 * steps); lane l = 16 g + i, g < 4, i < 16: U*S blocks of 2048 bytes, block
 * (u, s) at byte 2048*(u*S + s); bytes 1024e + 16l .. 1024e + 16l + 15
 * (e < 2) of it = w[16u + i][128s + 32g + 16e .. + 15]; bytes for rows >= N
 * are zero.  The channel scales are not part of the copy.
 */

/* prepack_fp8_size -- bytes of the packed copy: 16 * U * K.  Host only.
 * 0 <= N <= SKINNY_MAX_N; K % 256 == 0 (else SKINNY_ERR_SHAPE). */
int prepack_fp8_size(int N, int K, size_t *bytes);

/*
 * prepack_fp8 -- write the packed copy of an E4M3 weight matrix.
 *   w as for gemv_fp8_w8a16 (16-byte aligned); w_packed: prepack_fp8_size
 *   bytes, 16-byte aligned, caller-owned, not overlapping w.  Every byte of
 *   it is written.  K % 256 == 0.
 */
int prepack_fp8(const uint8_t *w, int N, int K, uint8_t *w_packed, void *stream);

/*
 * gemv_fp8_w8a16_packed -- gemv_fp8_w8a16 on the packed copy.
 *   w_packed from prepack_fp8 for the same N and K, 16-byte aligned;
 *   channel_scale, x, y, M as for gemv_fp8_w8a16 (0 <= M <= SKINNY_MAX_M_FP8);
 *   K % 256 == 0.  One weight pass for M <= 16; above, one pass on matrices
 *   of 1536 tiles or more, else one pass per group of 16 rows.  The result
 *   matches the definition to float32 summation-order rounding.
 */
int gemv_fp8_w8a16_packed(const uint8_t *w_packed, const float *channel_scale, int N, int K,
                          const uint16_t *x, int M, uint16_t *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_GEMM_H */
