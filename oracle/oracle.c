/*
 * oracle.c -- plain, slow CPU reference for the quantized skinny-GEMV path.
 *
 * TEST INFRASTRUCTURE.  This library exists only to check the GPU library.
 * Only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load or call it; the GPU library never does, and the
 * two share no source, header, table or helper.
 *
 * What it computes, and where that is defined:
 *   - "Machine Learning on NVIDIA CMP", sections "TL;DR" and "llama.cpp
 *     results": decode runs a quantized matrix x vector kernel (MMVQ) over
 *     Q4_0 weights; section "The DP2A patch": the block dot is a 4-way int8
 *     dot product with int32 accumulation, and rewriting it must stay
 *     bit-exact integer arithmetic.
 *   - "v100-skinny README", section "How QPN works": NVFP4 weights are E2M1
 *     codes with an FP8 (E4M3) scale per group of 16 and a global scale that
 *     is folded into the group scales, each 16-element group being flushed
 *     into an FP32 accumulator; FP8 weights are one E4M3 byte per weight.
 *     Weights stay packed and are decoded only where they are consumed.
 *   - The same page's model table runs Q4_K, Q6_K and IQ4_XS models through
 *     that MMVQ dot; their super-block arithmetic is the published GGUF
 *     definition (not on the pages), stated next to those functions.
 *   The pages do not spell out Q8_1, the nibble order, the FP8 scale
 *   granularity or the exact rounding rules; the readings taken here are the
 *   ones listed next to each function.
 *
 * Precision.  The three dot products are written as their plain definitions
 * in binary64, which holds every product and every 16- or 32-element partial
 * sum exactly; only the cross-block sum rounds, far below the float32 the GPU
 * accumulates in.  The Q8_1 quantizer is an encoding: a float decides an
 * integer, so it is computed in binary32 step by step, the precision the GPU
 * takes the same decision in.  Build with -ffp-contract=off so that no
 * multiply-add is fused behind our back.
 *
 * Every function is deterministic and independent of the OpenMP thread
 * count: each output element is computed by one thread in a fixed order.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Number formats, each decoded or encoded from its bit-field definition.    */
/* ------------------------------------------------------------------------ */

/* IEEE 754 binary16 -> double.  Sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is subnormal (fraction * 2^-24), exponent 31 is
 * infinity (fraction 0) or NaN. */
double oracle_f16_to_double(uint16_t h)
{
    double sign = (h & 0x8000) ? -1.0 : 1.0;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    if (e == 31)
        return f ? NAN : sign * INFINITY;
    if (e == 0)
        return sign * ldexp((double)f, -24);
    return sign * ldexp((double)(1024 + f), e - 25);
}

/* double -> IEEE 754 binary16, round to nearest, ties to even; values whose
 * magnitude reaches the rounding midpoint above the largest finite binary16
 * (65504 + 16 = 65520) overflow to infinity; subnormals are kept. */
uint16_t oracle_f16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7E00;
    if (a >= 65520.0)
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);            /* a = f * 2^e2 with f in [0.5, 1)            */
    int ue = e2 - 1;          /* a lies in the binade [2^ue, 2^(ue+1))      */
    if (ue < -14)
        ue = -14;             /* below 2^-14 the spacing stays 2^-24        */
    double quantum = ldexp(1.0, ue - 10);
    /* a / quantum is exact (power-of-two divisor); rint rounds half to even
     * in the default rounding mode. */
    double r = rint(a / quantum);
    /* Binade ue holds values r * 2^(ue-10) with r in [1024, 2048): exponent
     * field ue + 15, fraction r - 1024.  For ue = -14 and r < 1024 this is
     * the subnormal encoding; r = 2048 carries into the next exponent. */
    return sign | (uint16_t)((ue + 14) * 1024 + (int)r);
}

/* OCP FP8 E4M3 ("FN" variant) -> double.  Sign, 4-bit exponent (bias 7),
 * 3-bit mantissa; exponent 0 is subnormal (mantissa/8 * 2^-6); the single
 * pattern S.1111.111 is NaN and there is no infinity, so the largest finite
 * magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3_to_double(uint8_t b)
{
    double sign = (b & 0x80) ? -1.0 : 1.0;
    int e = (b >> 3) & 15;
    int m = b & 7;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        return sign * ldexp((double)m, -9);
    return sign * ldexp((double)(8 + m), e - 10);
}

/* FP4 E2M1 -> double (low four bits of c).  Sign, 2-bit exponent (bias 1),
 * 1-bit mantissa; exponent 0 is subnormal (mantissa/2).  No NaN or infinity;
 * code 8 is -0. */
double oracle_e2m1_to_double(uint8_t c)
{
    double sign = (c & 8) ? -1.0 : 1.0;
    int e = (c >> 1) & 3;
    int m = c & 1;
    if (e == 0)
        return sign * 0.5 * (double)m;
    return sign * ldexp((double)(2 + m), e - 2);
}

/* ------------------------------------------------------------------------ */
/* Q8_1 activation quantization.                                             */
/* ------------------------------------------------------------------------ */

/* Quantize each row of x (row-major [M][K], K % 32 == 0) in blocks of 32:
 *   amax  = max |x_i|
 *   d32   = amax / 127                       (binary32 division)
 *   q_i   = clamp(round_half_away(x_i / d32), -127, 127)   (binary32 division)
 *   d     = binary16(d32)
 *   s     = binary16(d32 * sum_i q_i)        (binary32 product)
 * and all zero when amax == 0.  Outputs: qs [M][K] int8, d and s [M][K/32]
 * as binary16 bit patterns.
 *
 * Readings: the pages name the quantized mat x vec kernel but never define
 * the activation format; the scale is amax/127 rounded to binary16, ties
 * round away from zero, codes use the binary32 scale, and the "sum" term is
 * the scale times the integer code sum, which is what makes the Q4_0 offset
 * identity below exact. */
void oracle_quantize_q8_1(const float *x, int M, int K,
                          int8_t *qs, uint16_t *d, uint16_t *s)
{
    int nb = K / 32;
    for (int m = 0; m < M; ++m) {
        for (int b = 0; b < nb; ++b) {
            const float *xb = x + (size_t)m * K + (size_t)b * 32;
            int8_t *qb = qs + (size_t)m * K + (size_t)b * 32;
            size_t bi = (size_t)m * nb + b;

            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax)
                    amax = a;
            }
            if (amax == 0.0f) {
                for (int i = 0; i < 32; ++i)
                    qb[i] = 0;
                d[bi] = 0;
                s[bi] = 0;
                continue;
            }
            float d32 = amax / 127.0f;
            int32_t sq = 0;
            for (int i = 0; i < 32; ++i) {
                float v = roundf(xb[i] / d32);   /* half away from zero */
                if (v > 127.0f)
                    v = 127.0f;
                if (v < -127.0f)
                    v = -127.0f;
                qb[i] = (int8_t)v;
                sq += qb[i];
            }
            float sum_scaled = d32 * (float)sq;
            d[bi] = oracle_f16_from_double((double)d32);
            s[bi] = oracle_f16_from_double((double)sum_scaled);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Q4_0 weights x Q8_1 activations.                                          */
/* ------------------------------------------------------------------------ */

/* Weight layout (planar): w_qs [N][K/2] bytes, w_d [N][K/32] binary16 bits.
 * Within block b of row n, byte j (0..15) holds code 32b+j in its low nibble
 * and code 32b+16+j in its high nibble.  A code q in 0..15 stands for the
 * weight (q - 8) * d.  (The pages keep llama.cpp's Q4_0 format unchanged and
 * do not show its byte order; this arrangement is our reading.) */
static inline int q4_code(const uint8_t *row, int k)
{
    int b = k / 32, i = k % 32;
    uint8_t byte = row[b * 16 + (i & 15)];
    return (i < 16) ? (byte & 15) : (byte >> 4);
}

/* Integer block dot: isum[m][n][b] = sum_{i<32} q4[n][32b+i] * q8[m][32b+i],
 * the raw unsigned code times the signed activation code, exact in int32
 * (|isum| <= 32 * 15 * 127).  This is the quantity the 4-way int8 dot
 * builds, four products at a time. */
void oracle_q4_0_blocksums(const uint8_t *w_qs, int N, int K,
                           const int8_t *a_qs, int M, int32_t *isum)
{
    int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = w_qs + (size_t)n * (K / 2);
        for (int m = 0; m < M; ++m) {
            const int8_t *a = a_qs + (size_t)m * K;
            for (int b = 0; b < nb; ++b) {
                int32_t acc = 0;
                for (int i = 0; i < 32; ++i)
                    acc += q4_code(row, 32 * b + i) * (int32_t)a[32 * b + i];
                isum[((size_t)m * N + n) * nb + b] = acc;
            }
        }
    }
}

/* y[m][n] = sum_b d4[n][b] * (d8[m][b] * isum_b - 8 * s8[m][b]).
 * Since s8 carries d8 * sum(q8), the -8 in every Q4_0 weight is applied
 * once per block through the sum term instead of per element.  Evaluated in
 * binary64 (isum is exact; products of the binary16 scales are exact).
 * Output y [M][N] as double. */
void oracle_mmvq_q4_0(const uint8_t *w_qs, const uint16_t *w_d, int N, int K,
                      const int8_t *a_qs, const uint16_t *a_d,
                      const uint16_t *a_s, int M, double *y)
{
    int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = w_qs + (size_t)n * (K / 2);
        for (int m = 0; m < M; ++m) {
            const int8_t *a = a_qs + (size_t)m * K;
            double acc = 0.0;
            for (int b = 0; b < nb; ++b) {
                int32_t isum = 0;
                for (int i = 0; i < 32; ++i)
                    isum += q4_code(row, 32 * b + i) * (int32_t)a[32 * b + i];
                double d4 = oracle_f16_to_double(w_d[(size_t)n * nb + b]);
                double d8 = oracle_f16_to_double(a_d[(size_t)m * nb + b]);
                double s8 = oracle_f16_to_double(a_s[(size_t)m * nb + b]);
                acc += d4 * (d8 * (double)isum - 8.0 * s8);
            }
            y[(size_t)m * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* K-quant weights (Q4_K, Q6_K) x Q8_1 activations.                          */
/* ------------------------------------------------------------------------ */

/* The CMP page ("llama.cpp results", table of models and quants) runs
 * Q4_K_M and Q6_K models through the same MMVQ int8 dot as Q4_0 but does not
 * define the formats.  The arithmetic below is the published GGUF K-quant
 * definition: super-blocks of 256 weights with per-sub-block integer scales.
 * The byte layouts are planar arrangements of our own with the same bits per
 * weight (the pages show no layout).
 *
 * Q4_K, per row and super-block S (256 weights = 8 sub-blocks of 32):
 *   qs  [N][K/2]: codes q in 0..15, same nibble order as Q4_0 (block b of
 *       32: byte j low nibble = element 32b+j, high nibble = 32b+16+j);
 *   hdr [N][K/256][16]: bytes 0-1 d (binary16), bytes 2-3 dmin (binary16),
 *       bytes 4..15 = p[0..11] holding the 6-bit scale sc_j and 6-bit min
 *       m_j of sub-block j = 0..7: sc_j = p[j] & 63,
 *       m_j = (p[j] >> 6) | (((p[8 + j/2] >> (4 (j%2))) & 15) << 2).
 *   weight = d * sc_j * q - dmin * m_j.
 * With Q8_1 activations (d8, s8 = d8 * sum q8 per block of 32), sub-block j
 * of super-block S is activation block b = 8S + j and contributes
 *   d * sc_j * d8_b * isum_b - dmin * m_j * s8_b,
 * isum_b = sum_{i<32} q * q8 (exact int32): the min is applied once per block
 * through the Q8_1 sum term, as Q4_0's -8 is. */
static inline void q4k_scale_min(const uint8_t *p, int j, int *sc, int *m)
{
    *sc = p[j] & 63;
    *m = (p[j] >> 6) | (((p[8 + j / 2] >> (4 * (j % 2))) & 15) << 2);
}

void oracle_mmvq_q4_k(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                      const int8_t *a_qs, const uint16_t *a_d,
                      const uint16_t *a_s, int M, double *y)
{
    int nb = K / 32, ns = K / 256;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = w_qs + (size_t)n * (K / 2);
        for (int m = 0; m < M; ++m) {
            const int8_t *a = a_qs + (size_t)m * K;
            double acc = 0.0;
            for (int b = 0; b < nb; ++b) {
                const uint8_t *h = w_hdr + ((size_t)n * ns + b / 8) * 16;
                int sc, mn;
                q4k_scale_min(h + 4, b % 8, &sc, &mn);
                double d = oracle_f16_to_double((uint16_t)(h[0] | (h[1] << 8)));
                double dmin = oracle_f16_to_double((uint16_t)(h[2] | (h[3] << 8)));
                int32_t isum = 0;
                for (int i = 0; i < 32; ++i)
                    isum += q4_code(row, 32 * b + i) * (int32_t)a[32 * b + i];
                double d8 = oracle_f16_to_double(a_d[(size_t)m * nb + b]);
                double s8 = oracle_f16_to_double(a_s[(size_t)m * nb + b]);
                acc += d * sc * (d8 * (double)isum) - dmin * mn * s8;
            }
            y[(size_t)m * N + n] = acc;
        }
    }
}

/* Q6_K, per row and super-block S (256 weights = 16 sub-blocks of 16):
 *   ql [N][K/2]: low 4 bits of each 6-bit code, Q4_0 nibble order per block
 *       of 32;
 *   qh [N][K/4]: high 2 bits, 8 bytes per block b of 32: byte 4h + t
 *       (h = 0, 1; t = 0..3), bits 2c..2c+1 = high bits of element
 *       32b + 16h + 4c + t (c = 0..3);
 *   sc [N][K/16]: int8 scale of each sub-block of 16;
 *   d  [N][K/256]: binary16.
 *   code q = low | (high << 4) in 0..63, weight = d * sc * (q - 32).
 * With Q8_1 activations, block b of 32 holds sub-blocks 2b and 2b+1:
 *   d * d8_b * (sc_2b * sum_{i<16} (q-32) q8 + sc_2b+1 * sum_{16<=i<32} (q-32) q8),
 * the bracket an exact integer; no Q8_1 sum term is needed. */
static inline int q6_code(const uint8_t *ql_row, const uint8_t *qh_row, int k)
{
    int b = k / 32, i = k % 32;
    int lo = q4_code(ql_row, k);
    int h = i / 16, c = (i % 16) / 4, t = i % 4;
    int hi = (qh_row[b * 8 + 4 * h + t] >> (2 * c)) & 3;
    return lo | (hi << 4);
}

void oracle_mmvq_q6_k(const uint8_t *w_ql, const uint8_t *w_qh, const int8_t *w_sc,
                      const uint16_t *w_d, int N, int K, const int8_t *a_qs,
                      const uint16_t *a_d, int M, double *y)
{
    int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        const uint8_t *ql = w_ql + (size_t)n * (K / 2);
        const uint8_t *qh = w_qh + (size_t)n * (K / 4);
        const int8_t *sc = w_sc + (size_t)n * (K / 16);
        for (int m = 0; m < M; ++m) {
            const int8_t *a = a_qs + (size_t)m * K;
            double acc = 0.0;
            for (int b = 0; b < nb; ++b) {
                int64_t itot = 0;
                for (int half = 0; half < 2; ++half) {
                    int32_t part = 0;
                    for (int i = 16 * half; i < 16 * half + 16; ++i)
                        part += (q6_code(ql, qh, 32 * b + i) - 32) * (int32_t)a[32 * b + i];
                    itot += (int64_t)sc[2 * b + half] * part;
                }
                double d = oracle_f16_to_double(w_d[(size_t)n * (K / 256) + b / 8]);
                double d8 = oracle_f16_to_double(a_d[(size_t)m * nb + b]);
                acc += d * (d8 * (double)itot);
            }
            y[(size_t)m * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* IQ4_XS weights x Q8_1 activations.                                        */
/* ------------------------------------------------------------------------ */

/* The CMP page's model table ("llama.cpp results") also runs a Qwen3-8B
 * IQ4_XS model through the MMVQ int8 dot, without defining the format.  The
 * published GGUF definition: super-blocks of 256 weights, one binary16 d,
 * and per sub-block j of 32 a 6-bit scale ls_j; each weight is a 4-bit
 * index into a fixed non-uniform table of 16 signed integers (the IQ4_NL
 * table, below), so weight = d * (ls_j - 32) * table[q].
 * Layout (planar, ours; the same 4.25 bits per weight as the original):
 *   qs  [N][K/2]: indices q in 0..15, same nibble order as Q4_0 (block b of
 *       32: byte j low nibble = element 32b+j, high nibble = 32b+16+j);
 *   hdr [N][K/256][8]: bytes 0-1 d (binary16), bytes 2-3 a little-endian
 *       16-bit word H whose bits 2j..2j+1 are the high two bits of ls_j,
 *       bytes 4..7 = L[0..3] whose nibble j%2 of L[j/2] is the low four bits:
 *       ls_j = ((L[j/2] >> (4 (j%2))) & 15) | (((H >> 2j) & 3) << 4).
 * With Q8_1 activations, sub-block j of super-block S is activation block
 * b = 8S + j and contributes d * (ls_j - 32) * d8_b * isum_b with
 * isum_b = sum_{i<32} table[q] * q8 (exact int32).  The table values are
 * signed, so there is no offset and the Q8_1 sum term is not used. */
static const int iq4nl_table[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                    1,    13,   25,  38,  53,  69,  89,  113};

static inline int iq4xs_scale(const uint8_t *hdr, int j)
{
    int H = hdr[2] | (hdr[3] << 8);
    int lo = (hdr[4 + j / 2] >> (4 * (j % 2))) & 15;
    int hi = (H >> (2 * j)) & 3;
    return lo | (hi << 4);
}

void oracle_mmvq_iq4_xs(const uint8_t *w_qs, const uint8_t *w_hdr, int N, int K,
                        const int8_t *a_qs, const uint16_t *a_d, int M, double *y)
{
    int nb = K / 32, ns = K / 256;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = w_qs + (size_t)n * (K / 2);
        for (int m = 0; m < M; ++m) {
            const int8_t *a = a_qs + (size_t)m * K;
            double acc = 0.0;
            for (int b = 0; b < nb; ++b) {
                const uint8_t *h = w_hdr + ((size_t)n * ns + b / 8) * 8;
                double d = oracle_f16_to_double((uint16_t)(h[0] | (h[1] << 8)));
                int ls = iq4xs_scale(h, b % 8);
                int32_t isum = 0;
                for (int i = 0; i < 32; ++i)
                    isum += iq4nl_table[q4_code(row, 32 * b + i)] * (int32_t)a[32 * b + i];
                double d8 = oracle_f16_to_double(a_d[(size_t)m * nb + b]);
                acc += d * (double)(ls - 32) * (d8 * (double)isum);
            }
            y[(size_t)m * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* NVFP4 weights x binary16 activations (W4A16).                             */
/* ------------------------------------------------------------------------ */

/* Layout: codes [N][K/2] bytes, element 2j in the low nibble of byte j and
 * element 2j+1 in the high nibble (our reading; the pages do not say);
 * scales [N][K/16] E4M3 bytes, one per 16 consecutive elements of a row;
 * g the per-tensor float32 scale.  x [M][K] and y [M][N] are binary16 bits.
 *
 * For each group j of 16: p_j = sum_i e2m1(c) * x, then acc += p_j *
 * (e4m3(scale_j) * g): the global scale folded into the group scale and each
 * group flushed into the wide accumulator.  y_acc receives acc (double),
 * y receives binary16(acc). */
void oracle_gemv_nvfp4_w4a16(const uint8_t *codes, const uint8_t *scales,
                             float g, int N, int K, const uint16_t *x, int M,
                             double *y_acc, uint16_t *y)
{
    int ng = K / 16;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = codes + (size_t)n * (K / 2);
        for (int m = 0; m < M; ++m) {
            const uint16_t *xr = x + (size_t)m * K;
            double acc = 0.0;
            for (int j = 0; j < ng; ++j) {
                double p = 0.0;
                for (int i = 0; i < 16; ++i) {
                    int k = 16 * j + i;
                    uint8_t byte = row[k / 2];
                    uint8_t c = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
                    p += oracle_e2m1_to_double(c) * oracle_f16_to_double(xr[k]);
                }
                double sc = oracle_e4m3_to_double(scales[(size_t)n * ng + j]) * (double)g;
                acc += p * sc;
            }
            y_acc[(size_t)m * N + n] = acc;
            y[(size_t)m * N + n] = oracle_f16_from_double(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 weights x binary16 activations (W8A16).                          */
/* ------------------------------------------------------------------------ */

/* Layout: w [N][K] E4M3 bytes, cs [N] float32 per-output-channel scales
 * (the pages do not state the FP8 scale granularity; per channel, applied
 * after the dot, is our reading).  y_acc = cs[n] * sum_k e4m3(w) * x,
 * y = binary16(y_acc). */
void oracle_gemv_fp8_w8a16(const uint8_t *w, const float *cs, int N, int K,
                           const uint16_t *x, int M, double *y_acc, uint16_t *y)
{
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        const uint8_t *row = w + (size_t)n * K;
        for (int m = 0; m < M; ++m) {
            const uint16_t *xr = x + (size_t)m * K;
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += oracle_e4m3_to_double(row[k]) * oracle_f16_to_double(xr[k]);
            double out = acc * (double)cs[n];
            y_acc[(size_t)m * N + n] = out;
            y[(size_t)m * N + n] = oracle_f16_from_double(out);
        }
    }
}

/* Threads the OpenMP loops above will use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Element-wise binary16 encode of an array (lets the tests sweep millions
 * of values through the same converter the functions above use). */
void oracle_f16_from_double_array(const double *v, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_f16_from_double(v[i]);
}
