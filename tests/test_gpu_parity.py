"""GPU parity: every entry point against the CPU oracle, element by element,
through the C ABI (via the thin binding), on seeded synthetic inputs.

Bars:
  * Q8_1 bytes (codes, d, s): bit-exact.
  * Q4_0 integer gate (unit scales, integer activations): bit-exact.
  * Q4_0 float32 output: normwise max|y - y_ref| / max|y_ref| <= 1e-3, and
    per element |y - y_ref| <= (K/32 + 8) * 2^-24 * mag, the float32
    summation bound (mag = sum over blocks of |d4| (|d8 isum| + 8 |s8|)).
  * binary16 outputs: normwise <= 2e-2, and per element
    |y - y_acc| <= 2^-10 |y_acc| + (K + 64) * 2^-24 * mag + 2^-24
    (one binary16 rounding plus float32 summation; mag = sum |w x|).
  * Exhaustive decode cases (every E4M3 code, every E2M1 x E4M3 pair):
    bit-exact, the products being exact in binary16.
The oracle is the reference throughout; nothing here derives an expected
value from the GPU.
"""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from skinny_gemm_amd import inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


# ------------------------------------------------------------------ helpers

def dev(a):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t, dtype=None):
    import torch

    torch.cuda.synchronize()
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def e4m3_table():
    return np.array([oracle.e4m3_to_double(b) for b in range(256)])


def e2m1_table():
    return np.array([oracle.e2m1_to_double(c) for c in range(16)])


def unpack_q4_0(w_qs):
    N, K2 = w_qs.shape
    b = w_qs.reshape(N, K2 // 16, 16)
    return np.concatenate([b & 15, b >> 4], axis=2).reshape(N, 2 * K2).astype(np.int64)


def unpack_nvfp4(codes):
    out = np.empty((codes.shape[0], 2 * codes.shape[1]), np.int64)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def check_f32(y, ref, mag, K, what):
    err = np.abs(y.astype(np.float64) - ref)
    norm = err.max() / max(np.abs(ref).max(), 1e-300)
    assert norm <= 1e-3, "%s: normwise %.3g" % (what, norm)
    bound = (K / 32 + 8) * 2.0 ** -24 * mag
    bad = err > bound
    assert not bad.any(), "%s: %d elements over the float32 bound, worst %s" % (
        what, bad.sum(), np.unravel_index(np.argmax(err - bound), err.shape))


def check_f16(y_bits, y_acc, mag, K, what):
    y = f16(y_bits)
    both_inf = np.isinf(y) & np.isinf(y_acc) & (np.sign(y) == np.sign(y_acc))
    assert np.all(np.isfinite(y) | both_inf), what + ": non-finite output"
    yf = np.where(both_inf, 0.0, y)
    ra = np.where(both_inf, 0.0, y_acc)
    err = np.abs(yf - ra)
    norm = err.max() / max(np.abs(ra).max(), 1e-300)
    assert norm <= 2e-2, "%s: normwise %.3g" % (what, norm)
    bound = 2.0 ** -10 * np.abs(ra) + (K + 64) * 2.0 ** -24 * mag + 2.0 ** -24
    bad = err > bound
    assert not bad.any(), "%s: %d elements over the bound, worst %s" % (
        what, bad.sum(), np.unravel_index(np.argmax(err - bound), err.shape))


def q4_mag(w_qs, w_d, a_qs, a_d, a_s):
    isum = oracle.q4_0_blocksums(w_qs, a_qs).astype(np.float64)          # [M][N][nb]
    d4 = np.abs(f16(w_d))                                                 # [N][nb]
    d8 = np.abs(f16(a_d))[:, None, :]
    s8 = np.abs(f16(a_s))[:, None, :]
    return (d4[None, :, :] * (d8 * np.abs(isum) + 8 * s8)).sum(axis=2)


def nvfp4_mag(codes, scales, g, x):
    W = np.abs(e2m1_table()[unpack_nvfp4(codes)] * np.repeat(e4m3_table()[scales], 16, axis=1) * g)
    return np.abs(f16(x)) @ W.T


def fp8_mag(w, cs, x):
    return (np.abs(f16(x)) @ np.abs(e4m3_table()[w]).T) * np.abs(cs)[None, :]


# ------------------------------------------------------------------ Q8_1

def run_quantize(x):
    import skinny_gemm_amd as sk

    qs, d, s = sk.quantize_act_q8_1(dev(x))
    return host(qs), host(d, np.uint16), host(s, np.uint16)


@pytest.mark.parametrize("M,K", [(1, 32), (1, 4096), (3, 96), (8, 11008), (5, 5120), (8, 17408),
                                 (37, 1024)])
def test_quantize_q8_1_bit_exact(M, K):
    x = inputs.normal_f32(M, K, 10 * M + K)
    got = run_quantize(x)
    want = oracle.quantize_q8_1(x)
    for g, w, name in zip(got, want, ("qs", "d", "s")):
        assert np.array_equal(g, w), name


def test_quantize_q8_1_adversarial_bit_exact():
    x = inputs.q8_1_unit_scale_source(4, 1024, 3)
    x[0, 1:64:2] += 0.5                       # exact halfway quotients
    x[1, :32] = 0.0                           # all-zero block
    x[1, 32:64] *= 1e-9                       # binary16 scale subnormal / zero
    x[2, :32] = 3.0e4                         # scaled sum overflows to +inf
    x[2, 32:64] = -3.0e4
    x[3] *= np.float32(1.0 / 3.0)             # inexact scales everywhere
    x[3, 64:96] = np.float32(1e-30)           # tiny amax
    got = run_quantize(x)
    want = oracle.quantize_q8_1(x)
    for g, w, name in zip(got, want, ("qs", "d", "s")):
        assert np.array_equal(g, w), name
    assert want[2][2, 0] == 0x7C00 and want[2][2, 1] == 0xFC00


# ------------------------------------------------------------------ Q4_0

def run_q4(w_qs, w_d, a_qs, a_d, a_s):
    import skinny_gemm_amd as sk

    return host(sk.mmvq_q4_0(dev(w_qs), dev(w_d), dev(a_qs), dev(a_d), dev(a_s)))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", [(1, 32), (4096 + 37, 256), (4099, 1376), (257, 11008),
                                 # matrix-core paths: wide / mid / narrow, chunks of 4
                                 # and 8 steps, ragged tiles, unequal K slices and
                                 # one empty slice
                                 (25000, 768), (9000, 1280), (40, 768), (700, 8192),
                                 # four waves sharing one activation chunk, ragged
                                 (30000, 1024),
                                 # narrow matrix-core route past the staged kernels'
                                 # N and K limits (eight K slices), and the staged
                                 # kernel in rounds at N = 6144
                                 (7000, 12800), (6144, 2048),
                                 # long rows at M <= 2: K split over two waves,
                                 # rounds of six
                                 (333, 20480), (97, 40960)])
def test_mmvq_q4_0_vs_oracle(M, N, K):
    _check_q4_0(M, N, K)


@pytest.mark.parametrize("M", [2, 3, 5, 8])
@pytest.mark.parametrize("N,K", [(9000, 1376),      # M * K / 32 not a multiple of 8
                                 (9000, 1280),      # ... a multiple of 8 for every M
                                 (4000, 288), (4096, 4096), (10000, 12288), (2000, 12320)])
def test_mmvq_q4_0_staged_activation_shapes(M, N, K):
    # the shapes that decide between the LDS-staged and the other kernels
    _check_q4_0(M, N, K)


def _check_q4_0(M, N, K):
    w_qs, w_d = inputs.q4_0_weights(N, K, 7 * N + K)
    x = inputs.normal_f32(M, K, 3 * M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    y = run_q4(w_qs, w_d, a_qs, a_d, a_s)
    ref = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    check_f32(y, ref, q4_mag(w_qs, w_d, a_qs, a_d, a_s), K, "q4_0 M=%d N=%d K=%d" % (M, N, K))


# ------------------------------------------------------------------ Q4_0, pre-permuted

def run_q4_packed(w_qs, w_d, a_qs, a_d, a_s):
    import skinny_gemm_amd as sk

    N, K = w_qs.shape[0], 2 * w_qs.shape[1]
    wp = sk.prepack_q4_0(dev(w_qs), dev(w_d))
    return host(sk.mmvq_q4_0_packed(wp, N, K, dev(a_qs), dev(a_d), dev(a_s)))


def q4_packed_layout_source(N, K):
    """From the layout the header defines: for every byte of the codes plane
    the flat index n * K/2 + byte of the code byte it holds, and for every
    binary16 of the scale plane the flat index n * K/32 + block of the scale
    it holds (-1 where zero)."""
    U, P, V, nb = (N + 15) // 16, K // 128, (K + 511) // 512, K // 32
    codes = np.full(1024 * U * P, -1, np.int64)
    scl = np.full(256 * U * V, -1, np.int64)
    for u in range(U):
        for l in range(64):
            j, g = l % 16, l // 16
            h, b = g // 2, g % 2
            n = 16 * u + j
            if n >= N:
                continue
            for p in range(P):
                for e in range(2):
                    at = 1024 * (u * P + p) + 16 * l + 8 * e
                    codes[at:at + 8] = n * (K // 2) + 16 * (4 * p + 2 * e + h) + 8 * b + np.arange(8)
        for h in range(2):
            for j in range(16):
                n = 16 * u + j
                if n >= N:
                    continue
                for v in range(V):
                    for t in range(8):
                        blk = 16 * v + 2 * t + h
                        if blk < nb:
                            scl[(512 * (u * V + v) + 256 * h + 16 * j + 2 * t) // 2] = n * nb + blk
    return codes, scl


@pytest.mark.parametrize("N,K", [(40, 2304), (16, 256), (3, 768)])
def test_prepack_q4_0_layout(N, K):
    # code bytes carry 16-bit labels (index + 1) sent as two byte planes,
    # scales carry their index + 1 directly; the packed copy must hold each
    # label exactly where the layout puts it, and 0 in the padding
    import skinny_gemm_amd as sk

    nc, ns = N * K // 2, N * K // 32
    label = np.arange(1, nc + 1, dtype=np.int64)
    assert nc < 1 << 16 and ns < 1 << 16
    w_d = np.arange(1, ns + 1, dtype=np.uint16).reshape(N, K // 32)
    size = sk.prepack_q4_0_size(N, K)
    U, P = (N + 15) // 16, K // 128
    got = np.zeros(size, np.int64)
    for shift in (0, 8):
        w_qs = ((label >> shift) & 255).astype(np.uint8).reshape(N, K // 2)
        packed = host(sk.prepack_q4_0(dev(w_qs), dev(w_d)))
        got |= packed.astype(np.int64) << shift
    scl = packed[1024 * U * P:].view(np.uint16)
    want_codes, want_scl = q4_packed_layout_source(N, K)
    assert np.array_equal(got[:1024 * U * P] - 1, want_codes)
    assert np.array_equal(scl.astype(np.int64) - 1, want_scl)


# (N, K) of the packed Q4_0 tests: every row of the packed dispatch table
# (>= 1100 tiles, 800..1099, 512..799, 257..511 with K >= 8192 or shorter,
# <= 256), each with chunks of 8 steps (K % 512 == 0) where it has them and
# of 4, ragged last tiles and K slices of unequal length
Q4P_SHAPES = [(30000, 1024), (30000, 768), (25000, 768), (16393, 4096), (16000, 1280),
              (9000, 1280), (9000, 2048), (5000, 8192), (5000, 1280), (3000, 4096),
              (129, 17408), (40, 768), (1, 256)]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", Q4P_SHAPES)
def test_mmvq_q4_0_packed_vs_oracle(M, N, K):
    w_qs, w_d = inputs.q4_0_weights(N, K, 5 * N + K)
    x = inputs.normal_f32(M, K, 7 * M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    y = run_q4_packed(w_qs, w_d, a_qs, a_d, a_s)
    ref = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    check_f32(y, ref, q4_mag(w_qs, w_d, a_qs, a_d, a_s), K,
              "q4_0 packed M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 2, 4, 6, 8])
@pytest.mark.parametrize("N,K", [(30000, 1024), (25000, 768), (16393, 4096), (16000, 1280),
                                 (9000, 1280), (5000, 8192), (3000, 4096), (5000, 1280),
                                 (40, 768)])
def test_mmvq_q4_0_packed_integer_gate_bit_exact(M, N, K):
    # unit scales and integer activations, as for the canonical layout:
    # every partial sum is an exact integer, so the result is the oracle's
    # bit for bit
    x = inputs.q8_1_unit_scale_source(M, K, 290 + M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    assert np.all(a_d == 0x3C00)
    assert 8 * np.abs(a_qs.astype(np.int64)).sum(axis=1).max() < 2 ** 24
    w_qs, _ = inputs.q4_0_weights(N, K, 291 + N)
    w_d = np.full((N, K // 32), 0x3C00, np.uint16)
    y = run_q4_packed(w_qs, w_d, a_qs, a_d, a_s)
    exact = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    assert np.array_equal(exact, np.rint(exact))
    assert np.array_equal(y.astype(np.float64), exact), "M=%d N=%d K=%d" % (M, N, K)


# (M, N, K) of the exact-integer gate, one or more per dispatch route of
# mmvq_q4_0 (the route each reaches is named).  With unit scales every block
# term isum - 8 s8 = sum (code - 8) q8 is an integer, and the sum of their
# magnitudes is checked below 2^24, so every partial sum in any order is an
# exact float32 integer and y must equal the oracle bit for bit.
Q4_GATE = [
    (1, 1031, 4096),      # vector kernel, one round of two blocks per lane
    (1, 25000, 4096),     # vector kernel, many workgroups
    (1, 300, 11008),      # vector kernel, six blocks per lane
    (1, 1031, 13824),     # vector kernel, one round of seven blocks per lane
    (1, 300, 10240),      # vector kernel, five blocks per lane
    (2, 301, 14336),      # vector kernel at M = 2, seven blocks per lane
    (1, 300, 20480),      # vector kernel, K split over two waves (six blocks each)
    (1, 1031, 28672),     # vector kernel, rounds of six blocks per lane
    (2, 1031, 4096),      # vector kernel at M = 2
    (2, 300, 16384),      # vector kernel at M = 2, eight blocks per lane
    (2, 301, 17408),      # vector kernel at M = 2, K split over two waves
    (2, 9000, 4096),      # plain staged-activation kernel (M = 2, N >= 8192)
    (1, 4096, 28672), (2, 4100, 13824),
                          # staged kernel in rounds for long rows at M <= 2
    (3, 1031, 4096), (4, 1031, 4096), (4, 2048, 8192),
                          # vector kernel (M <= 4, N <= 2048, K <= 8192)
    (3, 3000, 4096), (6, 1031, 4096), (8, 1031, 4096), (5, 6000, 4096),
    (6, 7000, 4096), (6, 8192, 4096),
                          # staged kernel in rounds (M <= 6 up to N = 8192, M = 7, 8
                          # up to N = 4096)
    (4, 5120, 13824), (3, 5000, 12800),
                          # staged kernel in rounds past the plain staged kernel's K
    (3, 9000, 4096), (4, 25000, 4096), (5, 9000, 4096),
                          # plain staged-activation kernel (M = 3..5, wider)
    (8, 7000, 4096), (8, 6144, 4096),
                          # matrix cores below 512 tiles: two K slices of 8 steps
    (8, 5000, 8192),      # ... two tiles per wave, four K slices (K >= 8192)
    (8, 3000, 16896),     # ... below 256 tiles: four K slices (activations past LDS)
    (8, 5000, 3840),      # ... eight K slices of 4 steps (K % 512 == 256)
    (6, 9000, 4096), (7, 9000, 4096), (8, 9000, 4096),
                          # matrix cores, two K slices, chunks of 8 steps
    (6, 14000, 4096), (8, 16393, 4096), (7, 14000, 3840),
                          # matrix cores, two waves share activations and two K slices
    (6, 25000, 4096), (8, 25000, 4096),
                          # matrix cores, two waves share each activation chunk
    (7, 30000, 4096), (8, 30000, 4096),
                          # matrix cores, four waves share each activation chunk
    (8, 25000, 3840),     # matrix cores, shared chunks of 4 steps (K % 512 == 256)
    (3, 9000, 12800), (4, 9000, 12800),
                          # matrix cores with 4 padded activation rows (K past the
                          # plain staged kernel's limit)
]


@pytest.mark.parametrize("M,N,K", Q4_GATE)
def test_mmvq_q4_0_integer_gate_bit_exact(M, N, K):
    x = inputs.q8_1_unit_scale_source(M, K, 90 + M + K)
    import skinny_gemm_amd as sk

    qs, d, s = sk.quantize_act_q8_1(dev(x))            # quantized on the device
    w_qs, _ = inputs.q4_0_weights(N, K, 91 + N)
    w_d = np.full((N, K // 32), 0x3C00, np.uint16)
    y = host(sk.mmvq_q4_0(dev(w_qs), dev(w_d), qs, d, s))
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    assert np.all(a_d == 0x3C00)                       # d8 = 1 in every block
    # |code - 8| <= 8, so the block terms' magnitudes sum to at most 8 sum |q8|
    assert 8 * np.abs(a_qs.astype(np.int64)).sum(axis=1).max() < 2 ** 24
    exact = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    assert np.array_equal(exact, np.rint(exact))
    assert np.array_equal(y.astype(np.float64), exact), "M=%d N=%d K=%d" % (M, N, K)
    # every code 8: all weights zero
    w8 = np.full((N, K // 2), 0x88, np.uint8)
    y8 = host(sk.mmvq_q4_0(dev(w8), dev(w_d), qs, d, s))
    assert np.all(y8 == 0.0)


@pytest.mark.parametrize("M,N", [(1, 1031), (1, 25000), (2, 9000)])
def test_mmvq_q4_0_f32act_integer_gate_bit_exact(M, N):
    # the fused entry point on integer activations and unit weight scales:
    # exact, equal to the oracle chain bit for bit
    K = 4096
    x = inputs.q8_1_unit_scale_source(M, K, 190 + M)
    w_qs, _ = inputs.q4_0_weights(N, K, 191 + N)
    w_d = np.full((N, K // 32), 0x3C00, np.uint16)
    y = run_q4_f32act(w_qs, w_d, x)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    assert 8 * np.abs(a_qs.astype(np.int64)).sum(axis=1).max() < 2 ** 24
    exact = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    assert np.array_equal(y.astype(np.float64), exact)


def test_q4_0_pipeline_device_quantize():
    # quantize on the device, then the GEMV, against the oracle chain
    M, N, K = 8, 2048 + 5, 4096
    import skinny_gemm_amd as sk

    x = inputs.normal_f32(M, K, 55)
    w_qs, w_d = inputs.q4_0_weights(N, K, 56)
    qs, d, s = sk.quantize_act_q8_1(dev(x))
    y = host(sk.mmvq_q4_0(dev(w_qs), dev(w_d), qs, d, s))
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    ref = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    check_f32(y, ref, q4_mag(w_qs, w_d, a_qs, a_d, a_s), K, "q4_0 pipeline")


def run_q4_f32act(w_qs, w_d, x):
    import skinny_gemm_amd as sk

    return host(sk.mmvq_q4_0_f32act(dev(w_qs), dev(w_d), dev(x)))


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("N,K", [(1, 32), (4096 + 37, 256), (4099, 1376), (257, 11008),
                                 (25000, 768), (40, 12288), (3000, 4096)])
def test_mmvq_q4_0_f32act_equals_two_calls_and_oracle(M, N, K):
    # one launch that quantizes in LDS: bit-identical to quantize_act_q8_1 +
    # mmvq_q4_0 (the same block arithmetic and dot), and within the float
    # tolerance of the oracle chain
    import skinny_gemm_amd as sk

    w_qs, w_d = inputs.q4_0_weights(N, K, 17 * N + K)
    x = inputs.normal_f32(M, K, 5 * M + K)
    y = run_q4_f32act(w_qs, w_d, x)
    qs, d, s = sk.quantize_act_q8_1(dev(x))
    y2 = host(sk.mmvq_q4_0(dev(w_qs), dev(w_d), qs, d, s))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    ref = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    check_f32(y, ref, q4_mag(w_qs, w_d, a_qs, a_d, a_s), K, "q4_0 f32act M=%d N=%d K=%d" % (M, N, K))


def test_mmvq_q4_0_f32act_adversarial_blocks():
    # integer blocks with unit scale, halves that round away from zero,
    # all-zero blocks: exact integer results, equal to the two-call path
    import skinny_gemm_amd as sk

    M, N, K = 2, 1031, 4096
    x = inputs.q8_1_unit_scale_source(M, K, 71)
    x[0, 64:96] = 0.0                                   # an all-zero block
    x[1, 128:160] = np.where(np.arange(32) % 2 == 0, 2.5, -2.5)   # ties
    x[1, 128] = 127.0
    w_qs, _ = inputs.q4_0_weights(N, K, 72)
    w_d = np.full((N, K // 32), 0x3C00, np.uint16)
    y = run_q4_f32act(w_qs, w_d, x)
    qs, d, s = sk.quantize_act_q8_1(dev(x))
    y2 = host(sk.mmvq_q4_0(dev(w_qs), dev(w_d), qs, d, s))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    exact = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    assert np.array_equal(y.astype(np.float64), exact)


# ------------------------------------------------------------------ K-quants

def q4_k_fields(hdr):
    """hdr [N][ns][16] -> d, dmin [N][ns] float64; sc, m [N][ns*8]."""
    N, ns, _ = hdr.shape
    d = f16(hdr[:, :, 0:2].copy().view(np.uint16)[:, :, 0])
    dmin = f16(hdr[:, :, 2:4].copy().view(np.uint16)[:, :, 0])
    p = hdr[:, :, 4:16].astype(np.int64)
    sc = p[:, :, 0:8] & 63
    hi = np.stack([(p[:, :, 8 + j // 2] >> (4 * (j % 2))) & 15 for j in range(8)], axis=2)
    return d, dmin, sc.reshape(N, ns * 8), ((p[:, :, 0:8] >> 6) | (hi << 2)).reshape(N, ns * 8)


def q4_k_mag(w_qs, w_hdr, a_qs, a_d, a_s):
    d, dmin, sc, m = q4_k_fields(w_hdr)
    W = unpack_q4_0(w_qs) * np.repeat(np.repeat(np.abs(d), 8, axis=1) * sc, 32, axis=1)
    A = np.abs(a_qs.astype(np.float64)) * np.repeat(np.abs(f16(a_d)), 32, axis=1)
    return A @ W.T + np.abs(f16(a_s)) @ (np.repeat(np.abs(dmin), 8, axis=1) * m).T


def unpack_q6_k(w_ql, w_qh):
    N, K2 = w_ql.shape
    K = 2 * K2
    qh = w_qh.reshape(N, K // 32, 2, 4).astype(np.int64)
    hi = np.stack([(qh >> (2 * c)) & 3 for c in range(4)], axis=3)     # [n][b][h][c][t]
    return unpack_q4_0(w_ql) | (hi.reshape(N, K) << 4)


def q6_k_mag(w_ql, w_qh, w_sc, w_d, a_qs, a_d):
    W = np.abs(unpack_q6_k(w_ql, w_qh) - 32) * np.repeat(np.abs(w_sc.astype(np.float64)), 16, axis=1) \
        * np.repeat(np.abs(f16(w_d)), 256, axis=1)
    A = np.abs(a_qs.astype(np.float64)) * np.repeat(np.abs(f16(a_d)), 32, axis=1)
    return A @ W.T


def run_q4_k(w_qs, w_hdr, a_qs, a_d, a_s):
    import skinny_gemm_amd as sk

    return host(sk.mmvq_q4_k(dev(w_qs), dev(w_hdr), dev(a_qs), dev(a_d), dev(a_s)))


def run_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d):
    import skinny_gemm_amd as sk

    return host(sk.mmvq_q6_k(dev(w_ql), dev(w_qh), dev(w_sc), dev(w_d), dev(a_qs), dev(a_d)))


KQ_SHAPES = [(1, 256), (4096 + 37, 256), (4099, 1280), (257, 12288), (1000, 4096), (63, 16384),
             (301, 13824), (77, 20480),   # one round of eight blocks per lane; rounds of six
             (5000, 8192),                # mid-width staged shapes (Q6_K: two or four rows)
             (4096, 17408),               # long rows staged at M <= 2
             (16384 + 9, 512),   # four-row vector shapes; two waves share activations (M >= 3)
             (28800 + 5, 512)]   # four waves share activations (Q4_K, M >= 3)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", KQ_SHAPES)
def test_mmvq_q4_k_vs_oracle(M, N, K):
    w_qs, w_hdr = inputs.q4_k_weights(N, K, 7 * N + K)
    x = inputs.normal_f32(M, K, 3 * M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    y = run_q4_k(w_qs, w_hdr, a_qs, a_d, a_s)
    ref = oracle.mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s)
    check_f32(y, ref, q4_k_mag(w_qs, w_hdr, a_qs, a_d, a_s), K,
              "q4_k M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", KQ_SHAPES)
def test_mmvq_q6_k_vs_oracle(M, N, K):
    w_ql, w_qh, w_sc, w_d = inputs.q6_k_weights(N, K, 11 * N + K)
    x = inputs.normal_f32(M, K, 5 * M + K)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    y = run_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    ref = oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    check_f32(y, ref, q6_k_mag(w_ql, w_qh, w_sc, w_d, a_qs, a_d), K,
              "q6_k M=%d N=%d K=%d" % (M, N, K))


def _q4_k_gate_weights(N, K, s, sc_mask):
    # d = dmin = 1, sub-block scales sc & sc_mask, mins in {0, 4}
    w_qs, w_hdr = inputs.q4_k_weights(N, K, s)
    w_hdr[:, :, 0:2] = np.array([0x3C00], np.uint16).view(np.uint8)
    w_hdr[:, :, 2:4] = np.array([0x3C00], np.uint16).view(np.uint8)
    w_hdr[:, :, 4:12] &= sc_mask
    w_hdr[:, :, 12:16] &= 0x11
    return w_qs, w_hdr


def _q4_k_gate_bound(w_qs, w_hdr, a_qs, a_s):
    # sum over blocks of |sc isum - m s8| <= sum_k sc q |q8| + sum_b m |s8|
    _, _, sc, mn = q4_k_fields(w_hdr)
    W = unpack_q4_0(w_qs) * np.repeat(sc, 32, axis=1)
    return (np.abs(a_qs.astype(np.float64)) @ W.T.astype(np.float64)
            + np.abs(f16(a_s)) @ mn.T.astype(np.float64)).max()


# (M, N, K, sc_mask) of the Q4_K exact-integer gate, one or more per route
Q4K_GATE = [
    (1, 300, 4096, 7), (2, 300, 4096, 7),       # vector kernel
    (1, 300, 5120, 7), (2, 300, 10240, 3),      # ... rounds of three and five blocks
    (1, 301, 14336, 3),                         # ... seven
    (1, 1031, 13824, 3), (2, 300, 16384, 3),    # vector kernel, eight blocks per lane
    (1, 300, 20480, 3),                         # vector kernel, rounds of six blocks
    (1, 4096, 13824, 3), (2, 4096, 13824, 3),   # staged kernel, long rows at M <= 2
    (3, 300, 4096, 7), (8, 300, 4096, 7),       # staged-activation kernel (N <= 6144)
    (4, 20000, 4096, 7),                        # vector kernel (M < 5, >= 1100 tiles)
    (3, 7000, 4096, 7), (8, 9000, 16640, 3),    # matrix cores, Q4_K narrow table: four
                                                # K slices of 4 steps
    (8, 5000, 16640, 3),                        # ... the same past the staged kernel's LDS
    (5, 10240, 2560, 7),                        # ... two K slices of 4 steps (600+ tiles)
    (4, 16393, 4096, 7), (8, 16393, 4096, 7),   # ... two waves share activations, two K
    (6, 14000, 3840, 7),                        # slices (800+ tiles), chunks of 8 and 4
    (8, 3000, 20480, 3), (8, 3000, 20736, 3),   # ... <= 256 tiles, activations past LDS:
                                                # four slices of 8 steps, eight of 4
    (6, 20000, 4096, 7),                        # matrix cores, two waves share activations
    (8, 28805, 4096, 7),                        # matrix cores, four waves share activations
]


@pytest.mark.parametrize("M,N,K,sc_mask", Q4K_GATE)
def test_q4_k_integer_gate_bit_exact(M, N, K, sc_mask):
    # unit d and dmin, small scales and mins, integer activations (d8 = 1,
    # s8 = sum q8 exactly): every block term is an integer and their
    # magnitudes sum below 2^24, so any summation order gives the exact result
    x = inputs.q8_1_unit_scale_source(M, K, 70 + M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    assert np.all(a_d == 0x3C00)
    w_qs, w_hdr = _q4_k_gate_weights(N, K, 71 + N, sc_mask)
    assert _q4_k_gate_bound(w_qs, w_hdr, a_qs, a_s) < 2 ** 24
    y = run_q4_k(w_qs, w_hdr, a_qs, a_d, a_s)
    ref = oracle.mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s)
    assert np.array_equal(ref, np.round(ref))
    assert np.array_equal(y.astype(np.float64), ref), "M=%d N=%d K=%d" % (M, N, K)


# ------------------------------------------------------------------ Q4_K, pre-permuted

def run_q4_k_packed(w_qs, w_hdr, a_qs, a_d, a_s):
    import skinny_gemm_amd as sk

    N, K = w_qs.shape[0], 2 * w_qs.shape[1]
    wp = sk.prepack_q4_k(dev(w_qs), dev(w_hdr))
    return host(sk.mmvq_q4_k_packed(wp, N, K, dev(a_qs), dev(a_d), dev(a_s)))


@pytest.mark.parametrize("N,K", [(40, 2304), (16, 256), (3, 768)])
def test_prepack_q4_k_layout(N, K):
    # code and header bytes carry 16-bit labels (index + 1) sent as two byte
    # planes: codes as in the Q4_0 layout, each row's 16-byte headers in
    # tile-major blocks of 256 bytes, zeros in the padding
    import skinny_gemm_amd as sk

    nc, nh = N * K // 2, N * K // 16
    label = np.arange(1, nc + nh + 1, dtype=np.int64)
    assert label[-1] < 1 << 16
    U, P, SB = (N + 15) // 16, K // 128, K // 256
    got = np.zeros(sk.prepack_q4_k_size(N, K), np.int64)
    for shift in (0, 8):
        plane = ((label >> shift) & 255).astype(np.uint8)
        w_qs = plane[:nc].reshape(N, K // 2)
        w_hdr = plane[nc:].reshape(N, SB, 16)
        got |= host(sk.prepack_q4_k(dev(w_qs), dev(w_hdr))).astype(np.int64) << shift
    want_codes, _ = q4_packed_layout_source(N, K)
    assert np.array_equal(got[:1024 * U * P] - 1, want_codes)
    hdr = np.full(256 * U * SB, -1, np.int64)
    for u in range(U):
        for q in range(SB):
            for j in range(16):
                n = 16 * u + j
                if n < N:
                    at = 256 * (u * SB + q) + 16 * j
                    hdr[at:at + 16] = nc + n * (K // 16) + 16 * q + np.arange(16)
    assert np.array_equal(got[1024 * U * P:] - 1, hdr)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", Q4P_SHAPES)
def test_mmvq_q4_k_packed_vs_oracle(M, N, K):
    w_qs, w_hdr = inputs.q4_k_weights(N, K, 9 * N + K)
    x = inputs.normal_f32(M, K, 11 * M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    y = run_q4_k_packed(w_qs, w_hdr, a_qs, a_d, a_s)
    ref = oracle.mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s)
    check_f32(y, ref, q4_k_mag(w_qs, w_hdr, a_qs, a_d, a_s), K,
              "q4_k packed M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 3, 5, 8])
@pytest.mark.parametrize("N,K,sc_mask", [(30000, 1024, 7), (25000, 768, 7), (16393, 4096, 7),
                                         (16000, 1280, 7), (9000, 1280, 7), (5000, 8192, 3),
                                         (3000, 4096, 7), (5000, 1280, 7), (40, 768, 7)])
def test_mmvq_q4_k_packed_integer_gate_bit_exact(M, N, K, sc_mask):
    # unit d and dmin, small scales and mins, integer activations, as for the
    # canonical layout: exact in any summation order
    x = inputs.q8_1_unit_scale_source(M, K, 170 + M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    w_qs, w_hdr = _q4_k_gate_weights(N, K, 171 + N, sc_mask)
    assert _q4_k_gate_bound(w_qs, w_hdr, a_qs, a_s) < 2 ** 24
    y = run_q4_k_packed(w_qs, w_hdr, a_qs, a_d, a_s)
    ref = oracle.mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s)
    assert np.array_equal(ref, np.round(ref))
    assert np.array_equal(y.astype(np.float64), ref), "M=%d N=%d K=%d" % (M, N, K)


# ------------------------------------------------------------------ Q6_K, pre-permuted

def run_q6_k_packed(w_ql, w_qh, w_sc, w_d, a_qs, a_d):
    import skinny_gemm_amd as sk

    N, K = w_ql.shape[0], 2 * w_ql.shape[1]
    wp = sk.prepack_q6_k(dev(w_ql), dev(w_qh), dev(w_sc), dev(w_d))
    return host(sk.mmvq_q6_k_packed(wp, N, K, dev(a_qs), dev(a_d)))


def q6_k_packed_expected(w_ql, w_qh, w_sc, w_d):
    """The packed bytes the header's layout defines, from the canonical arrays."""
    N, K = w_ql.shape[0], 2 * w_ql.shape[1]
    U, P, Q = (N + 15) // 16, K // 128, K // 256
    out = np.zeros(1024 * U * P + 1312 * U * Q, np.uint8)
    oH, oC = 1024 * U * P, 1024 * U * (P + Q)
    oD = oC + 256 * U * Q
    sc8 = w_sc.view(np.uint8)
    d8 = w_d.view(np.uint8)
    for u in range(U):
        for l in range(64):
            j, g = l % 16, l // 16
            n = 16 * u + j
            if n >= N:
                continue
            h = g % 2
            for p in range(P):
                for e in range(2):
                    b = 2 * (2 * p + e) + g // 2
                    low = (w_ql[n, 16 * b:16 * b + 16] >> (4 * h)) & 15
                    at = 1024 * (u * P + p) + 16 * l + 8 * e
                    out[at:at + 8] = low[:8] | (low[8:] << 4)
            for q in range(Q):
                for t in range(4):
                    b = 2 * (4 * q + t) + g // 2
                    at = oH + 1024 * (u * Q + q) + 16 * l + 4 * t
                    out[at:at + 4] = w_qh[n, 8 * b + 4 * h:8 * b + 4 * h + 4]
                    out[oC + 256 * (u * Q + q) + 4 * l + t] = sc8[n, 16 * q + 4 * t + g]
        for j in range(16):
            n = 16 * u + j
            if n < N:
                for q in range(Q):
                    at = oD + 32 * (u * Q + q) + 2 * j
                    out[at:at + 2] = d8[n, 2 * q:2 * q + 2]
    return out


@pytest.mark.parametrize("N,K", [(40, 2304), (16, 256), (3, 768)])
def test_prepack_q6_k_layout(N, K):
    # random canonical arrays through prepack_q6_k against the bytes the
    # header's layout defines (padding rows zero)
    import skinny_gemm_amd as sk

    w_ql, w_qh, w_sc, w_d = inputs.q6_k_weights(N, K, 5 + N + K)
    got = host(sk.prepack_q6_k(dev(w_ql), dev(w_qh), dev(w_sc), dev(w_d)))
    assert np.array_equal(got, q6_k_packed_expected(w_ql, w_qh, w_sc, w_d))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", Q4P_SHAPES)
def test_mmvq_q6_k_packed_vs_oracle(M, N, K):
    w_ql, w_qh, w_sc, w_d = inputs.q6_k_weights(N, K, 13 * N + K)
    x = inputs.normal_f32(M, K, 17 * M + K)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    y = run_q6_k_packed(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    ref = oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    check_f32(y, ref, q6_k_mag(w_ql, w_qh, w_sc, w_d, a_qs, a_d), K,
              "q6_k packed M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 3, 5, 8])
@pytest.mark.parametrize("N,K,sc_max", [(30000, 1024, 2), (16393, 4096, 2), (16000, 1280, 2),
                                        (9000, 1280, 2), (5000, 8192, 1), (3000, 4096, 2),
                                        (40, 768, 2)])
def test_mmvq_q6_k_packed_integer_gate_bit_exact(M, N, K, sc_max):
    # unit d, scales in -sc_max..sc_max, integer activations: exact in any
    # order, so equal to the oracle bit for bit
    x = inputs.q8_1_unit_scale_source(M, K, 370 + M + K)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    w_ql, w_qh, w_sc, _ = inputs.q6_k_weights(N, K, 372 + N)
    w_sc = (w_sc.astype(np.int64) % (2 * sc_max + 1) - sc_max).astype(np.int8)
    w_d = np.full((N, K // 256), 0x3C00, np.uint16)
    assert 32 * sc_max * np.abs(a_qs.astype(np.int64)).sum(axis=1).max() < 2 ** 24
    y = run_q6_k_packed(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    ref = oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    assert np.array_equal(ref, np.round(ref))
    assert np.array_equal(y.astype(np.float64), ref), "M=%d N=%d K=%d" % (M, N, K)


@pytest.mark.parametrize("M,N,K,sc_max", [
    (1, 300, 4096, 2), (4, 300, 4096, 2), (8, 300, 4096, 2),
    (1, 300, 5120, 2), (2, 300, 10240, 1),      # vector kernel, rounds of three and five
    (1, 301, 14336, 1),                         # ... seven
    (1, 1031, 13824, 1), (2, 300, 13824, 1),    # vector kernel, eight blocks per lane
    (2, 4100, 13824, 1),                        # staged, long rows at M = 2
    (3, 6000, 4096, 2),                         # staged, one row per wave (mid-width)
    (4, 5000, 8192, 1), (6, 5000, 8192, 1),     # staged, two / four rows per wave
])
def test_q6_k_integer_gate_bit_exact(M, N, K, sc_max):
    # unit d, scales in -sc_max..sc_max, integer activations: exact in any order
    x = inputs.q8_1_unit_scale_source(M, K, 70 + M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    w_ql, w_qh, w_sc, _ = inputs.q6_k_weights(N, K, 72)
    w_sc = (w_sc.astype(np.int64) % (2 * sc_max + 1) - sc_max).astype(np.int8)
    w_d = np.full((N, K // 256), 0x3C00, np.uint16)
    # |q - 32| <= 32 and |sc| <= sc_max: the block terms sum to at most
    # 32 sc_max sum |q8|
    assert 32 * sc_max * np.abs(a_qs.astype(np.int64)).sum(axis=1).max() < 2 ** 24
    y6 = run_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    ref6 = oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    assert np.array_equal(ref6, np.round(ref6))
    assert np.array_equal(y6.astype(np.float64), ref6)


def test_k_quant_pipeline_device_quantize():
    # quantize_act_q8_1 on the device feeding both K-quant GEMVs
    import skinny_gemm_amd as sk

    M, N, K = 3, 2048 + 5, 4096
    x = inputs.normal_f32(M, K, 81)
    qs, d, s = sk.quantize_act_q8_1(dev(x))
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    w_qs, w_hdr = inputs.q4_k_weights(N, K, 82)
    y = host(sk.mmvq_q4_k(dev(w_qs), dev(w_hdr), qs, d, s))
    check_f32(y, oracle.mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s),
              q4_k_mag(w_qs, w_hdr, a_qs, a_d, a_s), K, "q4_k pipeline")
    w_ql, w_qh, w_sc, w_d = inputs.q6_k_weights(N, K, 83)
    y6 = host(sk.mmvq_q6_k(dev(w_ql), dev(w_qh), dev(w_sc), dev(w_d), qs, d))
    check_f32(y6, oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d),
              q6_k_mag(w_ql, w_qh, w_sc, w_d, a_qs, a_d), K, "q6_k pipeline")


# ------------------------------------------------------------------ IQ4_XS

def iq4_table():
    from conftest import read_golden

    return np.array([int(v) for v in read_golden("iq4_nl_table.txt")[0]["table"]], np.int64)


def iq4_xs_abs_weights(w_qs, w_hdr):
    """|d (ls - 32) T[q]| per weight, [N][K] float64."""
    N, ns, _ = w_hdr.shape
    d = f16(w_hdr[:, :, 0:2].copy().view(np.uint16)[:, :, 0])
    H = w_hdr[:, :, 2].astype(np.int64) | (w_hdr[:, :, 3].astype(np.int64) << 8)
    L = w_hdr[:, :, 4:8].astype(np.int64)
    ls = np.stack([((L[:, :, j // 2] >> (4 * (j % 2))) & 15) | (((H >> (2 * j)) & 3) << 4)
                   for j in range(8)], axis=2).reshape(N, ns * 8)
    scale = np.repeat(np.repeat(np.abs(d), 8, axis=1) * np.abs(ls - 32), 32, axis=1)
    return np.abs(iq4_table()[unpack_q4_0(w_qs)]) * scale


def iq4_xs_mag(w_qs, w_hdr, a_qs, a_d):
    A = np.abs(a_qs.astype(np.float64)) * np.repeat(np.abs(f16(a_d)), 32, axis=1)
    return A @ iq4_xs_abs_weights(w_qs, w_hdr).T


def run_iq4_xs(w_qs, w_hdr, a_qs, a_d):
    import skinny_gemm_amd as sk

    return host(sk.mmvq_iq4_xs(dev(w_qs), dev(w_hdr), dev(a_qs), dev(a_d)))


# KQ_SHAPES, and matrices of 48M+ weights that take the matrix cores from
# M = 6 (four-way split; two-way split; two waves sharing activations; an
# eight-way split at 256 tiles; K % 512 == 256)
IQ4_SHAPES = KQ_SHAPES + [(5000 + 3, 12800), (16384 + 9, 4096), (20000 + 3, 4096),
                          (4096, 12288), (16000, 4352)]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", IQ4_SHAPES)
def test_mmvq_iq4_xs_vs_oracle(M, N, K):
    w_qs, w_hdr = inputs.iq4_xs_weights(N, K, 17 * N + K)
    x = inputs.normal_f32(M, K, 7 * M + K)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    y = run_iq4_xs(w_qs, w_hdr, a_qs, a_d)
    ref = oracle.mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d)
    check_f32(y, ref, iq4_xs_mag(w_qs, w_hdr, a_qs, a_d), K,
              "iq4_xs M=%d N=%d K=%d" % (M, N, K))


# (M, N, K) of the IQ4_XS exact-integer gate, one or more per route
IQ4_GATE = [
    (1, 300, 4096), (2, 300, 4096),             # vector kernel, two blocks per lane
    (1, 16400, 4096),                           # ... one block per round (M = 1, wide)
    (2, 16400, 4096),                           # ... four rows per wave (M = 2, wide)
    (1, 300, 5120), (1, 300, 8192),             # ... three and four blocks per lane
    (1, 300, 10240), (1, 300, 12288),           # ... five and six
    (1, 301, 13824),                            # ... seven
    (2, 300, 12288),                            # ... rounds of two blocks (M = 2)
    (1, 300, 16384), (2, 300, 16384),           # ... eight blocks per lane
    (1, 300, 20480), (2, 300, 20480),           # ... rounds of six blocks
    (3, 300, 4096), (5, 6000, 4096),            # vector kernel, M >= 3, two rows per wave
    (4, 16400, 4096), (8, 16400, 4096),         # ... four rows per wave (wide)
    (3, 300, 8192),                             # staged activations (long rows)
    (8, 300, 4096), (6, 4096, 4096),            # ... narrow matrices from M = 6
    (8, 300, 16384),                            # ... the largest staging batch
    (8, 77, 20480), (8, 16400, 20480),          # vector kernel past the LDS limit
    (6, 5003, 12800), (8, 5003, 12800),         # matrix cores: four-way K split
    (7, 16393, 4096),                           # ... two-way split
    (6, 20003, 4096), (8, 20003, 4096),         # ... two waves share activations
    (6, 4096, 12288),                           # ... eight-way split (256 tiles)
    (8, 4100, 12288),                           # ... four-way split, ragged tile
    (8, 16000, 4352),                           # ... K % 512 == 256
    (8, 4000, 12288),                           # staged kernel just below 48M weights
]


@pytest.mark.parametrize("M,N,K", IQ4_GATE)
def test_mmvq_iq4_xs_integer_gate_bit_exact(M, N, K):
    # d = 1, every scale ls = 33 (weight = T[q]), integer activations with
    # d8 = 1: every block sum and every partial sum is an integer below 2^24,
    # so the result is exact in any summation order
    x = inputs.q8_1_unit_scale_source(M, K, 90 + M + K, spread=60 if K <= 4096 else 6)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    w_qs, w_hdr = inputs.iq4_xs_weights(N, K, 91 + N)
    w_hdr[:, :, 0:2] = np.array([0x3C00], np.uint16).view(np.uint8)
    w_hdr[:, :, 2:4] = 0xAA                       # high bits 2 in every sub-block
    w_hdr[:, :, 4:8] = 0x11                       # low bits 1: ls = 33
    W = np.abs(iq4_table()[unpack_q4_0(w_qs)]).astype(np.float64)
    assert (np.abs(a_qs.astype(np.float64)) @ W.T).max() < 2 ** 24
    y = run_iq4_xs(w_qs, w_hdr, a_qs, a_d)
    ref = oracle.mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d)
    assert np.array_equal(ref, np.round(ref))
    assert np.array_equal(y.astype(np.float64), ref)


def test_mmvq_iq4_xs_device_quantize_and_zero_sizes():
    import skinny_gemm_amd as sk
    import torch

    M, N, K = 5, 3000 + 7, 5120
    x = inputs.normal_f32(M, K, 93)
    qs, d, _ = sk.quantize_act_q8_1(dev(x))
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    w_qs, w_hdr = inputs.iq4_xs_weights(N, K, 94)
    y = host(sk.mmvq_iq4_xs(dev(w_qs), dev(w_hdr), qs, d))
    check_f32(y, oracle.mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d), iq4_xs_mag(w_qs, w_hdr, a_qs, a_d),
              K, "iq4_xs pipeline")
    # M = 0 and N = 0 enqueue nothing and leave y untouched
    y0 = torch.full((0, N), 1.0, device="cuda")
    sk.mmvq_iq4_xs(dev(w_qs), dev(w_hdr), qs[:0], d[:0], y0)
    yn = torch.full((M, 0), 1.0, device="cuda")
    sk.mmvq_iq4_xs(dev(w_qs[:0]), dev(w_hdr[:0]), qs, d, yn)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ IQ4_XS, pre-permuted

def run_iq4_xs_packed(w_qs, w_hdr, a_qs, a_d):
    import skinny_gemm_amd as sk

    N, K = w_qs.shape[0], 2 * w_qs.shape[1]
    wp = sk.prepack_iq4_xs(dev(w_qs), dev(w_hdr))
    return host(sk.mmvq_iq4_xs_packed(wp, N, K, dev(a_qs), dev(a_d)))


@pytest.mark.parametrize("N,K", [(40, 2304), (16, 256), (3, 768), (17, 512)])
def test_prepack_iq4_xs_layout(N, K):
    # code and header bytes carry 16-bit labels (index + 1) sent as two byte
    # planes: codes as in the Q4_0 layout, each row's 8-byte headers in
    # tile-major blocks of 128 bytes, zeros in the padding
    import skinny_gemm_amd as sk

    nc, nh = N * K // 2, N * K // 32
    label = np.arange(1, nc + nh + 1, dtype=np.int64)
    assert label[-1] < 1 << 16
    U, P, SB = (N + 15) // 16, K // 128, K // 256
    got = np.zeros(sk.prepack_iq4_xs_size(N, K), np.int64)
    for shift in (0, 8):
        plane = ((label >> shift) & 255).astype(np.uint8)
        w_qs = plane[:nc].reshape(N, K // 2)
        w_hdr = plane[nc:].reshape(N, SB, 8)
        got |= host(sk.prepack_iq4_xs(dev(w_qs), dev(w_hdr))).astype(np.int64) << shift
    want_codes, _ = q4_packed_layout_source(N, K)
    assert np.array_equal(got[:1024 * U * P] - 1, want_codes)
    hdr = np.full(128 * U * SB, -1, np.int64)
    for u in range(U):
        for q in range(SB):
            for j in range(16):
                n = 16 * u + j
                if n < N:
                    at = 128 * (u * SB + q) + 8 * j
                    hdr[at:at + 8] = nc + n * (K // 32) + 8 * q + np.arange(8)
    assert np.array_equal(got[1024 * U * P:] - 1, hdr)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", Q4P_SHAPES)
def test_mmvq_iq4_xs_packed_vs_oracle(M, N, K):
    w_qs, w_hdr = inputs.iq4_xs_weights(N, K, 23 * N + K)
    x = inputs.normal_f32(M, K, 29 * M + K)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    y = run_iq4_xs_packed(w_qs, w_hdr, a_qs, a_d)
    ref = oracle.mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d)
    check_f32(y, ref, iq4_xs_mag(w_qs, w_hdr, a_qs, a_d), K,
              "iq4_xs packed M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 3, 5, 8])
@pytest.mark.parametrize("N,K", [(30000, 1024), (25000, 768), (16393, 4096), (16000, 1280),
                                 (9000, 1280), (5000, 8192), (3000, 4096), (5000, 1280),
                                 (40, 768)])
def test_mmvq_iq4_xs_packed_integer_gate_bit_exact(M, N, K):
    # d = 1, ls = 33, integer activations with d8 = 1, as for the canonical
    # layout: exact in any summation order
    x = inputs.q8_1_unit_scale_source(M, K, 190 + M + K, spread=60 if K <= 4096 else 6)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    w_qs, w_hdr = inputs.iq4_xs_weights(N, K, 191 + N)
    w_hdr[:, :, 0:2] = np.array([0x3C00], np.uint16).view(np.uint8)
    w_hdr[:, :, 2:4] = 0xAA
    w_hdr[:, :, 4:8] = 0x11
    W = np.abs(iq4_table()[unpack_q4_0(w_qs)]).astype(np.float64)
    assert (np.abs(a_qs.astype(np.float64)) @ W.T).max() < 2 ** 24
    y = run_iq4_xs_packed(w_qs, w_hdr, a_qs, a_d)
    ref = oracle.mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d)
    assert np.array_equal(ref, np.round(ref))
    assert np.array_equal(y.astype(np.float64), ref), "M=%d N=%d K=%d" % (M, N, K)


# ------------------------------------------------------------------ NVFP4

def run_nvfp4(codes, scales, g, x):
    import skinny_gemm_amd as sk

    return host(sk.gemv_nvfp4_w4a16(dev(codes), dev(scales), g, dev(x)), np.uint16)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16])
@pytest.mark.parametrize("N,K,g", [(1, 32, 1.0), (4096 + 19, 320, 1.0), (1030, 5120, 0.5),
                                   (129, 17408, 2.0 ** -3),
                                   # matrix-core paths: wide / mid / narrow, chunk of 2
                                   # steps (K % 512 == 256), ragged tiles, K slices
                                   # of unequal length and one empty slice
                                   (25000, 768, 1.0), (9000, 1280, 1.0), (40, 768, 1.0),
                                   # narrow (<= 256 tiles): eight K slices of 2-step
                                   # chunks, the last one short
                                   (2000, 11008, 1.0)])
def test_gemv_nvfp4_vs_oracle(M, N, K, g):
    codes, scales, _ = inputs.nvfp4_weights(N, K, 5 * N + K)
    x = inputs.normal_f16_bits(M, K, 2 * M + K)
    y = run_nvfp4(codes, scales, g, x)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, g, x)
    check_f16(y, y_acc, nvfp4_mag(codes, scales, g, x), K, "nvfp4 M=%d N=%d K=%d" % (M, N, K))


def test_gemv_nvfp4_every_code_and_scale_bit_exact():
    # row n: the 16 E2M1 codes at elements 0..15 under group scale n (NaN
    # scale codes replaced by 1.0); x row m is one-hot at element e, so
    # y[m][n] = e2m1(e) * e4m3(n): exact in binary16
    N, K = 256, 32
    codes = np.zeros((N, K // 2), np.uint8)
    codes[:, :8] = np.array([c0 | (c1 << 4) for c0, c1 in zip(range(0, 16, 2), range(1, 16, 2))],
                            np.uint8)
    codes[:, 8:] = np.array([0x12, 0x34, 0x56, 0x70, 0x89, 0xAB, 0xCD, 0xEF], np.uint8)
    scales = np.zeros((N, 2), np.uint8)
    scales[:, 0] = np.arange(256)
    scales[:, 1] = np.arange(256)[::-1]
    scales[scales == 0x7F] = 0x38
    scales[scales == 0xFF] = 0x38
    for base in (0, 8, 16, 24):
        x = np.zeros((8, K), np.float16)
        for m in range(8):
            x[m, base + m] = 1.0
        xb = x.view(np.uint16)
        # M = 1, 2 and 3: the staged-activation kernel; M = 8: the plain one
        for M in (1, 2, 3, 8):
            y = run_nvfp4(codes, scales, 1.0, xb[:M])
            _, want = oracle.gemv_nvfp4_w4a16(codes, scales, 1.0, xb[:M])
            assert np.array_equal(y, want), (base, M)


@pytest.mark.parametrize("N,K", [(8192, 5120), (8193, 5120), (16385, 5120), (8195, 3072),
                                 (16384, 3072)])
def test_gemv_nvfp4_flat_vs_oracle(N, K):
    # M = 1 with K / 32 an odd multiple of 32 chunks on wide matrices: the
    # flat mapping (two adjacent rows spread evenly over a wave's lanes); an
    # odd N leaves the last wave one row
    codes, scales, g = inputs.nvfp4_weights(N, K, 3 * N + K)
    x = inputs.normal_f16_bits(1, K, N + 1)
    y = run_nvfp4(codes, scales, g, x)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, g, x)
    check_f16(y, y_acc, nvfp4_mag(codes, scales, g, x), K, "nvfp4 flat N=%d K=%d" % (N, K))


def test_gemv_nvfp4_flat_bit_exact():
    # flat mapping, exact: row n holds the 16 E2M1 codes (twice) in chunk
    # n % nc only, under group scales n % 256 and its mirror (NaN codes
    # replaced by 1.0); x holds one 1.0 per chunk at element (base + 5 c) %
    # 32, so y[n] is one code times one scale, exact in binary16 -- a chunk
    # credited to the wrong row, lane or position shows as a wrong bit
    N, K = 8193, 3072
    nc = K // 32
    pattern = np.array([c0 | (c1 << 4) for c0, c1 in zip(range(0, 16, 2), range(1, 16, 2))] +
                       [0x12, 0x34, 0x56, 0x70, 0x89, 0xAB, 0xCD, 0xEF], np.uint8)
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    for n in range(N):
        c = n % nc
        codes[n, 16 * c:16 * c + 16] = pattern
        scales[n, 2 * c] = n % 256
        scales[n, 2 * c + 1] = 255 - n % 256
    scales[(scales & 0x7F) == 0x7F] = 0x38
    for base in (0, 11, 22):
        x = np.zeros((1, K), np.float16)
        for c in range(nc):
            x[0, 32 * c + (base + 5 * c) % 32] = 1.0
        xb = x.view(np.uint16)
        y = run_nvfp4(codes, scales, 1.0, xb)
        _, want = oracle.gemv_nvfp4_w4a16(codes, scales, 1.0, xb)
        assert np.array_equal(y, want), base
        assert np.count_nonzero(f16(want)) > N // 2


# (M, N, K) of the outlier test, one per route of gemv_nvfp4_w4a16
NV_OUTLIER = [
    (1, 512, 5120),       # staged activations, two rows per wave (small matrix)
    (1, 512, 17408),      # staged activations, three rows per wave
    (1, 8192, 5120),      # flat mapping
    (2, 512, 5120),       # staged activations at M = 2
    (2, 512, 40992),      # plain vector kernel (activations past the LDS limit)
    (3, 512, 5120),       # staged activations at M = 3
    (4, 512, 5120),       # matrix cores, 4 padded activation rows
    (8, 512, 5120),       # matrix cores, 8 padded activation rows
    (8, 512, 5152),       # plain vector kernel (K % 256 != 0)
    (16, 512, 5120),      # matrix cores, 16 activation rows
]


@pytest.mark.parametrize("M,N,K", NV_OUTLIER)
def test_gemv_nvfp4_outliers(M, N, K):
    # activation outliers of +-2e4: any binary16 partial sum would overflow
    codes, scales, _ = inputs.nvfp4_weights(N, K, 61 + K)
    x = inputs.normal_f16_bits(M, K, 62 + M).view(np.float16).copy()
    rng = np.random.Generator(np.random.PCG64(63 + M))
    idx = rng.integers(0, K, size=(M, 24))
    for m in range(M):
        x[m, idx[m]] = np.float16(2.0e4) * np.where(rng.integers(0, 2, 24) == 0, -1, 1)
    xb = x.view(np.uint16)
    y = run_nvfp4(codes, scales, 1.0, xb)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, 1.0, xb)
    assert np.all(np.isfinite(y_acc))
    check_f16(y, y_acc, nvfp4_mag(codes, scales, 1.0, xb), K, "nvfp4 outliers M=%d N=%d K=%d" % (
        M, N, K))


def test_gemv_nvfp4_sixteen_rows_bit_exact():
    # M = 16 on the matrix-core path (K % 256 == 0): row n holds code n % 16
    # at element n under group scale n (NaN codes replaced by 1.0), every
    # other code +0; x row m is 1 at the elements k with k % 16 == m, so
    # y[m][n] = e2m1(n % 16) * e4m3(n) when n % 16 == m and 0 otherwise --
    # one exact term per output, which pins the mapping of all 16 columns
    N = K = 256
    codes = np.zeros((N, K // 2), np.uint8)
    n = np.arange(N)
    codes[n, n // 2] = np.where(n % 2 == 0, n % 16, (n % 16) << 4).astype(np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    sc = np.arange(256)
    sc[[0x7F, 0xFF]] = 0x38
    scales[n, n // 16] = sc
    x = np.zeros((16, K), np.float16)
    for m in range(16):
        x[m, m::16] = 1.0
    xb = x.view(np.uint16)
    y = run_nvfp4(codes, scales, 1.0, xb)
    _, want = oracle.gemv_nvfp4_w4a16(codes, scales, 1.0, xb)
    assert np.array_equal(y, want)
    assert np.count_nonzero(f16(want)) > 200


# ------------------------------------------------------------------ NVFP4, pre-permuted

def run_nvfp4_packed(codes, scales, g, x):
    import skinny_gemm_amd as sk

    N, K = codes.shape[0], 2 * codes.shape[1]
    wp = sk.prepack_nvfp4(dev(codes), dev(scales))
    return host(sk.gemv_nvfp4_w4a16_packed(wp, N, K, g, dev(x)), np.uint16)


def packed_layout_source(N, K):
    """For every byte of the packed copy, the flat index of the canonical
    byte it holds (codes: n * K/2 + b; scales: N * K/2 + n * K/16 + b), or -1
    for a zero byte, from the layout the header defines."""
    U, S = (N + 15) // 16, K // 128
    V = (S + 7) // 8
    src = np.full(1024 * U * (S + V), -1, np.int64)
    for u in range(U):
        for l in range(64):
            i, g = l % 16, l // 16
            n = 16 * u + i
            if n >= N:
                continue
            for s in range(S):
                at = 1024 * (u * S + s) + 16 * l
                src[at:at + 16] = n * (K // 2) + 64 * s + 16 * g + np.arange(16)
            for v in range(V):
                for t in range(8):
                    step = 8 * v + t
                    if step >= S:
                        continue
                    at = 1024 * (U * S + u * V + v) + 16 * l + 2 * t
                    src[at:at + 2] = N * (K // 2) + n * (K // 16) + 8 * step + 2 * g + np.arange(2)
    return src


@pytest.mark.parametrize("N,K", [(40, 2304), (16, 256), (1, 1280)])
def test_prepack_nvfp4_layout(N, K):
    # every canonical byte gets a distinct 16-bit label (index + 1), sent
    # through prepack_nvfp4 as two byte planes; the packed copy must hold
    # each label exactly where the layout puts it, and 0 in the padding
    import skinny_gemm_amd as sk

    nc, ns = N * K // 2, N * K // 16
    label = np.arange(1, nc + ns + 1, dtype=np.int64)
    assert label[-1] < 1 << 16
    got = np.zeros(sk.prepack_nvfp4_size(N, K), np.int64)
    for shift in (0, 8):
        plane = ((label >> shift) & 255).astype(np.uint8)
        codes = plane[:nc].reshape(N, K // 2)
        scales = plane[nc:].reshape(N, K // 16)
        got |= host(sk.prepack_nvfp4(dev(codes), dev(scales))).astype(np.int64) << shift
    assert np.array_equal(got - 1, packed_layout_source(N, K))


# (N, K) of the packed parity test: every row of the packed dispatch tables
# at M <= 2, M = 3..4 and M = 5..16 (tiles >= 1536, 1100..1535, 800..1099,
# 600..799, 512..599, 257..511 with K >= 8192 or shorter, <= 256 with
# K <= 8192 or longer), each with chunks of 4 steps (K % 512 == 0) and of 2
# (K % 512 == 256), ragged last tiles, and K slices of unequal length
NVP_SHAPES = [(25000, 768), (25000, 1024), (20000, 768), (20000, 1024), (16000, 1280),
              (16000, 1024), (9000, 1280), (9000, 2048), (5000, 8192), (5000, 8448),
              (5000, 1280), (2000, 4096), (40, 768), (2000, 11008), (1, 256), (129, 17408)]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 12, 16])
@pytest.mark.parametrize("N,K", NVP_SHAPES)
def test_gemv_nvfp4_packed_vs_oracle(M, N, K):
    codes, scales, g = inputs.nvfp4_weights(N, K, 7 * N + K)
    x = inputs.normal_f16_bits(M, K, 3 * M + K)
    y = run_nvfp4_packed(codes, scales, g, x)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, g, x)
    check_f16(y, y_acc, nvfp4_mag(codes, scales, g, x), K,
              "nvfp4 packed M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(1, 512, 5120), (2, 512, 5120), (8, 512, 5120),
                                   (16, 512, 5120), (8, 25000, 768)])
def test_gemv_nvfp4_packed_outliers(M, N, K):
    # activation outliers of +-2e4, as for the canonical layout
    codes, scales, _ = inputs.nvfp4_weights(N, K, 61 + K)
    x = inputs.normal_f16_bits(M, K, 62 + M).view(np.float16).copy()
    rng = np.random.Generator(np.random.PCG64(63 + M))
    idx = rng.integers(0, K, size=(M, 24))
    for m in range(M):
        x[m, idx[m]] = np.float16(2.0e4) * np.where(rng.integers(0, 2, 24) == 0, -1, 1)
    xb = x.view(np.uint16)
    y = run_nvfp4_packed(codes, scales, 1.0, xb)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, 1.0, xb)
    assert np.all(np.isfinite(y_acc))
    check_f16(y, y_acc, nvfp4_mag(codes, scales, 1.0, xb), K,
              "nvfp4 packed outliers M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_gemv_nvfp4_packed_one_term_bit_exact(M):
    # one exact E2M1 x E4M3 term per output through the packed copy, at every
    # padded row count: row n holds code (n // 16) % 16 at element n under
    # group scale n (NaN codes replaced by 1.0), every other code +0; x row m
    # is 1 at the elements k with k % 16 == m, so y[m][n] is that one term
    # when n % 16 == m and 0 otherwise, and each row m < M meets every code
    N = K = 256
    codes = np.zeros((N, K // 2), np.uint8)
    n = np.arange(N)
    code = (n // 16) % 16
    codes[n, n // 2] = np.where(n % 2 == 0, code, code << 4).astype(np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    sc = np.arange(256)
    sc[[0x7F, 0xFF]] = 0x38
    scales[n, n // 16] = sc
    x = np.zeros((16, K), np.float16)
    for m in range(16):
        x[m, m::16] = 1.0
    xb = x.view(np.uint16)[:M]
    y = run_nvfp4_packed(codes, scales, 1.0, xb)
    _, want = oracle.gemv_nvfp4_w4a16(codes, scales, 1.0, xb)
    assert np.array_equal(y, want)
    assert np.count_nonzero(f16(want)) >= 12 * M


# ------------------------------------------------------------------ FP8

def run_fp8(w, cs, x):
    import skinny_gemm_amd as sk

    return host(sk.gemv_fp8_w8a16(dev(w), dev(cs), dev(x)), np.uint16)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16])
@pytest.mark.parametrize("N,K", [(1, 16), (4096 + 3, 272), (1030, 5120), (129, 17408),
                                 # matrix-core paths, as for NVFP4
                                 (25000, 768), (9000, 1280), (40, 768), (2000, 11008)])
def test_gemv_fp8_vs_oracle(M, N, K):
    w, cs = inputs.fp8_weights(N, K, 3 * N + K)
    x = inputs.normal_f16_bits(M, K, 4 * M + K)
    y = run_fp8(w, cs, x)
    y_acc, _ = oracle.gemv_fp8_w8a16(w, cs, x)
    check_f16(y, y_acc, fp8_mag(w, cs, x), K, "fp8 M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("N,K", [(8192, 8192), (8193, 8192), (8192, 8224), (2048 + 5, 5120),
                                 (4096, 4096), (4097, 4096), (8, 32)])
def test_small_matrix_route_vs_oracle(M, N, K):
    # one activation row on a matrix with N and K up to 8192, or two on one of
    # up to 2^24 weights, takes two weight rows per wave in both binary16
    # formats; one step past a bound takes three
    x = inputs.normal_f16_bits(M, K, 7 + K)
    codes, scales, _ = inputs.nvfp4_weights(N, K, 11 * N + K)
    y = run_nvfp4(codes, scales, 0.75, x)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, 0.75, x)
    check_f16(y, y_acc, nvfp4_mag(codes, scales, 0.75, x), K, "nvfp4 M=%d N=%d K=%d" % (M, N, K))
    w, cs = inputs.fp8_weights(N, K, 13 * N + K)
    y = run_fp8(w, cs, x)
    y_acc, _ = oracle.gemv_fp8_w8a16(w, cs, x)
    check_f16(y, y_acc, fp8_mag(w, cs, x), K, "fp8 M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [17, 31, 48, 64, 80, 96])
@pytest.mark.parametrize("N,K", [(4096 + 3, 272),     # K % 256 != 0: passes of 8 rows
                                 (1030, 5120),        # narrow: activation rows in groups
                                 (3000, 1280),
                                 (9000, 768),         # mid (row groups above M = 48)
                                 (24576 + 40, 256),   # wide: more waves share each chunk
                                 (40, 768),
                                 (600, 17408)])       # narrow, long: row groups of 16 / 32
def test_gemv_fp8_chunked_vs_oracle(M, N, K):
    w, cs = inputs.fp8_weights(N, K, 13 * N + K)
    x = inputs.normal_f16_bits(M, K, 6 * M + K)
    y = run_fp8(w, cs, x)
    y_acc, _ = oracle.gemv_fp8_w8a16(w, cs, x)
    check_f16(y, y_acc, fp8_mag(w, cs, x), K, "fp8 M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("N,K", [(256, 256),          # narrow: three groups of 32 rows
                                 (256, 512),          # narrow, K % 512 == 0: six groups
                                                      # of 16 rows with a K split
                                 (24576 + 256, 256)]) # wide: one pass, six column tiles
def test_gemv_fp8_ninety_six_rows_bit_exact(N, K):
    # M = 96 on the chunked path: row n holds code n % 256 at element n % 256;
    # x row m is 1 at the elements k with k % 96 == m (so each output has at
    # most one exact term) -- pins the mapping of all 96 activation rows
    w = np.zeros((N, K), np.uint8)
    codes = np.arange(256)
    codes[[0x7F, 0xFF]] = 0x38
    w[np.arange(N), np.arange(N) % 256] = codes[np.arange(N) % 256]
    cs = np.ones(N, np.float32)
    x = np.zeros((96, K), np.float16)
    for m in range(96):
        x[m, m::96] = 1.0
    xb = x.view(np.uint16)
    y = run_fp8(w, cs, xb)
    _, want = oracle.gemv_fp8_w8a16(w, cs, xb)
    assert np.array_equal(y, want)
    assert np.count_nonzero(f16(want)) > 200


def test_gemv_fp8_every_code_bit_exact():
    # row n holds code n at element n % 16; x row m is one-hot at m and m+8
    N, K = 256, 16
    w = np.zeros((N, K), np.uint8)
    codes = np.arange(256)
    codes[[0x7F, 0xFF]] = 0x38                # NaN codes are unspecified
    w[np.arange(N), np.arange(N) % 16] = codes
    cs = np.ones(N, np.float32)
    x = np.zeros((8, K), np.float16)
    for m in range(8):
        x[m, m] = 1.0
        x[m, m + 8] = 1.0
    xb = x.view(np.uint16)
    # M <= 6: the staged-activation kernel; M = 8: the plain one
    for M in (1, 2, 3, 4, 5, 6, 8):
        y = run_fp8(w, cs, xb[:M])
        _, want = oracle.gemv_fp8_w8a16(w, cs, xb[:M])
        assert np.array_equal(y, want), M


def test_gemv_fp8_sixteen_rows_bit_exact():
    # M = 16 on the matrix-core path: row n holds code n at element n; x row
    # m is 1 at the elements k with k % 16 == m, so y[m][n] = e4m3(n) when
    # n % 16 == m and 0 otherwise
    N = K = 256
    w = np.zeros((N, K), np.uint8)
    codes = np.arange(256)
    codes[[0x7F, 0xFF]] = 0x38
    w[np.arange(N), np.arange(N)] = codes
    cs = np.ones(N, np.float32)
    x = np.zeros((16, K), np.float16)
    for m in range(16):
        x[m, m::16] = 1.0
    xb = x.view(np.uint16)
    y = run_fp8(w, cs, xb)
    _, want = oracle.gemv_fp8_w8a16(w, cs, xb)
    assert np.array_equal(y, want)
    assert np.count_nonzero(f16(want)) > 200


# ------------------------------------------------------------------ FP8, pre-permuted

def run_fp8_packed(w, cs, x):
    import skinny_gemm_amd as sk

    N, K = w.shape
    wp = sk.prepack_fp8(dev(w))
    return host(sk.gemv_fp8_w8a16_packed(wp, N, K, dev(cs), dev(x)), np.uint16)


def fp8_packed_layout_source(N, K):
    """From the layout the header defines: for every packed byte the flat
    index n * K + k of the weight byte it holds (-1 where zero)."""
    U, S = (N + 15) // 16, K // 128
    src = np.full(2048 * U * S, -1, np.int64)
    for u in range(U):
        for l in range(64):
            i, g = l % 16, l // 16
            n = 16 * u + i
            if n >= N:
                continue
            for s in range(S):
                for e in range(2):
                    at = 2048 * (u * S + s) + 1024 * e + 16 * l
                    src[at:at + 16] = n * K + 128 * s + 32 * g + 16 * e + np.arange(16)
    return src


@pytest.mark.parametrize("N,K", [(40, 768), (16, 256), (3, 512)])
def test_prepack_fp8_layout(N, K):
    # every weight byte gets a distinct 16-bit label (index + 1) sent as two
    # byte planes; each must land where the layout puts it, 0 in the padding
    import skinny_gemm_amd as sk

    label = np.arange(1, N * K + 1, dtype=np.int64)
    assert label[-1] < 1 << 16
    got = np.zeros(sk.prepack_fp8_size(N, K), np.int64)
    for shift in (0, 8):
        w = ((label >> shift) & 255).astype(np.uint8).reshape(N, K)
        got |= host(sk.prepack_fp8(dev(w))).astype(np.int64) << shift
    assert np.array_equal(got - 1, fp8_packed_layout_source(N, K))


# (N, K) of the packed FP8 parity test: every row of the packed dispatch
# tables at M <= 2, M = 3..4 and M = 5..16 (tiles >= 1536, 1100..1535,
# 600..1099, 512..599, 257..511 with K >= 8192 or shorter, <= 256), with
# chunks of 4 steps (K % 512 == 0) and of 2, ragged last tiles and unequal K
# slices; the one row these sizes cannot reach at oracle cost (>= 1536 tiles
# with K >= 8192 at M > 8) is in the sampled full-size test
F8P_SHAPES = [(25000, 768), (25000, 1024), (20000, 768), (20000, 1024), (16000, 1280),
              (16000, 1024), (9000, 1280), (9000, 2048), (5000, 8192), (5000, 8448),
              (5000, 1280), (2000, 4096), (2000, 11008), (129, 17408), (40, 768), (1, 256)]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 12, 16])
@pytest.mark.parametrize("N,K", F8P_SHAPES)
def test_gemv_fp8_packed_vs_oracle(M, N, K):
    w, cs = inputs.fp8_weights(N, K, 17 * N + K)
    x = inputs.normal_f16_bits(M, K, 5 * M + K)
    y = run_fp8_packed(w, cs, x)
    y_acc, _ = oracle.gemv_fp8_w8a16(w, cs, x)
    check_f16(y, y_acc, fp8_mag(w, cs, x), K, "fp8 packed M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [17, 31, 48, 64, 80, 96])
@pytest.mark.parametrize("N,K", [(24576 + 40, 256),   # wide: one pass, MP / 16 column tiles
                                 (24576 + 40, 768),
                                 (9000, 1280),        # narrower: groups of 16 rows, two
                                 (3000, 1280),        # tiles per wave and four waves sharing
                                 (600, 17408),        # (below 512 tiles up to M = 48: one
                                 (40, 768)])          # tile per wave)
def test_gemv_fp8_packed_many_rows_vs_oracle(M, N, K):
    w, cs = inputs.fp8_weights(N, K, 19 * N + K)
    x = inputs.normal_f16_bits(M, K, 8 * M + K)
    y = run_fp8_packed(w, cs, x)
    y_acc, _ = oracle.gemv_fp8_w8a16(w, cs, x)
    check_f16(y, y_acc, fp8_mag(w, cs, x), K, "fp8 packed M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (2, 256, 256), (4, 256, 256), (8, 256, 256),
                                   (16, 256, 256), (96, 256, 256), (96, 24576 + 256, 256)])
def test_gemv_fp8_packed_one_term_bit_exact(M, N, K):
    # row n holds code n % 256 at element n % 256 (NaN codes replaced by 1.0);
    # x row m is 1 at the elements k with k % M' == m (M' = 16, or 96 for
    # M = 96), so each output has at most one exact term: pins the packed
    # order and the mapping of every activation row
    w = np.zeros((N, K), np.uint8)
    codes = np.arange(256)
    codes[[0x7F, 0xFF]] = 0x38
    w[np.arange(N), np.arange(N) % 256] = codes[np.arange(N) % 256]
    cs = np.ones(N, np.float32)
    period = 96 if M == 96 else 16
    x = np.zeros((M, K), np.float16)
    for m in range(M):
        x[m, m::period] = 1.0
    xb = x.view(np.uint16)
    y = run_fp8_packed(w, cs, xb)
    _, want = oracle.gemv_fp8_w8a16(w, cs, xb)
    assert np.array_equal(y, want)
    assert np.count_nonzero(f16(want)) >= 12 * min(M, 16)


@pytest.mark.parametrize("fmt,M,K", [
    # activations staged in LDS up to M K = 80 K elements: at the limit the
    # staging takes several batches per thread; just past it, the plain kernel
    ("nvfp4", 1, 81920), ("nvfp4", 1, 81952), ("nvfp4", 2, 40960), ("nvfp4", 2, 40992),
    ("nvfp4", 3, 27296), ("nvfp4", 3, 27328),
    ("fp8", 1, 81920), ("fp8", 3, 27296), ("fp8", 4, 20480), ("fp8", 4, 20496),
    ("fp8", 5, 16384), ("fp8", 5, 16400), ("fp8", 6, 13648), ("fp8", 6, 13664)])
@pytest.mark.parametrize("N", [5, 37])
def test_staged_activation_limits(fmt, M, K, N):
    x = inputs.normal_f16_bits(M, K, 7 * M + N, std=0.25)
    if fmt == "nvfp4":
        codes, scales, g = inputs.nvfp4_weights(N, K, 11 * N + K)
        y = run_nvfp4(codes, scales, g, x)
        y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, g, x)
        mag = nvfp4_mag(codes, scales, g, x)
    else:
        w, cs = inputs.fp8_weights(N, K, 13 * N + K)
        y = run_fp8(w, cs, x)
        y_acc, _ = oracle.gemv_fp8_w8a16(w, cs, x)
        mag = fp8_mag(w, cs, x)
    check_f16(y, y_acc, mag, K, "%s staged limit M=%d N=%d K=%d" % (fmt, M, N, K))


# ------------------------------------------------------------------ seeded random shapes

def random_shapes(seed, count, kmult, kmax, max_m, nk_max=1.6e7, mnk_max=1e8):
    """(M, N, K) drawn log-uniformly over the valid range of an entry point:
    N in [1, 40000], K a multiple of kmult up to kmax, M in [1, max_m], sized
    so that the oracle finishes quickly.  The hand-picked shapes above pin
    the routing boundaries they name; these reach the combinations between."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < count:
        K = max(kmult, int(np.exp(rng.uniform(np.log(kmult), np.log(kmax)))) // kmult * kmult)
        if K >= 256 and rng.uniform() < 0.5:
            K = K // 256 * 256               # half of them tile the matrix-core chunks
        M = int(rng.integers(1, max_m + 1))
        n_max = min(40000.0, nk_max / K, mnk_max / (M * K))
        if n_max < 1:
            continue
        N = int(np.exp(rng.uniform(0.0, np.log(n_max))))
        out.append((M, max(N, 1), K))
    return out


@pytest.mark.parametrize("M,N,K", random_shapes(101, 64, 32, 16384, 8))
def test_mmvq_q4_0_random_shapes(M, N, K):
    _check_q4_0(M, N, K)


@pytest.mark.parametrize("M,N,K", random_shapes(102, 24, 32, 12288, 2))
def test_mmvq_q4_0_f32act_random_shapes(M, N, K):
    w_qs, w_d = inputs.q4_0_weights(N, K, 5 * N + K)
    x = inputs.normal_f32(M, K, 7 * M + K)
    y = run_q4_f32act(w_qs, w_d, x)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    ref = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    check_f32(y, ref, q4_mag(w_qs, w_d, a_qs, a_d, a_s), K,
              "q4_0 f32act M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", random_shapes(103, 64, 32, 20480, 16))
def test_gemv_nvfp4_random_shapes(M, N, K):
    codes, scales, g = inputs.nvfp4_weights(N, K, 9 * N + K)
    x = inputs.normal_f16_bits(M, K, 5 * M + K)
    y = run_nvfp4(codes, scales, g, x)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, g, x)
    check_f16(y, y_acc, nvfp4_mag(codes, scales, g, x), K,
              "nvfp4 M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", random_shapes(104, 64, 16, 20480, 96))
def test_gemv_fp8_random_shapes(M, N, K):
    w, cs = inputs.fp8_weights(N, K, 13 * N + K)
    x = inputs.normal_f16_bits(M, K, 3 * M + K)
    y = run_fp8(w, cs, x)
    y_acc, _ = oracle.gemv_fp8_w8a16(w, cs, x)
    check_f16(y, y_acc, fp8_mag(w, cs, x), K, "fp8 M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", random_shapes(105, 32, 256, 16384, 8))
def test_k_quants_random_shapes(M, N, K):
    w_qs, w_hdr = inputs.q4_k_weights(N, K, 3 * N + K)
    w_ql, w_qh, w_sc, w_d = inputs.q6_k_weights(N, K, 5 * N + K)
    x = inputs.normal_f32(M, K, 11 * M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    check_f32(run_q4_k(w_qs, w_hdr, a_qs, a_d, a_s), oracle.mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s),
              q4_k_mag(w_qs, w_hdr, a_qs, a_d, a_s), K, "q4_k M=%d N=%d K=%d" % (M, N, K))
    check_f32(run_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d),
              oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d),
              q6_k_mag(w_ql, w_qh, w_sc, w_d, a_qs, a_d), K, "q6_k M=%d N=%d K=%d" % (M, N, K))


def iq4_random_big():
    # matrices of 48M+ weights at M >= 6 (the matrix-core route), drawn the
    # same way with a larger size budget
    return [s for s in random_shapes(107, 400, 512, 16384, 8, nk_max=1.2e8, mnk_max=1e9)
            if s[0] >= 6 and s[1] * s[2] >= 51e6]


@pytest.mark.parametrize("M,N,K", random_shapes(106, 32, 256, 16384, 8) + iq4_random_big())
def test_mmvq_iq4_xs_random_shapes(M, N, K):
    w_qs, w_hdr = inputs.iq4_xs_weights(N, K, 13 * N + K)
    x = inputs.normal_f32(M, K, 17 * M + K)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    check_f32(run_iq4_xs(w_qs, w_hdr, a_qs, a_d), oracle.mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d),
              iq4_xs_mag(w_qs, w_hdr, a_qs, a_d), K, "iq4_xs M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", random_shapes(108, 24, 256, 16384, 8))
def test_packed_q4_family_random_shapes(M, N, K):
    # Q4_0, Q4_K, Q6_K and IQ4_XS through their pre-permuted copies (K % 256
    # == 0), against the oracle on the canonical weights
    x = inputs.normal_f32(M, K, 19 * M + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    w_qs, w_d = inputs.q4_0_weights(N, K, 2 * N + K)
    check_f32(run_q4_packed(w_qs, w_d, a_qs, a_d, a_s), oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s),
              q4_mag(w_qs, w_d, a_qs, a_d, a_s), K, "q4_0 packed M=%d N=%d K=%d" % (M, N, K))
    k_qs, k_hdr = inputs.q4_k_weights(N, K, 3 * N + K)
    check_f32(run_q4_k_packed(k_qs, k_hdr, a_qs, a_d, a_s),
              oracle.mmvq_q4_k(k_qs, k_hdr, a_qs, a_d, a_s),
              q4_k_mag(k_qs, k_hdr, a_qs, a_d, a_s), K, "q4_k packed M=%d N=%d K=%d" % (M, N, K))
    ql, qh, sc, d6 = inputs.q6_k_weights(N, K, 5 * N + K)
    check_f32(run_q6_k_packed(ql, qh, sc, d6, a_qs, a_d),
              oracle.mmvq_q6_k(ql, qh, sc, d6, a_qs, a_d),
              q6_k_mag(ql, qh, sc, d6, a_qs, a_d), K, "q6_k packed M=%d N=%d K=%d" % (M, N, K))
    i_qs, i_hdr = inputs.iq4_xs_weights(N, K, 7 * N + K)
    check_f32(run_iq4_xs_packed(i_qs, i_hdr, a_qs, a_d), oracle.mmvq_iq4_xs(i_qs, i_hdr, a_qs, a_d),
              iq4_xs_mag(i_qs, i_hdr, a_qs, a_d), K, "iq4_xs packed M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", random_shapes(110, 24, 256, 20480, 16))
def test_packed_nvfp4_random_shapes(M, N, K):
    codes, scales, g = inputs.nvfp4_weights(N, K, 11 * N + K)
    x = inputs.normal_f16_bits(M, K, 13 * M + K)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, g, x)
    check_f16(run_nvfp4_packed(codes, scales, g, x), y_acc, nvfp4_mag(codes, scales, g, x), K,
              "nvfp4 packed M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", random_shapes(111, 24, 256, 20480, 96))
def test_packed_fp8_random_shapes(M, N, K):
    w, cs = inputs.fp8_weights(N, K, 17 * N + K)
    x = inputs.normal_f16_bits(M, K, 19 * M + K)
    y_acc, _ = oracle.gemv_fp8_w8a16(w, cs, x)
    check_f16(run_fp8_packed(w, cs, x), y_acc, fp8_mag(w, cs, x), K,
              "fp8 packed M=%d N=%d K=%d" % (M, N, K))


# ------------------------------------------------------------------ full sizes (sampled rows)

LLAMA_Q4 = [(12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008), (32000, 4096)]
QWEN_FP = [(10240, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]


def sample_rows(N, k=48, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.unique(np.concatenate([[0, 1, N - 2, N - 1], rng.integers(0, N, k)]))


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_q4_0_full_sizes_sampled(M):
    import skinny_gemm_amd as sk

    for si, (N, K) in enumerate(LLAMA_Q4):
        w_qs, w_d = inputs.q4_0_weights(N, K, inputs.seed(1, si, 0))
        x = inputs.normal_f32(M, K, inputs.seed(2, si, 2) + M)
        qs, d, s = sk.quantize_act_q8_1(dev(x))
        y = host(sk.mmvq_q4_0(dev(w_qs), dev(w_d), qs, d, s))
        a_qs, a_d, a_s = oracle.quantize_q8_1(x)
        assert np.array_equal(host(qs), a_qs) and np.array_equal(host(d, np.uint16), a_d)
        rows = sample_rows(N, seed=si)
        ref = oracle.mmvq_q4_0(w_qs[rows], w_d[rows], a_qs, a_d, a_s)
        mag = q4_mag(w_qs[rows], w_d[rows], a_qs, a_d, a_s)
        check_f32(y[:, rows], ref, mag, K, "q4_0 full M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_q4_0_packed_full_sizes_sampled(M):
    import skinny_gemm_amd as sk

    for si, (N, K) in enumerate(LLAMA_Q4):
        w_qs, w_d = inputs.q4_0_weights(N, K, inputs.seed(1, si, 0))
        x = inputs.normal_f32(M, K, inputs.seed(2, si, 2) + M)
        a_qs, a_d, a_s = oracle.quantize_q8_1(x)
        wp = sk.prepack_q4_0(dev(w_qs), dev(w_d))
        y = host(sk.mmvq_q4_0_packed(wp, N, K, dev(a_qs), dev(a_d), dev(a_s)))
        rows = sample_rows(N, seed=si)
        ref = oracle.mmvq_q4_0(w_qs[rows], w_d[rows], a_qs, a_d, a_s)
        mag = q4_mag(w_qs[rows], w_d[rows], a_qs, a_d, a_s)
        check_f32(y[:, rows], ref, mag, K, "q4_0 packed full M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 4, 8])
def test_q4_k_packed_full_sizes_sampled(M):
    import skinny_gemm_amd as sk

    for si, (N, K) in enumerate([(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]):
        w_qs, w_hdr = inputs.q4_k_weights(N, K, inputs.seed(5, si, 0))
        x = inputs.normal_f32(M, K, inputs.seed(5, si, 2) + M)
        a_qs, a_d, a_s = oracle.quantize_q8_1(x)
        wp = sk.prepack_q4_k(dev(w_qs), dev(w_hdr))
        y = host(sk.mmvq_q4_k_packed(wp, N, K, dev(a_qs), dev(a_d), dev(a_s)))
        rows = sample_rows(N, seed=si)
        ref = oracle.mmvq_q4_k(w_qs[rows], w_hdr[rows], a_qs, a_d, a_s)
        mag = q4_k_mag(w_qs[rows], w_hdr[rows], a_qs, a_d, a_s)
        check_f32(y[:, rows], ref, mag, K, "q4_k packed full M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 4, 8])
def test_q6_k_packed_full_sizes_sampled(M):
    import skinny_gemm_amd as sk

    for si, (N, K) in enumerate([(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]):
        w_ql, w_qh, w_sc, w_d = inputs.q6_k_weights(N, K, inputs.seed(6, si, 0))
        x = inputs.normal_f32(M, K, inputs.seed(6, si, 2) + M)
        a_qs, a_d, _ = oracle.quantize_q8_1(x)
        wp = sk.prepack_q6_k(dev(w_ql), dev(w_qh), dev(w_sc), dev(w_d))
        y = host(sk.mmvq_q6_k_packed(wp, N, K, dev(a_qs), dev(a_d)))
        rows = sample_rows(N, seed=si)
        ref = oracle.mmvq_q6_k(w_ql[rows], w_qh[rows], w_sc[rows], w_d[rows], a_qs, a_d)
        mag = q6_k_mag(w_ql[rows], w_qh[rows], w_sc[rows], w_d[rows], a_qs, a_d)
        check_f32(y[:, rows], ref, mag, K, "q6_k packed full M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 4, 8])
def test_iq4_xs_full_sizes_sampled(M):
    # the Qwen3-8B projection shapes (K x N: 4096 x 6144, 4096 x 4096,
    # 4096 x 24576, 12288 x 4096), launched as the benchmark launches them
    for si, (N, K) in enumerate([(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]):
        w_qs, w_hdr = inputs.iq4_xs_weights(N, K, inputs.seed(7, si, 0))
        x = inputs.normal_f32(M, K, inputs.seed(7, si, 2) + M)
        a_qs, a_d, _ = oracle.quantize_q8_1(x)
        y = run_iq4_xs(w_qs, w_hdr, a_qs, a_d)
        rows = sample_rows(N, seed=si)
        ref = oracle.mmvq_iq4_xs(w_qs[rows], w_hdr[rows], a_qs, a_d)
        mag = iq4_xs_mag(w_qs[rows], w_hdr[rows], a_qs, a_d)
        check_f32(y[:, rows], ref, mag, K, "iq4_xs full M=%d %dx%d" % (M, N, K))
        y = run_iq4_xs_packed(w_qs, w_hdr, a_qs, a_d)
        check_f32(y[:, rows], ref, mag, K, "iq4_xs packed full M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 2])
def test_q4_0_f32act_full_sizes_sampled(M):
    for si, (N, K) in enumerate(LLAMA_Q4):
        w_qs, w_d = inputs.q4_0_weights(N, K, inputs.seed(1, si, 0))
        x = inputs.normal_f32(M, K, inputs.seed(2, si, 2) + M)
        y = run_q4_f32act(w_qs, w_d, x)
        rows = sample_rows(N, seed=si)
        a_qs, a_d, a_s = oracle.quantize_q8_1(x)
        ref = oracle.mmvq_q4_0(w_qs[rows], w_d[rows], a_qs, a_d, a_s)
        mag = q4_mag(w_qs[rows], w_d[rows], a_qs, a_d, a_s)
        check_f32(y[:, rows], ref, mag, K, "q4_0 f32act full M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_nvfp4_full_sizes_sampled(M):
    for si, (N, K) in enumerate(QWEN_FP):
        codes, scales, g = inputs.nvfp4_weights(N, K, inputs.seed(3, si, 0))
        x = inputs.normal_f16_bits(M, K, inputs.seed(3, si, 2) + M)
        y = run_nvfp4(codes, scales, g, x)
        rows = sample_rows(N, seed=si)
        y_acc, _ = oracle.gemv_nvfp4_w4a16(codes[rows], scales[rows], g, x)
        check_f16(y[:, rows], y_acc, nvfp4_mag(codes[rows], scales[rows], g, x), K,
                  "nvfp4 full M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_nvfp4_packed_full_sizes_sampled(M):
    import skinny_gemm_amd as sk

    for si, (N, K) in enumerate(QWEN_FP):
        codes, scales, g = inputs.nvfp4_weights(N, K, inputs.seed(3, si, 0))
        x = inputs.normal_f16_bits(M, K, inputs.seed(3, si, 2) + M)
        wp = sk.prepack_nvfp4(dev(codes), dev(scales))
        y = host(sk.gemv_nvfp4_w4a16_packed(wp, N, K, g, dev(x)), np.uint16)
        rows = sample_rows(N, seed=si)
        y_acc, _ = oracle.gemv_nvfp4_w4a16(codes[rows], scales[rows], g, x)
        check_f16(y[:, rows], y_acc, nvfp4_mag(codes[rows], scales[rows], g, x), K,
                  "nvfp4 packed full M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 4, 8, 16, 32, 96])
def test_fp8_packed_full_sizes_sampled(M):
    import skinny_gemm_amd as sk

    # the Qwen-shaped matrices, and a wide one with long rows (>= 1536 tiles,
    # K >= 8192: its own table row at M = 9..16)
    for si, (N, K) in enumerate(QWEN_FP + [(24576 + 16, 8192)]):
        w, cs = inputs.fp8_weights(N, K, inputs.seed(4, si, 0))
        x = inputs.normal_f16_bits(M, K, inputs.seed(4, si, 2) + M)
        wp = sk.prepack_fp8(dev(w))
        y = host(sk.gemv_fp8_w8a16_packed(wp, N, K, dev(cs), dev(x)), np.uint16)
        rows = sample_rows(N, seed=si)
        y_acc, _ = oracle.gemv_fp8_w8a16(w[rows], cs[rows], x)
        check_f16(y[:, rows], y_acc, fp8_mag(w[rows], cs[rows], x), K,
                  "fp8 packed full M=%d %dx%d" % (M, N, K))


@pytest.mark.parametrize("M", [1, 4, 8, 16, 32, 96])
def test_fp8_full_sizes_sampled(M):
    for si, (N, K) in enumerate(QWEN_FP):
        w, cs = inputs.fp8_weights(N, K, inputs.seed(4, si, 0))
        x = inputs.normal_f16_bits(M, K, inputs.seed(4, si, 2) + M)
        y = run_fp8(w, cs, x)
        rows = sample_rows(N, seed=si)
        y_acc, _ = oracle.gemv_fp8_w8a16(w[rows], cs[rows], x)
        check_f16(y[:, rows], y_acc, fp8_mag(w[rows], cs[rows], x), K,
                  "fp8 full M=%d %dx%d" % (M, N, K))


# ------------------------------------------------------------------ determinism, streams, limits

def test_repeat_runs_bit_identical_and_side_stream():
    import torch

    import skinny_gemm_amd as sk

    M, N, K = 8, 3000, 5120
    w_qs, w_d = inputs.q4_0_weights(N, K, 1)
    codes, scales, g = inputs.nvfp4_weights(N, K, 2)
    w8, cs = inputs.fp8_weights(N, K, 3)
    xf = inputs.normal_f32(M, K, 4)
    xh = inputs.normal_f16_bits(M, K, 5)
    args = [dev(a) for a in (w_qs, w_d, codes, scales, w8, cs, xf, xh)]

    def once(stream):
        qs, d, s = sk.quantize_act_q8_1(args[6], stream=stream)
        return (sk.mmvq_q4_0(args[0], args[1], qs, d, s, stream=stream),
                sk.gemv_nvfp4_w4a16(args[2], args[3], g, args[7], stream=stream),
                sk.gemv_fp8_w8a16(args[4], args[5], args[7], stream=stream))

    a = [host(t) for t in once(None)]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        b = once(side)
    side.synchronize()
    b = [host(t) for t in b]
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_concurrent_host_threads_on_their_own_streams():
    # four host threads call the library at once, each on its own stream and
    # at its own M (so through different kernel families); every thread's
    # results must equal the same calls made alone
    import threading

    import torch

    import skinny_gemm_amd as sk

    d = torch.device("cuda:0")
    N, K = 3000, 4096
    w_qs, w_d = inputs.q4_0_weights_torch(N, K, 31, d)
    codes, scales = inputs.nvfp4_weights_torch(N, K, 32, d)
    w8, cs = inputs.fp8_weights_torch(N, K, 33, d)
    xs = {M: (inputs.normal_f32_torch(M, K, 40 + M, d), inputs.normal_f16_torch(M, K, 50 + M, d))
          for M in (1, 2, 8, 16)}

    def work(M):
        xf, xh = xs[M]
        out = []
        if M <= 8:
            qs, dd, ss = sk.quantize_act_q8_1(xf)
            out.append(sk.mmvq_q4_0(w_qs, w_d, qs, dd, ss))
        out.append(sk.gemv_nvfp4_w4a16(codes, scales, 1.0, xh))
        out.append(sk.gemv_fp8_w8a16(w8, cs, xh))
        return out

    alone = {M: [host(t).view(np.uint8).copy() for t in work(M)] for M in xs}
    got, errors = {}, []

    def run(M):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                res = [work(M) for _ in range(5)]
            stream.synchronize()
            got[M] = [[t.cpu().numpy().view(np.uint8) for t in r] for r in res]
        except Exception as e:          # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=(M,)) for M in xs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for M in xs:
        for r in got[M]:
            for u, v in zip(r, alone[M]):
                assert np.array_equal(u, v), M


def test_graph_replays_match_eager():
    # every entry point, at M values that reach each kernel family, captured
    # in one HIP graph; each replay (with eager work and synchronizations in
    # between) must reproduce the eager bytes -- no memsets or host-side state
    # may hide in a captured launch
    import torch

    import skinny_gemm_amd as sk

    d = torch.device("cuda:0")
    N, K = 1000, 4096                        # K % 256 == 0: matrix-core paths too
    w_qs, w_d = inputs.q4_0_weights_torch(N, K, 21, d)
    k_qs, k_hdr = inputs.q4_k_weights_torch(N, K, 22, d)
    ql, qh, sc, dd = inputs.q6_k_weights_torch(N, K, 23, d)
    i_qs, i_hdr = inputs.iq4_xs_weights_torch(N, K, 28, d)
    bi_qs, bi_hdr = inputs.iq4_xs_weights_torch(16400, K, 29, d)   # IQ4_XS matrix cores (M = 8)
    codes, scales = inputs.nvfp4_weights_torch(N, K, 24, d)
    w8, cs = inputs.fp8_weights_torch(N, K, 25, d)
    fc, fs = inputs.nvfp4_weights_torch(8192, 5120, 26, d)   # the flat NVFP4 mapping (M = 1)
    fx = inputs.normal_f16_torch(1, 5120, 27, d)
    xf = {M: inputs.normal_f32_torch(M, K, 30 + M, d) for M in (1, 2, 8)}
    xh = {M: inputs.normal_f16_torch(M, K, 40 + M, d) for M in (1, 2, 4, 8, 32)}
    q8 = {M: sk.quantize_act_q8_1(xf[M]) for M in (1, 2, 8)}
    # pre-permuted copies (prepacked outside the graph, as at load time)
    p_q4, p_q4k = sk.prepack_q4_0(w_qs, w_d), sk.prepack_q4_k(k_qs, k_hdr)
    p_nv, p_f8 = sk.prepack_nvfp4(codes, scales), sk.prepack_fp8(w8)
    p_q6k = sk.prepack_q6_k(ql, qh, sc, dd)
    p_iq4 = sk.prepack_iq4_xs(i_qs, i_hdr)
    outs = []

    def run():
        outs.clear()
        for M in (1, 2, 8):
            sk.quantize_act_q8_1(xf[M], *q8[M])
            outs.append(sk.mmvq_q4_0(w_qs, w_d, *q8[M]))
            outs.append(sk.mmvq_q4_k(k_qs, k_hdr, *q8[M]))
            outs.append(sk.mmvq_q6_k(ql, qh, sc, dd, q8[M][0], q8[M][1]))
            outs.append(sk.mmvq_iq4_xs(i_qs, i_hdr, q8[M][0], q8[M][1]))
        outs.append(sk.mmvq_iq4_xs(bi_qs, bi_hdr, q8[8][0], q8[8][1]))
        for M in (1, 2):
            outs.append(sk.mmvq_q4_0_f32act(w_qs, w_d, xf[M]))
        for M in (1, 2, 4, 8):
            outs.append(sk.gemv_nvfp4_w4a16(codes, scales, 1.0, xh[M]))
        outs.append(sk.gemv_nvfp4_w4a16(fc, fs, 1.0, fx))
        for M in (1, 2, 4, 8, 32):
            outs.append(sk.gemv_fp8_w8a16(w8, cs, xh[M]))
        for M in (1, 2, 8):
            outs.append(sk.mmvq_q4_0_packed(p_q4, N, K, *q8[M]))
            outs.append(sk.mmvq_q4_k_packed(p_q4k, N, K, *q8[M]))
            outs.append(sk.mmvq_q6_k_packed(p_q6k, N, K, q8[M][0], q8[M][1]))
            outs.append(sk.mmvq_iq4_xs_packed(p_iq4, N, K, q8[M][0], q8[M][1]))
        for M in (1, 2, 4, 8):
            outs.append(sk.gemv_nvfp4_w4a16_packed(p_nv, N, K, 1.0, xh[M]))
        for M in (1, 2, 4, 8, 32):
            outs.append(sk.gemv_fp8_w8a16_packed(p_f8, N, K, cs, xh[M]))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                # warm every path before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    graph_outs = list(outs)
    torch.cuda.synchronize()
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    for _ in range(3):
        for o in graph_outs:
            o.view(torch.uint8).fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(graph_outs, ref)):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), i
        run()                                # eager work between replays
        torch.cuda.synchronize()


def test_largest_k_small_n():
    # K at the documented maximum, a handful of rows, ragged N
    M, N, K = 2, 5, 1 << 20
    w8, cs = inputs.fp8_weights(N, K, 8)
    x = inputs.normal_f16_bits(M, K, 9, std=0.1)
    y = run_fp8(w8, cs, x)
    y_acc, _ = oracle.gemv_fp8_w8a16(w8, cs, x)
    check_f16(y, y_acc, fp8_mag(w8, cs, x), K, "fp8 max K")
    w_qs, w_d = inputs.q4_0_weights(N, K, 10)
    xf = inputs.normal_f32(M, K, 11)
    a_qs, a_d, a_s = oracle.quantize_q8_1(xf)
    y = run_q4(w_qs, w_d, a_qs, a_d, a_s)
    ref = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    check_f32(y, ref, q4_mag(w_qs, w_d, a_qs, a_d, a_s), K, "q4_0 max K")


def test_largest_k_packed():
    # K at the documented maximum through every pre-permuted entry point:
    # long K slices, the last tile ragged (N = 17)
    import skinny_gemm_amd as sk

    N, K = 17, 1 << 20
    w_qs, w_d = inputs.q4_0_weights(N, K, 12)
    k_qs, k_hdr = inputs.q4_k_weights(N, K, 13)
    q6 = inputs.q6_k_weights(N, K, 18)
    for M in (1, 8):
        xf = inputs.normal_f32(M, K, 14 + M)
        a_qs, a_d, a_s = oracle.quantize_q8_1(xf)
        y = run_q4_packed(w_qs, w_d, a_qs, a_d, a_s)
        check_f32(y, oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s),
                  q4_mag(w_qs, w_d, a_qs, a_d, a_s), K, "q4_0 packed max K M=%d" % M)
        y = run_q4_k_packed(k_qs, k_hdr, a_qs, a_d, a_s)
        check_f32(y, oracle.mmvq_q4_k(k_qs, k_hdr, a_qs, a_d, a_s),
                  q4_k_mag(k_qs, k_hdr, a_qs, a_d, a_s), K, "q4_k packed max K M=%d" % M)
        y = run_q6_k_packed(*q6, a_qs, a_d)
        check_f32(y, oracle.mmvq_q6_k(*q6, a_qs, a_d), q6_k_mag(*q6, a_qs, a_d), K,
                  "q6_k packed max K M=%d" % M)
    codes, scales, g = inputs.nvfp4_weights(N, K, 15)
    w8, cs = inputs.fp8_weights(N, K, 16)
    for M in (1, 8, 16):
        x = inputs.normal_f16_bits(M, K, 17 + M, std=0.1)
        y = run_nvfp4_packed(codes, scales, g, x)
        y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, g, x)
        check_f16(y, y_acc, nvfp4_mag(codes, scales, g, x), K, "nvfp4 packed max K M=%d" % M)
        y = run_fp8_packed(w8, cs, x)
        y_acc, _ = oracle.gemv_fp8_w8a16(w8, cs, x)
        check_f16(y, y_acc, fp8_mag(w8, cs, x), K, "fp8 packed max K M=%d" % M)


def test_empty_and_invalid_calls_on_device():
    import torch

    import skinny_gemm_amd as sk

    z = torch.empty((0, 4096), dtype=torch.float16, device="cuda")
    w = torch.zeros((64, 4096), dtype=torch.uint8, device="cuda")
    cs = torch.ones(64, device="cuda")
    y = sk.gemv_fp8_w8a16(w, cs, z)
    assert tuple(y.shape) == (0, 64)
    x97 = torch.zeros((97, 4096), dtype=torch.float16, device="cuda")
    with pytest.raises(sk.SkinnyError) as e:
        sk.gemv_fp8_w8a16(w, cs, x97)
    assert e.value.status == -4
    # NVFP4 takes at most 16 rows
    codes = torch.zeros((64, 2048), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((64, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(sk.SkinnyError) as e:
        sk.gemv_nvfp4_w4a16(codes, scales, 1.0, x97[:17])
    assert e.value.status == -4
    # Q4_0 takes at most 8 rows
    qs, d, s = sk.quantize_act_q8_1(torch.zeros((9, 4096), device="cuda"))
    w_qs = torch.zeros((64, 2048), dtype=torch.uint8, device="cuda")
    w_d = torch.zeros((64, 128), dtype=torch.int16, device="cuda")
    with pytest.raises(sk.SkinnyError) as e:
        sk.mmvq_q4_0(w_qs, w_d, qs, d, s)
    assert e.value.status == -4
