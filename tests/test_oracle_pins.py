"""Pins for the CPU oracle: tie it to things other than itself.

Each check compares the oracle with a library routine (numpy binary16,
torch float8_e4m3fn), a hand-worked golden fixture under tests/golden/, a
closed form, an invariant, or an fp64 brute force written here
independently (dequantize the whole matrix, then one matmul).  A few
"sensitivity" checks show the brute force would notice the plausible
mistakes (swapped nibbles, a dropped -8 offset, a dropped group scale).

Runs on the CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden, read_table
from skinny_gemm_amd import inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------ independent decoders

def f16_bits_to_f64(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def e4m3_table_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e2m1_table_golden():
    t = np.zeros(16)
    for c, v in read_table("e2m1_values.txt"):
        t[int(c)] = float(v)
    return t


def unpack_q4_0(w_qs):
    """[N][K/2] bytes -> [N][K] codes; byte j of a block holds element j
    (low nibble) and element j+16 (high nibble)."""
    N, K2 = w_qs.shape
    b = w_qs.reshape(N, K2 // 16, 16)
    lo = b & 15
    hi = b >> 4
    return np.concatenate([lo, hi], axis=2).reshape(N, 2 * K2).astype(np.int64)


def unpack_nvfp4(codes):
    """[N][K/2] bytes -> [N][K] codes; element 2j low nibble, 2j+1 high."""
    N, K2 = codes.shape
    out = np.empty((N, 2 * K2), np.int64)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def brute_q4_0(w_qs, w_d, a_qs, a_d):
    """Dequantize both sides to fp64 and take one matmul: the plain
    definition, with the -8 applied to each weight and no sum term."""
    N = w_qs.shape[0]
    M, K = a_qs.shape
    W = (unpack_q4_0(w_qs) - 8).astype(np.float64) * np.repeat(f16_bits_to_f64(w_d), 32, axis=1)
    A = a_qs.astype(np.float64) * np.repeat(f16_bits_to_f64(a_d), 32, axis=1)
    return A @ W.T


def brute_nvfp4(codes, scales, g, x_bits):
    e2 = e2m1_table_golden()
    e4 = e4m3_table_torch()
    W = e2[unpack_nvfp4(codes)] * np.repeat(e4[scales], 16, axis=1) * float(g)
    return f16_bits_to_f64(x_bits) @ W.T


def brute_fp8(w, cs, x_bits):
    e4 = e4m3_table_torch()
    W = e4[w]
    return (f16_bits_to_f64(x_bits) @ W.T) * cs.astype(np.float64)[None, :]


# ------------------------------------------------------------ number formats

def test_f16_decode_all_codes_vs_numpy():
    ref = f16_bits_to_f64(np.arange(65536, dtype=np.uint16))
    got = np.array([oracle.f16_to_double(h) for h in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def _f16_encode_check(v32):
    v32 = np.asarray(v32, np.float32)
    want = v32.astype(np.float16).view(np.uint16)
    got = oracle.f16_from_double_array(v32.astype(np.float64))
    nan = np.isnan(v32)
    assert np.array_equal(want[~nan], got[~nan]), (
        v32[~nan][want[~nan] != got[~nan]][:10], want[~nan][want[~nan] != got[~nan]][:10],
        got[~nan][want[~nan] != got[~nan]][:10])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all(got[nan] & 0x3FF)


def test_f16_encode_random_vs_numpy():
    rng = np.random.Generator(np.random.PCG64(11))
    # random bit patterns cover every exponent, including huge and tiny ones
    bits = rng.integers(0, 2**32, size=1_500_000, dtype=np.uint64).astype(np.uint32)
    _f16_encode_check(bits.view(np.float32))
    # values concentrated inside the binary16 range
    _f16_encode_check((rng.standard_normal(1_000_000) * 10.0 ** rng.uniform(-8, 5, 1_000_000))
                      .astype(np.float32))


def test_f16_encode_midpoints_and_edges():
    # every midpoint between consecutive positive finite binary16 values is
    # exact in float32: ties must go to the even neighbour
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    _f16_encode_check(np.concatenate([mid, -mid]))
    # just around the midpoints
    _f16_encode_check(np.nextafter(mid, np.float32(np.inf)))
    _f16_encode_check(np.nextafter(mid, np.float32(0)))
    edges = np.array([65504, 65519.996, 65520, 65536, 1e9, np.inf, -65520, -np.inf,
                      2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26, 2.0 ** -14,
                      2.0 ** -14 - 2.0 ** -25, 0.0, -0.0, 1e-30, np.nan], np.float32)
    _f16_encode_check(edges)
    assert oracle.f16_from_double(65519.99) == 0x7BFF
    assert oracle.f16_from_double(65520.0) == 0x7C00
    assert oracle.f16_from_double(-0.0) == 0x8000
    assert oracle.f16_from_double(2.0 ** -25) == 0x0000      # tie to even (zero)
    assert oracle.f16_from_double(3 * 2.0 ** -25) == 0x0002  # tie to even (2)


def test_e4m3_decode_all_codes_vs_torch():
    ref = e4m3_table_torch()
    got = np.array([oracle.e4m3_to_double(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert np.nanmax(got) == 448.0 and np.nanmin(np.abs(got[got != 0])) == 2.0 ** -9


def test_e4m3_golden_points():
    for hx, v in read_table("e4m3_points.txt"):
        got = oracle.e4m3_to_double(int(hx, 16))
        if v == "nan":
            assert math.isnan(got), hx
        else:
            assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), hx


def test_e2m1_golden_all_codes():
    for c, v in read_table("e2m1_values.txt"):
        got = oracle.e2m1_to_double(int(c))
        assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), c
    # only the low nibble matters
    assert oracle.e2m1_to_double(0xF7) == 6.0


# ------------------------------------------------------------ Q8_1 quantization

def test_q8_1_golden_blocks():
    for rec in read_golden("q8_1_blocks.txt"):
        xv = [float(v) for v in rec["x"]]
        qv = [int(v) for v in rec["q"]]
        x = np.zeros((1, 32), np.float32)
        x[0, :len(xv)] = xv
        want_q = np.zeros(32, np.int8)
        want_q[:len(qv)] = qv
        qs, d, s = oracle.quantize_q8_1(x)
        assert np.array_equal(qs[0], want_q), rec["block"]
        assert d[0, 0] == int(rec["d"][0], 16), rec["block"]
        assert s[0, 0] == int(rec["s"][0], 16), rec["block"]


def _check_q8_1_properties(x, qs, d, s):
    """Invariants of any correct Q8_1 encoder under our reading, checked
    with numpy's own float32 division and binary16 conversion."""
    M, K = x.shape
    xb = x.reshape(M, K // 32, 32)
    qb = qs.reshape(M, K // 32, 32).astype(np.int64)
    amax = np.abs(xb).max(axis=2)
    d32 = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    zero = amax == 0
    # scale: binary16 of the binary32 scale
    assert np.array_equal(d, d32.astype(np.float16).view(np.uint16))
    # zero blocks are all zero
    assert np.all(qb[zero] == 0) and np.all(s[zero] == 0) and np.all(d[zero] == 0)
    nz = ~zero
    # codes: the integer nearest to the float32 quotient, ties away from zero
    quo = (xb[nz] / d32[nz][:, None]).astype(np.float32).astype(np.float64)
    q = qb[nz]
    assert np.all(np.abs(q) <= 127)
    assert np.all(np.abs(quo - q) <= 0.5)
    tie = np.abs(np.abs(quo - q) - 0.5) == 0
    assert np.all(np.abs(q[tie]) > np.abs(quo[tie]))
    # the largest entry of a block maps to +-127
    assert np.all(np.abs(q).max(axis=1) == 127)
    # round trip: |x - q d| <= d/2 (plus float32 rounding of the quotient)
    err = np.abs(xb[nz].astype(np.float64) - q * d32[nz][:, None].astype(np.float64))
    assert np.all(err <= 0.5 * d32[nz][:, None] * (1 + 2.0 ** -20))
    # sum term: binary16 of float32(d32 * sum q)
    sq = qb.sum(axis=2)
    want_s = (d32 * sq.astype(np.float32)).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(s[nz], want_s[nz])


def test_q8_1_random_rows_properties():
    x = inputs.normal_f32(5, 1024, 7)
    x[1] *= 1e-3
    x[2] *= 1e3
    x[3, :32] = 0.0                 # all-zero block
    x[3, 32:64] = 0.0
    x[3, 40] = -2.0                 # single non-zero element
    x[4, :32] *= 1e-7               # binary16 scale goes subnormal
    x[4, 32:64] = 2.5e3             # s overflows binary16 to +inf
    qs, d, s = oracle.quantize_q8_1(x)
    _check_q8_1_properties(x, qs, d, s)
    assert np.all(qs[3, 32:64][np.arange(32) != 8] == 0) and qs[3, 40] == -127
    assert d[4, 0] < 0x0400         # subnormal binary16
    assert s[4, 1] == 0x7C00


def test_q8_1_halfway_adversarial():
    # integer rows with one +-127 per block: scale is exactly 1, x/d = x
    x = inputs.q8_1_unit_scale_source(3, 256, 5)
    x[0, 1:32:2] = x[0, 1:32:2] + 0.5
    x[0, 0] = 127.0
    x[1, 0] = -127.0
    x[1, 1:9] = [-2.5, 2.5, -0.5, 0.5, 1.5, -1.5, 125.5, -125.5]
    qs, d, s = oracle.quantize_q8_1(x)
    _check_q8_1_properties(x, qs, d, s)
    assert qs[1, 1:9].tolist() == [-3, 3, -1, 1, 2, -2, 126, -126]


def test_q8_1_unit_scale_source():
    x = inputs.q8_1_unit_scale_source(4, 512, 9)
    qs, d, s = oracle.quantize_q8_1(x)
    assert np.all(d == 0x3C00)
    assert np.array_equal(qs.astype(np.float32), x)
    sq = qs.reshape(4, 16, 32).astype(np.int64).sum(axis=2)
    assert np.array_equal(f16_bits_to_f64(s), sq.astype(np.float64))


# ------------------------------------------------------------ Q4_0 x Q8_1

def test_q4_0_golden_block():
    rec = read_golden("q4_0_block.txt")[0]
    w_qs = np.array([[int(v, 16) for v in rec["w_qs"]]], np.uint8)
    a_qs = np.array([[int(v) for v in rec["a_qs"]]], np.int8)
    assert w_qs.shape == (1, 16) and a_qs.shape == (1, 32)
    isum = oracle.q4_0_blocksums(w_qs, a_qs)
    assert isum[0, 0, 0] == int(rec["isum"][0])
    assert isum[0, 0, 0] - 8 * int(a_qs.astype(np.int64).sum()) == int(rec["offset_identity"][0])
    w_d = np.array([[int(rec["w_d"][0], 16)]], np.uint16)
    a_d = np.array([[int(rec["a_d"][0], 16)]], np.uint16)
    a_s = np.array([[int(rec["a_s"][0], 16)]], np.uint16)
    y = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    assert y[0, 0] == float(rec["y"][0])


def test_q4_0_integer_offset_identity():
    # sum_i (q4 - 8) q8 == isum - 8 * sum_i q8, exact, per block
    rng = np.random.Generator(np.random.PCG64(3))
    w_qs = rng.integers(0, 256, (23, 96), dtype=np.uint8)
    a_qs = rng.integers(-127, 128, (3, 192), dtype=np.int8)
    isum = oracle.q4_0_blocksums(w_qs, a_qs).astype(np.int64)       # [M][N][nb]
    codes = unpack_q4_0(w_qs).reshape(23, 6, 32)
    a = a_qs.astype(np.int64).reshape(3, 6, 32)
    raw = np.einsum("nbi,mbi->mnb", codes, a)
    assert np.array_equal(isum, raw)
    centred = np.einsum("nbi,mbi->mnb", codes - 8, a)
    assert np.array_equal(isum - 8 * a.sum(axis=2)[:, None, :], centred)


@pytest.mark.parametrize("M,N,K", [(1, 7, 32), (4, 37, 256), (8, 64, 1024), (3, 5, 11008 // 8)])
def test_q4_0_vs_fp64_bruteforce(M, N, K):
    w_qs, w_d = inputs.q4_0_weights(N, K, 100 + K)
    x = inputs.normal_f32(M, K, 200 + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    y = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    y_bf = brute_q4_0(w_qs, w_d, a_qs, a_d)
    # closed-form bound: binary16 rounding of the sum term, times 8 d4, plus
    # binary64 summation error
    nb = K // 32
    d4 = f16_bits_to_f64(w_d)                                   # [N][nb]
    d8 = f16_bits_to_f64(a_d)                                   # [M][nb]
    s8 = f16_bits_to_f64(a_s)
    sq = a_qs.astype(np.int64).reshape(M, nb, 32).sum(axis=2)
    sround = np.abs(s8 - d8 * sq)                               # [M][nb]
    bound = 8.0 * sround @ np.abs(d4).T
    mag = (np.abs(a_qs.astype(np.float64)) * np.repeat(d8, 32, axis=1)) @ \
        (np.abs(unpack_q4_0(w_qs) - 8) * np.repeat(d4, 32, axis=1)).T
    bound += (nb + 3) * 2.0 ** -52 * (mag + 8 * np.abs(s8) @ np.abs(d4).T)
    assert np.all(np.abs(y - y_bf) <= bound + 1e-300)
    # and the bound is small beside the magnitude of the terms it bounds
    assert np.max(bound / mag) < 1e-3


def test_q4_0_unit_scale_exact():
    M, N, K = 4, 19, 4096
    x = inputs.q8_1_unit_scale_source(M, K, 31)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    w_qs, _ = inputs.q4_0_weights(N, K, 32)
    w_d = np.full((N, K // 32), 0x3C00, np.uint16)
    y = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    exact = a_qs.astype(np.int64) @ (unpack_q4_0(w_qs) - 8).T
    assert np.array_equal(y, exact.astype(np.float64))
    # all codes 8 -> every weight is zero
    w8 = np.full((N, K // 2), 0x88, np.uint8)
    assert np.all(oracle.mmvq_q4_0(w8, w_d, a_qs, a_d, a_s) == 0.0)


def test_q4_0_bruteforce_is_sensitive():
    # the brute force tells apart the plausible mistakes
    M, N, K = 2, 9, 256
    w_qs, w_d = inputs.q4_0_weights(N, K, 5)
    x = inputs.normal_f32(M, K, 6)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    y = oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s)
    swapped = ((w_qs & 15) << 4) | (w_qs >> 4)
    assert np.max(np.abs(brute_q4_0(swapped, w_d, a_qs, a_d) - y)) > 1e-2 * np.max(np.abs(y))
    no_offset = a_qs.astype(np.float64) * np.repeat(f16_bits_to_f64(a_d), 32, axis=1) @ \
        (unpack_q4_0(w_qs) * np.repeat(f16_bits_to_f64(w_d), 32, axis=1)).T
    assert np.max(np.abs(no_offset - y)) > 1e-2 * np.max(np.abs(y))


# ------------------------------------------------------------ K-quants x Q8_1

def q4_k_fields(hdr):
    """hdr [N][ns][16] -> d, dmin [N][ns] float64; sc, m [N][ns*8] int."""
    N, ns, _ = hdr.shape
    d = f16_bits_to_f64(hdr[:, :, 0:2].copy().view(np.uint16)[:, :, 0])
    dmin = f16_bits_to_f64(hdr[:, :, 2:4].copy().view(np.uint16)[:, :, 0])
    p = hdr[:, :, 4:16].astype(np.int64)
    sc = p[:, :, 0:8] & 63
    hi = np.stack([(p[:, :, 8 + j // 2] >> (4 * (j % 2))) & 15 for j in range(8)], axis=2)
    m = (p[:, :, 0:8] >> 6) | (hi << 2)
    return d, dmin, sc.reshape(N, ns * 8), m.reshape(N, ns * 8)


def brute_q4_k(w_qs, w_hdr, a_qs, a_d):
    """Dequantize (d sc q - dmin m per weight) and the Q8_1 codes to fp64,
    then one matmul: no sum term."""
    d, dmin, sc, m = q4_k_fields(w_hdr)
    W = unpack_q4_0(w_qs).astype(np.float64) * np.repeat(np.repeat(d, 8, axis=1) * sc, 32, axis=1) \
        - np.repeat(np.repeat(dmin, 8, axis=1) * m, 32, axis=1)
    A = a_qs.astype(np.float64) * np.repeat(f16_bits_to_f64(a_d), 32, axis=1)
    return A @ W.T


def unpack_q6_k(w_ql, w_qh):
    """-> [N][K] codes 0..63 (low nibbles in Q4_0 order, high bits from qh)."""
    N, K2 = w_ql.shape
    K = 2 * K2
    lo = unpack_q4_0(w_ql)
    qh = w_qh.reshape(N, K // 32, 2, 4).astype(np.int64)          # [n][b][h][t]
    hi = np.empty((N, K // 32, 2, 4, 4), np.int64)                 # [n][b][h][c][t]
    for c in range(4):
        hi[:, :, :, c, :] = (qh >> (2 * c)) & 3
    return lo | (hi.reshape(N, K) << 4)


def brute_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d):
    q = unpack_q6_k(w_ql, w_qh)
    scale = np.repeat(w_sc.astype(np.float64), 16, axis=1) * np.repeat(f16_bits_to_f64(w_d), 256, axis=1)
    W = (q - 32).astype(np.float64) * scale
    A = a_qs.astype(np.float64) * np.repeat(f16_bits_to_f64(a_d), 32, axis=1)
    return A @ W.T


def test_q4_k_golden_superblock():
    rec = read_golden("q4_k_superblock.txt")[0]
    hdr = np.zeros((1, 1, 16), np.uint8)
    hdr[0, 0, 0:2] = np.array([int(rec["d"][0], 16)], np.uint16).view(np.uint8)
    hdr[0, 0, 2:4] = np.array([int(rec["dmin"][0], 16)], np.uint16).view(np.uint8)
    hdr[0, 0, 4:16] = [int(v, 16) for v in rec["p"]]
    w_qs = np.repeat(np.array([int(v, 16) for v in rec["block_byte"]], np.uint8), 16)[None, :]
    halves = [int(v) for v in rec["a_half_values"]]
    a_qs = np.repeat(np.array(halves, np.int8), 16)[None, :]
    a_d = np.array([[int(v, 16) for v in rec["a_d"]]], np.uint16)
    a_s = np.array([[int(v, 16) for v in rec["a_s"]]], np.uint16)
    y = oracle.mmvq_q4_k(w_qs, hdr, a_qs, a_d, a_s)
    assert y[0, 0] == float(rec["y"][0])


def test_q6_k_golden_superblock():
    rec = read_golden("q6_k_superblock.txt")[0]
    K = 256
    w_ql = np.zeros((1, K // 2), np.uint8)
    w_ql[0, :16] = [int(v, 16) for v in rec["ql0"]]
    w_qh = np.zeros((1, K // 4), np.uint8)
    w_qh[0, :8] = [int(v, 16) for v in rec["qh0"]]
    w_sc = np.array([[int(v) for v in rec["sc"]]], np.int8)
    w_d = np.array([[int(rec["d"][0], 16)]], np.uint16)
    a_qs = np.ones((1, K), np.int8)
    sp = [int(v) for v in rec["a_special"]]
    for i in range(0, len(sp), 2):
        a_qs[0, sp[i]] = sp[i + 1]
    a_d = np.full((1, K // 32), int(rec["a_d"][0], 16), np.uint16)
    y = oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    assert y[0, 0] == float(rec["y"][0])
    # and the fixture's code table agrees with an independent unpacking
    q = unpack_q6_k(w_ql, w_qh)[0, :32]
    assert list(q[[0, 4, 5, 12, 16, 20, 21, 28]]) == [40, 40, 63, 0, 33, 16, 33, 33]


def test_q4_k_reduces_to_q4_0():
    # sc_j = 1, m_j = 8, d = dmin = d0: weight = d0 (q - 8), i.e. Q4_0 with d0
    # in every block of the super-block
    M, N, K = 3, 21, 1024
    w_qs, _ = inputs.q4_0_weights(N, K, 41)
    d0 = inputs.q4_0_weights(N, K // 8, 42)[1][:, : K // 256]       # binary16 bits [N][ns]
    hdr = np.zeros((N, K // 256, 16), np.uint8)
    hdr[:, :, 0:2] = d0.view(np.uint8).reshape(N, K // 256, 2)
    hdr[:, :, 2:4] = hdr[:, :, 0:2]
    hdr[:, :, 4:12] = 0x01                       # sc 1, low bits of m = 8 & 3 = 0
    hdr[:, :, 12:16] = 0x22                      # high bits of m = 8 >> 2 = 2
    x = inputs.normal_f32(M, K, 43)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    y_k = oracle.mmvq_q4_k(w_qs, hdr, a_qs, a_d, a_s)
    y_0 = oracle.mmvq_q4_0(w_qs, np.repeat(d0, 8, axis=1), a_qs, a_d, a_s)
    assert np.allclose(y_k, y_0, rtol=1e-12, atol=1e-12 * np.abs(y_0).max())


@pytest.mark.parametrize("M,N,K", [(1, 7, 256), (4, 37, 1024), (8, 16, 4096)])
def test_q4_k_vs_fp64_bruteforce(M, N, K):
    w_qs, w_hdr = inputs.q4_k_weights(N, K, 300 + K)
    x = inputs.normal_f32(M, K, 400 + K)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    y = oracle.mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s)
    y_bf = brute_q4_k(w_qs, w_hdr, a_qs, a_d)
    # bound: binary16 rounding of s8 times dmin m per block, plus fp64 sums
    nb = K // 32
    d, dmin, sc, m = q4_k_fields(w_hdr)
    dm = np.repeat(dmin, 8, axis=1) * m                          # [N][nb]
    d8 = f16_bits_to_f64(a_d)
    s8 = f16_bits_to_f64(a_s)
    sq = a_qs.astype(np.int64).reshape(M, nb, 32).sum(axis=2)
    bound = np.abs(s8 - d8 * sq) @ np.abs(dm).T
    mag = (np.abs(a_qs.astype(np.float64)) * np.repeat(d8, 32, axis=1)) @ np.abs(
        unpack_q4_0(w_qs) * np.repeat(np.repeat(d, 8, axis=1) * sc, 32, axis=1)
        - np.repeat(dm, 32, axis=1)).T
    bound += (nb + 3) * 2.0 ** -52 * (mag + np.abs(s8) @ np.abs(dm).T)
    assert np.all(np.abs(y - y_bf) <= bound + 1e-300)
    assert np.max(bound / mag) < 1e-3


@pytest.mark.parametrize("M,N,K", [(1, 7, 256), (4, 37, 1024), (8, 16, 4096)])
def test_q6_k_vs_fp64_bruteforce(M, N, K):
    w_ql, w_qh, w_sc, w_d = inputs.q6_k_weights(N, K, 500 + K)
    x = inputs.normal_f32(M, K, 600 + K)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    y = oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    y_bf = brute_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    q = unpack_q6_k(w_ql, w_qh)
    scale = np.repeat(np.abs(w_sc.astype(np.float64)), 16, axis=1) * np.repeat(f16_bits_to_f64(w_d), 256, axis=1)
    mag = (np.abs(a_qs.astype(np.float64)) * np.repeat(f16_bits_to_f64(a_d), 32, axis=1)) @ \
        (np.abs(q - 32) * scale).T
    # the block brackets are exact integers: only binary64 rounding remains
    assert np.all(np.abs(y - y_bf) <= (K // 32 + 3) * 2.0 ** -52 * mag + 1e-300)


def test_q6_k_unit_scale_exact():
    # d = 1, sc = 1, integer activations with d8 = 1: y = sum (q - 32) q8 exactly
    M, N, K = 3, 11, 2048
    x = inputs.q8_1_unit_scale_source(M, K, 51)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    w_ql, w_qh, _, _ = inputs.q6_k_weights(N, K, 52)
    w_sc = np.ones((N, K // 16), np.int8)
    w_d = np.full((N, K // 256), 0x3C00, np.uint16)
    y = oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    exact = a_qs.astype(np.int64) @ (unpack_q6_k(w_ql, w_qh) - 32).T
    assert np.array_equal(y, exact.astype(np.float64))


def test_k_quant_bruteforce_is_sensitive():
    M, N, K = 2, 9, 512
    x = inputs.normal_f32(M, K, 61)
    a_qs, a_d, a_s = oracle.quantize_q8_1(x)
    w_qs, w_hdr = inputs.q4_k_weights(N, K, 62)
    y = oracle.mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s)
    tol = 1e-2 * np.max(np.abs(y))
    # swapping the scale and min fields, or dropping the min, is noticed
    swapped = w_hdr.copy()
    swapped[:, :, 4:8], swapped[:, :, 8:12] = w_hdr[:, :, 8:12], w_hdr[:, :, 4:8]
    assert np.max(np.abs(brute_q4_k(w_qs, swapped, a_qs, a_d) - y)) > tol
    no_min = w_hdr.copy()
    no_min[:, :, 2:4] = 0
    assert np.max(np.abs(brute_q4_k(w_qs, no_min, a_qs, a_d) - y)) > tol
    # Q6_K: a wrong high-bit position or a dropped -32 is noticed
    w_ql, w_qh, w_sc, w_d = inputs.q6_k_weights(N, K, 63)
    y6 = oracle.mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d)
    tol6 = 1e-2 * np.max(np.abs(y6))
    rolled = np.roll(w_qh.reshape(N, -1, 8), 1, axis=2).reshape(N, -1)
    assert np.max(np.abs(brute_q6_k(w_ql, rolled, w_sc, w_d, a_qs, a_d) - y6)) > tol6
    q = unpack_q6_k(w_ql, w_qh)
    scale = np.repeat(w_sc.astype(np.float64), 16, axis=1) * np.repeat(f16_bits_to_f64(w_d), 256, axis=1)
    no_offset = (a_qs.astype(np.float64) * np.repeat(f16_bits_to_f64(a_d), 32, axis=1)) @ (q * scale).T
    assert np.max(np.abs(no_offset - y6)) > tol6


# ------------------------------------------------------------ NVFP4 W4A16

# ------------------------------------------------------------ IQ4_XS x Q8_1

def iq4_table():
    """The 16-entry IQ4_NL table from its fixture (not from the oracle)."""
    return np.array([int(v) for v in read_golden("iq4_nl_table.txt")[0]["table"]], np.int64)


def iq4_xs_scales(hdr):
    """hdr [N][ns][8] -> d [N][ns] float64, ls [N][ns*8] int (0..63)."""
    N, ns, _ = hdr.shape
    d = f16_bits_to_f64(hdr[:, :, 0:2].copy().view(np.uint16)[:, :, 0])
    H = hdr[:, :, 2].astype(np.int64) | (hdr[:, :, 3].astype(np.int64) << 8)
    L = hdr[:, :, 4:8].astype(np.int64)
    ls = np.stack([((L[:, :, j // 2] >> (4 * (j % 2))) & 15) | (((H >> (2 * j)) & 3) << 4)
                   for j in range(8)], axis=2)
    return d, ls.reshape(N, ns * 8)


def iq4_xs_header(d_bits, ls):
    """Encode binary16 d [N][ns] and 6-bit scales ls [N][ns][8] into the
    8-byte headers [N][ns][8]."""
    N, ns = d_bits.shape
    hdr = np.zeros((N, ns, 8), np.uint8)
    hdr[:, :, 0:2] = d_bits.astype(np.uint16).view(np.uint8).reshape(N, ns, 2)
    H = np.zeros((N, ns), np.int64)
    for j in range(8):
        H |= (ls[:, :, j].astype(np.int64) >> 4) << (2 * j)
        hdr[:, :, 4 + j // 2] |= ((ls[:, :, j] & 15) << (4 * (j % 2))).astype(np.uint8)
    hdr[:, :, 2] = (H & 255).astype(np.uint8)
    hdr[:, :, 3] = (H >> 8).astype(np.uint8)
    return hdr


def brute_iq4_xs(w_qs, w_hdr, a_qs, a_d, table=None):
    """Dequantize (d (ls - 32) T[q] per weight) and the Q8_1 codes to fp64,
    then one matmul."""
    T = iq4_table() if table is None else table
    d, ls = iq4_xs_scales(w_hdr)
    W = T[unpack_q4_0(w_qs)].astype(np.float64) * np.repeat(np.repeat(d, 8, axis=1) * (ls - 32), 32, axis=1)
    A = a_qs.astype(np.float64) * np.repeat(f16_bits_to_f64(a_d), 32, axis=1)
    return A @ W.T


def test_iq4_xs_golden_superblock():
    rec = read_golden("iq4_xs_superblock.txt")[0]
    K = 256
    hdr = np.array([int(v, 16) for v in rec["hdr"]], np.uint8).reshape(1, 1, 8)
    w_qs = np.zeros((1, K // 2), np.uint8)
    w_qs[0, 0:16] = [int(v, 16) for v in rec["qs0"]]
    w_qs[0, 16:32] = [int(v, 16) for v in rec["qs1"]]
    a_qs = np.ones((1, K), np.int8)
    for blk, key in ((0, "a0_special"), (1, "a1_special")):
        sp = [int(v) for v in rec[key]]
        for i in range(0, len(sp), 2):
            a_qs[0, 32 * blk + sp[i]] = sp[i + 1]
    a_d = np.full((1, K // 32), int(rec["a_d"][0], 16), np.uint16)
    y = oracle.mmvq_iq4_xs(w_qs, hdr, a_qs, a_d)
    assert y[0, 0] == float(rec["y"][0])
    # the fixture's block sums agree with an independent unpacking
    q = iq4_table()[unpack_q4_0(w_qs)[0]]
    isum = [int(np.dot(q[32 * b:32 * b + 32], a_qs[0, 32 * b:32 * b + 32].astype(np.int64)))
            for b in range(2)]
    assert isum == [int(v) for v in rec["isum"]]
    d, ls = iq4_xs_scales(hdr)
    assert d[0, 0] == 0.5 and list(ls[0]) == [35, 30, 32, 32, 32, 32, 32, 32]


def test_iq4_xs_unit_vectors_recover_table_and_scales():
    # row n holds index n everywhere, d = 1; sub-block j has scale ls_j - 32;
    # activation row m is one code 1 (d8 = 1) in sub-block j(m), so
    # y[m][n] = T[n] * (ls_j(m) - 32)
    N, K = 16, 512
    ls = np.array([0, 63, 17, 46, 32, 5, 50, 31, 33, 47, 16, 1, 62, 40, 24, 9])
    w_qs = np.repeat((np.arange(16, dtype=np.uint8) * 17)[:, None], K // 2, axis=1)
    hdr = iq4_xs_header(np.full((N, 2), 0x3C00), np.tile(ls.reshape(1, 2, 8), (N, 1, 1)))
    pos = [0, 37, 70, 127, 129, 191, 200, 255, 256, 300, 330, 383, 400, 450, 480, 511]
    M = len(pos)
    a_qs = np.zeros((M, K), np.int8)
    a_qs[np.arange(M), pos] = 1
    a_d = np.full((M, K // 32), 0x3C00, np.uint16)
    y = oracle.mmvq_iq4_xs(w_qs, hdr, a_qs, a_d)
    T = iq4_table()
    expect = np.array([[T[n] * (ls[p // 32] - 32) for n in range(N)] for p in pos], np.float64)
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("M,N,K", [(1, 7, 256), (4, 37, 1024), (8, 16, 4096)])
def test_iq4_xs_vs_fp64_bruteforce(M, N, K):
    w_qs, w_hdr = inputs.iq4_xs_weights(N, K, 700 + K)
    x = inputs.normal_f32(M, K, 800 + K)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    y = oracle.mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d)
    y_bf = brute_iq4_xs(w_qs, w_hdr, a_qs, a_d)
    d, ls = iq4_xs_scales(w_hdr)
    W = np.abs(iq4_table()[unpack_q4_0(w_qs)] * np.repeat(np.repeat(d, 8, axis=1) * (ls - 32), 32, axis=1))
    mag = (np.abs(a_qs.astype(np.float64)) * np.repeat(f16_bits_to_f64(a_d), 32, axis=1)) @ W.T
    # block sums are exact integers: only binary64 rounding remains
    assert np.all(np.abs(y - y_bf) <= (K // 32 + 3) * 2.0 ** -52 * mag + 1e-300)


def test_iq4_xs_unit_scale_exact():
    # d = 1, ls = 33 (scale 1), integer activations with d8 = 1:
    # y = sum T[q] q8 exactly
    M, N, K = 3, 11, 2048
    x = inputs.q8_1_unit_scale_source(M, K, 71)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    w_qs, _ = inputs.iq4_xs_weights(N, K, 72)
    hdr = iq4_xs_header(np.full((N, K // 256), 0x3C00), np.full((N, K // 256, 8), 33))
    y = oracle.mmvq_iq4_xs(w_qs, hdr, a_qs, a_d)
    exact = a_qs.astype(np.int64) @ iq4_table()[unpack_q4_0(w_qs)].T
    assert np.array_equal(y, exact.astype(np.float64))


def test_iq4_xs_bruteforce_is_sensitive():
    M, N, K = 2, 9, 512
    x = inputs.normal_f32(M, K, 81)
    a_qs, a_d, _ = oracle.quantize_q8_1(x)
    w_qs, w_hdr = inputs.iq4_xs_weights(N, K, 82)
    y = oracle.mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d)
    tol = 1e-2 * np.max(np.abs(y))
    # swapped nibbles, a dropped -32, high scale bits read from the other
    # header byte, or the table read backwards are all noticed
    swapped = ((w_qs >> 4) | (w_qs << 4)).astype(np.uint8)
    assert np.max(np.abs(brute_iq4_xs(swapped, w_hdr, a_qs, a_d) - y)) > tol
    d, ls = iq4_xs_scales(w_hdr)
    no_offset = iq4_xs_header(w_hdr[:, :, 0:2].copy().view(np.uint16)[:, :, 0],
                              (ls.reshape(N, -1, 8) + 32) % 64)
    assert np.max(np.abs(brute_iq4_xs(w_qs, no_offset, a_qs, a_d) - y)) > tol
    hswap = w_hdr.copy()
    hswap[:, :, 2], hswap[:, :, 3] = w_hdr[:, :, 3], w_hdr[:, :, 2]
    assert np.max(np.abs(brute_iq4_xs(w_qs, hswap, a_qs, a_d) - y)) > tol
    assert np.max(np.abs(brute_iq4_xs(w_qs, w_hdr, a_qs, a_d, iq4_table()[::-1]) - y)) > tol


def test_nvfp4_golden_row():
    rec = read_golden("nvfp4_row.txt")[0]
    codes = np.array([[int(v, 16) for v in rec["codes"]]], np.uint8)
    scales = np.array([[int(v, 16) for v in rec["scales"]]], np.uint8)
    xv = np.array([[float(v) for v in rec["x"]]], np.float64)
    assert codes.shape == (1, 16) and xv.shape == (1, 32)
    x = xv.astype(np.float16).view(np.uint16)
    y_acc, y = oracle.gemv_nvfp4_w4a16(codes, scales, float(rec["g"][0]), x)
    assert y_acc[0, 0] == float(rec["y"][0])
    assert y[0, 0] == int(rec["y_bits"][0], 16)


@pytest.mark.parametrize("M,N,K,g", [(1, 5, 16, 1.0), (4, 33, 512, 1.0), (8, 17, 5120 // 4, 0.375),
                                     (3, 8, 64, 2.0 ** -3)])
def test_nvfp4_vs_fp64_bruteforce(M, N, K, g):
    codes, scales, _ = inputs.nvfp4_weights(N, K, 300 + K)
    x = inputs.normal_f16_bits(M, K, 301 + K)
    y_acc, y = oracle.gemv_nvfp4_w4a16(codes, scales, g, x)
    y_bf = brute_nvfp4(codes, scales, g, x)
    e2 = e2m1_table_golden()
    e4 = e4m3_table_torch()
    Wabs = np.abs(e2[unpack_nvfp4(codes)] * np.repeat(e4[scales], 16, axis=1) * g)
    mag = np.abs(f16_bits_to_f64(x)) @ Wabs.T
    assert np.all(np.abs(y_acc - y_bf) <= (K + 2) * 2.0 ** -52 * mag)
    assert np.array_equal(y, oracle.f16_from_double_array(y_acc).reshape(y.shape))


def test_nvfp4_unit_scales_exact_and_global_scale():
    M, N, K = 2, 6, 256
    codes, _, _ = inputs.nvfp4_weights(N, K, 41)
    ones = np.full((N, K // 16), 0x38, np.uint8)
    rng = np.random.Generator(np.random.PCG64(42))
    xi = rng.integers(-8, 9, (M, K)).astype(np.float16)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, ones, 1.0, xi.view(np.uint16))
    e2 = e2m1_table_golden()
    exact = xi.astype(np.float64) @ e2[unpack_nvfp4(codes)].T
    assert np.array_equal(y_acc, exact)
    # a power-of-two global scale scales the result exactly
    y4, _ = oracle.gemv_nvfp4_w4a16(codes, ones, 4.0, xi.view(np.uint16))
    assert np.array_equal(y4, 4.0 * exact)


def test_nvfp4_outliers_stay_finite():
    # binary16 activations with +-2e4 entries: any binary16 partial sum would
    # overflow; the wide accumulator must not
    M, N, K = 2, 8, 256
    codes = np.full((N, K // 2), 0x77, np.uint8)            # every weight 6.0
    scales = np.full((N, K // 16), 0x7E, np.uint8)          # group scale 448
    x = np.full((M, K), 2.0e4, np.float64)
    x[:, 1::2] = -2.0e4
    x[0, 0] = 2.0e4 + 16.0
    xb = x.astype(np.float16).view(np.uint16)
    y_acc, y = oracle.gemv_nvfp4_w4a16(codes, scales, 1.0, xb)
    want = brute_nvfp4(codes, scales, 1.0, xb)
    assert np.all(np.isfinite(y_acc)) and np.array_equal(y_acc, want)
    assert y_acc[0, 0] == 16.0 * 6.0 * 448.0


def test_nvfp4_bruteforce_is_sensitive():
    M, N, K = 2, 9, 256
    codes, scales, _ = inputs.nvfp4_weights(N, K, 7)
    x = inputs.normal_f16_bits(M, K, 8)
    y_acc, _ = oracle.gemv_nvfp4_w4a16(codes, scales, 1.0, x)
    swapped = ((codes & 15) << 4) | (codes >> 4)
    assert np.max(np.abs(brute_nvfp4(swapped, scales, 1.0, x) - y_acc)) > 1e-2 * np.max(np.abs(y_acc))
    e2 = e2m1_table_golden()
    no_scale = f16_bits_to_f64(x) @ e2[unpack_nvfp4(codes)].T
    assert np.max(np.abs(no_scale - y_acc)) > 1e-2 * np.max(np.abs(y_acc))


# ------------------------------------------------------------ FP8 W8A16

def test_fp8_golden_row():
    rec = read_golden("fp8_row.txt")[0]
    w = np.array([[int(v, 16) for v in rec["w"]]], np.uint8)
    x = np.array([[float(v) for v in rec["x"]]]).astype(np.float16).view(np.uint16)
    cs = np.array([float(rec["cs"][0])], np.float32)
    y_acc, y = oracle.gemv_fp8_w8a16(w, cs, x)
    assert y_acc[0, 0] == float(rec["y"][0]) and y[0, 0] == int(rec["y_bits"][0], 16)


@pytest.mark.parametrize("M,N,K", [(1, 3, 16), (4, 29, 512), (8, 16, 17408 // 8)])
def test_fp8_vs_fp64_bruteforce(M, N, K):
    w, cs = inputs.fp8_weights(N, K, 500 + K)
    x = inputs.normal_f16_bits(M, K, 501 + K)
    y_acc, y = oracle.gemv_fp8_w8a16(w, cs, x)
    y_bf = brute_fp8(w, cs, x)
    e4 = e4m3_table_torch()
    mag = (np.abs(f16_bits_to_f64(x)) @ np.abs(e4[w]).T) * cs[None, :]
    assert np.all(np.abs(y_acc - y_bf) <= (K + 2) * 2.0 ** -52 * mag)
    assert np.array_equal(y, oracle.f16_from_double_array(y_acc).reshape(y.shape))


def test_fp8_unit_weights():
    M, N, K = 3, 4, 128
    w = np.full((N, K), 0x38, np.uint8)
    cs = np.ones(N, np.float32)
    rng = np.random.Generator(np.random.PCG64(77))
    xi = rng.integers(-100, 101, (M, K)).astype(np.float16)
    y_acc, y = oracle.gemv_fp8_w8a16(w, cs, xi.view(np.uint16))
    sums = xi.astype(np.float64).sum(axis=1)
    assert np.array_equal(y_acc, np.repeat(sums[:, None], N, axis=1))
    assert np.array_equal(y, np.repeat(sums[:, None], N, axis=1).astype(np.float16).view(np.uint16))


def test_fp8_generator_saturates_and_hits_subnormals():
    w, _ = inputs.fp8_weights(64, 256, 9)
    e4 = e4m3_table_torch()
    v = e4[w]
    assert np.all(np.isfinite(v))
    sub = ((w & 0x78) == 0) & ((w & 7) != 0)
    assert 0.05 < sub.mean() < 0.5


# ------------------------------------------------------------ determinism

def test_oracle_thread_count_invariance():
    M, N, K = 4, 97, 512
    w_qs, w_d = inputs.q4_0_weights(N, K, 1)
    a_qs, a_d, a_s = oracle.quantize_q8_1(inputs.normal_f32(M, K, 2))
    codes, scales, _ = inputs.nvfp4_weights(N, K, 3)
    w8, cs = inputs.fp8_weights(N, K, 4)
    x = inputs.normal_f16_bits(M, K, 5)
    k_qs, k_hdr = inputs.q4_k_weights(N, K, 6)
    q6 = inputs.q6_k_weights(N, K, 7)
    i_qs, i_hdr = inputs.iq4_xs_weights(N, K, 8)
    prev = oracle.num_threads()
    try:
        outs = []
        for t in (1, 7):
            oracle.set_num_threads(t)
            outs.append((oracle.mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s),
                         oracle.gemv_nvfp4_w4a16(codes, scales, 0.75, x)[0],
                         oracle.gemv_fp8_w8a16(w8, cs, x)[0],
                         oracle.mmvq_q4_k(k_qs, k_hdr, a_qs, a_d, a_s),
                         oracle.mmvq_q6_k(*q6, a_qs, a_d),
                         oracle.mmvq_iq4_xs(i_qs, i_hdr, a_qs, a_d)))
        for a, b in zip(*outs):
            assert np.array_equal(a, b)
    finally:
        oracle.set_num_threads(prev)
