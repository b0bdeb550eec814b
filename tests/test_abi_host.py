"""C-ABI checks that need no GPU: the library loads, exports every function
include/skinny_gemm.h declares, and rejects bad arguments on the host with
the documented status codes before making any HIP call.

Only invalid calls (and the M == 0 / N == 0 no-ops, which return before any
HIP call) are made here; nothing is launched.
"""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "skinny_gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    import skinny_gemm_amd

    return skinny_gemm_amd.lib()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["skinny_status_string", "quantize_act_q8_1",
                                           "mmvq_q4_0", "mmvq_q4_0_f32act", "mmvq_q4_k",
                                           "mmvq_q6_k", "gemv_nvfp4_w4a16", "gemv_fp8_w8a16",
                                           "prepack_nvfp4_size", "prepack_nvfp4",
                                           "gemv_nvfp4_w4a16_packed", "prepack_q4_0_size",
                                           "prepack_q4_0", "mmvq_q4_0_packed", "prepack_fp8_size",
                                           "prepack_fp8", "gemv_fp8_w8a16_packed", "prepack_q4_k_size",
                                           "prepack_q4_k", "mmvq_q4_k_packed", "prepack_q6_k_size",
                                           "prepack_q6_k", "mmvq_q6_k_packed", "mmvq_iq4_xs",
                                           "prepack_iq4_xs_size", "prepack_iq4_xs",
                                           "mmvq_iq4_xs_packed"])


def test_library_exports_every_declared_symbol(L):
    import skinny_gemm_amd

    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", skinny_gemm_amd.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, name


def test_status_strings(L):
    import skinny_gemm_amd

    for code in (0, -1, -2, -3, -4, -5):
        assert skinny_gemm_amd.status_string(code) != "unknown status"
    assert skinny_gemm_amd.status_string(7) == "unknown status"


A = 0x10000          # a 16-byte aligned stand-in address (never dereferenced)
V = ctypes.c_void_p


def q4(L, w=A, wd=A, N=64, K=256, aq=A, ad=A, as_=A, M=1, y=A):
    return L.mmvq_q4_0(V(w), V(wd), N, K, V(aq), V(ad), V(as_), M, V(y), None)


def nv(L, c=A, s=A, N=64, K=256, x=A, M=1, y=A):
    return L.gemv_nvfp4_w4a16(V(c), V(s), 1.0, N, K, V(x), M, V(y), None)


def f8(L, w=A, cs=A, N=64, K=256, x=A, M=1, y=A):
    return L.gemv_fp8_w8a16(V(w), V(cs), N, K, V(x), M, V(y), None)


def q4k(L, w=A, h=A, N=64, K=256, aq=A, ad=A, as_=A, M=1, y=A):
    return L.mmvq_q4_k(V(w), V(h), N, K, V(aq), V(ad), V(as_), M, V(y), None)


def q6k(L, ql=A, qh=A, sc=A, d=A, N=64, K=256, aq=A, ad=A, M=1, y=A):
    return L.mmvq_q6_k(V(ql), V(qh), V(sc), V(d), N, K, V(aq), V(ad), M, V(y), None)


def iq4(L, w=A, h=A, N=64, K=256, aq=A, ad=A, M=1, y=A):
    return L.mmvq_iq4_xs(V(w), V(h), N, K, V(aq), V(ad), M, V(y), None)


def qa(L, x=A, M=1, K=256, qs=A, d=A, s=A):
    return L.quantize_act_q8_1(V(x), M, K, V(qs), V(d), V(s), None)


@pytest.mark.parametrize("fn,max_m", [(q4, 8), (q4k, 8), (q6k, 8), (iq4, 8), (nv, 16), (f8, 96)])
def test_gemv_rejects_m_out_of_range(L, fn, max_m):
    assert fn(L, M=max_m + 1) == -4
    assert fn(L, M=-1) == -4
    assert fn(L, M=1000) == -4
    # the largest M passes M validation (stopped here by a NULL pointer)
    assert fn(L, M=max_m, y=0) == -1


@pytest.mark.parametrize("fn,kmult", [(q4, 32), (nv, 32), (f8, 16)])
def test_gemv_rejects_bad_shapes(L, fn, kmult):
    assert fn(L, K=0) == -2
    assert fn(L, K=-32) == -2
    assert fn(L, K=kmult + kmult // 2) == -2
    assert fn(L, K=(1 << 20) + kmult) == -2
    assert fn(L, N=-1) == -2
    assert fn(L, N=(1 << 24) + 1) == -2
    assert fn(L, N=1 << 28) == -2
    # the largest N passes shape validation
    assert fn(L, N=1 << 24, y=0) == -1
    # the largest K passes shape validation (stopped here by a NULL pointer)
    assert fn(L, K=1 << 20, y=0) == -1


def test_fp8_accepts_k_multiple_of_16(L):
    assert f8(L, K=48, y=0) == -1
    assert q4(L, K=48, y=0) == -2
    assert nv(L, K=48, y=0) == -2


def test_gemv_null_pointers(L):
    for kw in ("w", "wd", "aq", "ad", "as_", "y"):
        assert q4(L, **{kw: 0}) == -1, kw
    for kw in ("c", "s", "x", "y"):
        assert nv(L, **{kw: 0}) == -1, kw
    for kw in ("w", "cs", "x", "y"):
        assert f8(L, **{kw: 0}) == -1, kw


def test_gemv_misaligned(L):
    for kw, off in (("w", 8), ("aq", 4), ("wd", 8), ("ad", 8), ("as_", 2), ("y", 2)):
        assert q4(L, **{kw: A + off}) == -3, kw
    for kw, off in (("c", 8), ("s", 8), ("x", 8), ("y", 1)):
        assert nv(L, **{kw: A + off}) == -3, kw
    for kw, off in (("w", 8), ("cs", 2), ("x", 8), ("y", 1)):
        assert f8(L, **{kw: A + off}) == -3, kw
    # the weaker requirements really are weaker
    assert q4(L, y=A + 4, w=0) == -1
    assert nv(L, y=A + 2, c=0) == -1
    assert f8(L, cs=A + 4, y=0) == -1


def test_empty_calls_are_noops(L):
    # M == 0 or N == 0: nothing to compute, pointers may be NULL, no HIP call
    assert q4(L, w=0, wd=0, aq=0, ad=0, as_=0, y=0, M=0) == 0
    assert q4(L, w=0, wd=0, aq=0, ad=0, as_=0, y=0, N=0) == 0
    assert nv(L, c=0, s=0, x=0, y=0, M=0) == 0
    assert nv(L, c=0, s=0, x=0, y=0, N=0) == 0
    assert f8(L, w=0, cs=0, x=0, y=0, M=0) == 0
    assert f8(L, w=0, cs=0, x=0, y=0, N=0) == 0
    assert qa(L, x=0, qs=0, d=0, s=0, M=0) == 0


def test_quantize_validation(L):
    assert qa(L, K=48) == -2
    assert qa(L, K=0) == -2
    assert qa(L, M=-1) == -4
    assert qa(L, M=65537) == -4
    # M * K is capped at 2^32 elements (the grid has one thread per 8)
    assert qa(L, M=65536, K=1 << 20) == -2
    assert qa(L, M=4097, K=1 << 20) == -2
    assert qa(L, M=4096, K=1 << 20, x=0) == -1
    assert qa(L, M=65536, K=65536, x=0) == -1
    assert qa(L, x=0) == -1
    assert qa(L, s=0) == -1
    assert qa(L, x=A + 4) == -3
    assert qa(L, qs=A + 8) == -3
    assert qa(L, d=A + 1) == -3


def test_binding_raises_without_gpu_tensors():
    import torch

    import skinny_gemm_amd

    with pytest.raises(ValueError):
        skinny_gemm_amd.gemv_fp8_w8a16(torch.zeros((4, 16), dtype=torch.uint8),
                                       torch.ones(4), torch.zeros((1, 16), dtype=torch.float16))
    with pytest.raises(TypeError):
        skinny_gemm_amd.quantize_act_q8_1(torch.zeros((1, 32), dtype=torch.float64))


def test_binding_rejects_tensors_on_two_devices():
    # the check runs before any device context or library call, so stand-ins
    # that only carry a device are enough
    import types

    import torch

    from skinny_gemm_amd import _lib

    a = types.SimpleNamespace(device=torch.device("cuda", 0))
    b = types.SimpleNamespace(device=torch.device("cuda", 1))
    with pytest.raises(ValueError, match="one device"):
        _lib._run("mmvq_q4_0", (a, a, b), None)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from skinny_gemm_amd import _lib

    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_f32act_validation(L):
    f = L.mmvq_q4_0_f32act
    f.restype = ctypes.c_int
    ok = dict(w=V(A), d=V(A), x=V(A), y=V(A))
    def call(N=64, K=256, M=1, **kw):
        a = dict(ok, **kw)
        return f(a["w"], a["d"], N, K, a["x"], M, a["y"], None)
    assert call(M=3) == -4 and call(M=-1) == -4          # decode widths only
    assert call(K=12288 + 32) == -2 and call(K=48) == -2 and call(K=0) == -2
    assert call(M=0) == 0 and call(N=0) == 0              # nothing to do
    assert call(x=None) == -1 and call(w=None) == -1
    assert call(x=V(A + 4)) == -3 and call(w=V(A + 8)) == -3 and call(y=V(A + 2)) == -3


@pytest.mark.parametrize("fn", [q4k, q6k, iq4])
def test_k_quant_validation(L, fn):
    # K must be a whole number of 256-weight super-blocks
    for K in (0, 32, 128, 256 + 32, 4096 + 128, (1 << 20) + 256):
        assert fn(L, K=K) == -2, K
    assert fn(L, K=1 << 20, y=0) == -1
    assert fn(L, N=-1) == -2
    # no-ops
    assert fn(L, M=0, y=0, aq=0) == 0
    assert fn(L, N=0, y=0, aq=0) == 0


def test_k_quant_null_and_alignment(L):
    for kw in ("w", "h", "aq", "ad", "as_", "y"):
        assert q4k(L, **{kw: 0}) == -1, kw
    for kw, off in (("w", 8), ("h", 8), ("aq", 8), ("ad", 8), ("as_", 2), ("y", 2)):
        assert q4k(L, **{kw: A + off}) == -3, kw
    for kw in ("ql", "qh", "sc", "d", "aq", "ad", "y"):
        assert q6k(L, **{kw: 0}) == -1, kw
    for kw, off in (("ql", 8), ("qh", 4), ("sc", 1), ("d", 1), ("aq", 8), ("ad", 8), ("y", 2)):
        assert q6k(L, **{kw: A + off}) == -3, kw
    # the weaker requirements really are weaker
    assert q6k(L, qh=A + 8, y=0) == -1
    assert q6k(L, sc=A + 2, y=0) == -1
    for kw in ("w", "h", "aq", "ad", "y"):
        assert iq4(L, **{kw: 0}) == -1, kw
    for kw, off in (("w", 8), ("h", 8), ("aq", 8), ("ad", 8), ("y", 2)):
        assert iq4(L, **{kw: A + off}) == -3, kw


def nvp(L, w=A, N=64, K=256, x=A, M=1, y=A):
    return L.gemv_nvfp4_w4a16_packed(V(w), 1.0, N, K, V(x), M, V(y), None)


def pre(L, c=A, s=A, N=64, K=256, w=A):
    return L.prepack_nvfp4(V(c), V(s), N, K, V(w), None)


def test_prepack_size_is_whole_tiles_and_scale_blocks(L):
    import skinny_gemm_amd

    n = ctypes.c_size_t(0)
    # U = ceil(N/16) tiles, S = K/128 steps, V = ceil(S/8) scale blocks: 1024 U (S + V)
    for N, K, want in ((1, 256, 1024 * 1 * (2 + 1)), (16, 1024, 1024 * (8 + 1)),
                       (17, 2304, 1024 * 2 * (18 + 3)), (4096, 4096, 1024 * 256 * (32 + 4)),
                       (0, 256, 0)):
        assert L.prepack_nvfp4_size(N, K, ctypes.byref(n)) == 0
        assert n.value == want, (N, K)
        assert skinny_gemm_amd.prepack_nvfp4_size(N, K) == want
    # whole 16-row tiles and 1024-element K give exactly the canonical bytes
    assert skinny_gemm_amd.prepack_nvfp4_size(5120, 17408) == 5120 * 17408 * 9 // 16
    assert L.prepack_nvfp4_size(16, 128, ctypes.byref(n)) == -2
    assert L.prepack_nvfp4_size(16, 0, ctypes.byref(n)) == -2
    assert L.prepack_nvfp4_size(-1, 256, ctypes.byref(n)) == -2
    assert L.prepack_nvfp4_size((1 << 24) + 1, 256, ctypes.byref(n)) == -2
    assert L.prepack_nvfp4_size(16, 256, None) == -1


def test_packed_validation(L):
    assert nvp(L, M=17) == -4
    assert nvp(L, M=-1) == -4
    assert nvp(L, M=16, y=0) == -1
    for K in (0, 128, 32, 384, (1 << 20) + 256):
        assert nvp(L, K=K) == -2, K
        assert pre(L, K=K) == -2, K
    assert nvp(L, K=1 << 20, y=0) == -1
    assert nvp(L, N=-1) == -2
    assert nvp(L, N=(1 << 24) + 1) == -2
    for kw in ("w", "x", "y"):
        assert nvp(L, **{kw: 0}) == -1, kw
    for kw in ("c", "s", "w"):
        assert pre(L, **{kw: 0}) == -1, kw
    for kw, off in (("w", 8), ("x", 8), ("y", 1)):
        assert nvp(L, **{kw: A + off}) == -3, kw
    for kw, off in (("c", 8), ("s", 1), ("w", 8)):
        assert pre(L, **{kw: A + off}) == -3, kw
    # scales need only 2-byte alignment, y only 2
    assert pre(L, s=A + 2, c=0) == -1
    assert nvp(L, y=A + 2, w=0) == -1
    # nothing to compute
    assert nvp(L, w=0, x=0, y=0, M=0) == 0
    assert nvp(L, w=0, x=0, y=0, N=0) == 0
    assert pre(L, c=0, s=0, w=0, N=0) == 0


def q4p(L, w=A, N=64, K=256, aq=A, ad=A, as_=A, M=1, y=A):
    return L.mmvq_q4_0_packed(V(w), N, K, V(aq), V(ad), V(as_), M, V(y), None)


def q4pre(L, w=A, d=A, N=64, K=256, p=A):
    return L.prepack_q4_0(V(w), V(d), N, K, V(p), None)


def test_prepack_q4_0_size(L):
    import skinny_gemm_amd

    n = ctypes.c_size_t(0)
    # 1024 U P + 512 U V, U = ceil(N/16), P = K/128, V = ceil(K/512)
    for N, K, want in ((1, 256, 1024 * 2 + 512), (16, 512, 1024 * 4 + 512),
                       (17, 768, 2 * (1024 * 6 + 512 * 2)), (0, 256, 0),
                       (4096, 4096, 256 * (1024 * 32 + 512 * 8))):
        assert L.prepack_q4_0_size(N, K, ctypes.byref(n)) == 0
        assert n.value == want, (N, K)
        assert skinny_gemm_amd.prepack_q4_0_size(N, K) == want
    # whole tiles and K % 512 == 0: exactly the canonical bytes
    assert skinny_gemm_amd.prepack_q4_0_size(4096, 11264) == 4096 * 11264 * 18 // 32
    for N, K in ((16, 128), (16, 0), (-1, 256), ((1 << 24) + 1, 256)):
        assert L.prepack_q4_0_size(N, K, ctypes.byref(n)) == -2
    assert L.prepack_q4_0_size(16, 256, None) == -1


def test_q4_0_packed_validation(L):
    assert q4p(L, M=9) == -4
    assert q4p(L, M=-1) == -4
    assert q4p(L, M=8, y=0) == -1
    for K in (0, 128, 32, 384, (1 << 20) + 256):
        assert q4p(L, K=K) == -2, K
        assert q4pre(L, K=K) == -2, K
    assert q4p(L, K=1 << 20, y=0) == -1
    assert q4p(L, N=-1) == -2
    assert q4p(L, N=(1 << 24) + 1) == -2
    for kw in ("w", "aq", "ad", "as_", "y"):
        assert q4p(L, **{kw: 0}) == -1, kw
    for kw in ("w", "d", "p"):
        assert q4pre(L, **{kw: 0}) == -1, kw
    for kw, off in (("w", 8), ("aq", 8), ("ad", 8), ("as_", 8), ("y", 2)):
        assert q4p(L, **{kw: A + off}) == -3, kw
    for kw, off in (("w", 8), ("d", 1), ("p", 8)):
        assert q4pre(L, **{kw: A + off}) == -3, kw
    assert q4pre(L, d=A + 2, w=0) == -1
    assert q4p(L, y=A + 4, w=0) == -1
    assert q4p(L, w=0, aq=0, ad=0, as_=0, y=0, M=0) == 0
    assert q4p(L, w=0, aq=0, ad=0, as_=0, y=0, N=0) == 0
    assert q4pre(L, w=0, d=0, p=0, N=0) == 0


def f8p(L, w=A, cs=A, N=64, K=256, x=A, M=1, y=A):
    return L.gemv_fp8_w8a16_packed(V(w), V(cs), N, K, V(x), M, V(y), None)


def f8pre(L, w=A, N=64, K=256, p=A):
    return L.prepack_fp8(V(w), N, K, V(p), None)


def test_fp8_packed_validation(L):
    import skinny_gemm_amd

    n = ctypes.c_size_t(0)
    for N, K, want in ((1, 256, 16 * 256), (17, 512, 32 * 512), (0, 256, 0)):
        assert L.prepack_fp8_size(N, K, ctypes.byref(n)) == 0
        assert n.value == want
        assert skinny_gemm_amd.prepack_fp8_size(N, K) == want
    assert L.prepack_fp8_size(16, 128, ctypes.byref(n)) == -2
    assert L.prepack_fp8_size(16, 256, None) == -1
    assert f8p(L, M=97) == -4
    assert f8p(L, M=-1) == -4
    assert f8p(L, M=96, y=0) == -1
    for K in (0, 128, 16, 384, (1 << 20) + 256):
        assert f8p(L, K=K) == -2, K
        assert f8pre(L, K=K) == -2, K
    assert f8p(L, N=-1) == -2
    for kw in ("w", "cs", "x", "y"):
        assert f8p(L, **{kw: 0}) == -1, kw
    for kw in ("w", "p"):
        assert f8pre(L, **{kw: 0}) == -1, kw
    for kw, off in (("w", 8), ("cs", 2), ("x", 8), ("y", 1)):
        assert f8p(L, **{kw: A + off}) == -3, kw
    for kw, off in (("w", 8), ("p", 8)):
        assert f8pre(L, **{kw: A + off}) == -3, kw
    assert f8p(L, cs=A + 4, y=A + 2, w=0) == -1
    assert f8p(L, w=0, cs=0, x=0, y=0, M=0) == 0
    assert f8p(L, w=0, cs=0, x=0, y=0, N=0) == 0
    assert f8pre(L, w=0, p=0, N=0) == 0


def q4kp(L, w=A, N=64, K=256, aq=A, ad=A, as_=A, M=1, y=A):
    return L.mmvq_q4_k_packed(V(w), N, K, V(aq), V(ad), V(as_), M, V(y), None)


def iq4p(L, w=A, N=64, K=256, aq=A, ad=A, M=1, y=A):
    return L.mmvq_iq4_xs_packed(V(w), N, K, V(aq), V(ad), M, V(y), None)


def test_iq4_xs_packed_validation(L):
    import skinny_gemm_amd

    n = ctypes.c_size_t(0)
    for N, K, want in ((1, 256, 1024 * 2 + 128), (17, 512, 2 * (1024 * 4 + 256)), (0, 256, 0)):
        assert L.prepack_iq4_xs_size(N, K, ctypes.byref(n)) == 0
        assert n.value == want
        assert skinny_gemm_amd.prepack_iq4_xs_size(N, K) == want
    # whole tiles: exactly the canonical bytes (codes + 8-byte headers)
    assert skinny_gemm_amd.prepack_iq4_xs_size(4096, 12288) == 4096 * 12288 * 17 // 32
    assert L.prepack_iq4_xs_size(16, 128, ctypes.byref(n)) == -2
    assert L.prepack_iq4_xs_size(16, 256, None) == -1
    assert iq4p(L, M=9) == -4
    assert iq4p(L, M=8, y=0) == -1
    for K in (0, 128, 384):
        assert iq4p(L, K=K) == -2, K
        assert L.prepack_iq4_xs(V(A), V(A), 64, K, V(A), None) == -2, K
    for kw in ("w", "aq", "ad", "y"):
        assert iq4p(L, **{kw: 0}) == -1, kw
    assert L.prepack_iq4_xs(V(0), V(A), 64, 256, V(A), None) == -1
    assert L.prepack_iq4_xs(V(A), V(A + 8), 64, 256, V(A), None) == -3
    assert L.prepack_iq4_xs(V(A), V(A), 64, 256, V(A + 8), None) == -3
    for kw, off in (("w", 8), ("aq", 8), ("ad", 8), ("y", 2)):
        assert iq4p(L, **{kw: A + off}) == -3, kw
    assert iq4p(L, w=0, aq=0, ad=0, y=0, M=0) == 0
    assert L.prepack_iq4_xs(V(0), V(0), 0, 256, V(0), None) == 0


def test_q4_k_packed_validation(L):
    import skinny_gemm_amd

    n = ctypes.c_size_t(0)
    for N, K, want in ((1, 256, 1024 * 2 + 256), (17, 512, 2 * (1024 * 4 + 512)), (0, 256, 0)):
        assert L.prepack_q4_k_size(N, K, ctypes.byref(n)) == 0
        assert n.value == want
        assert skinny_gemm_amd.prepack_q4_k_size(N, K) == want
    # whole tiles: exactly the canonical bytes (codes + 16-byte headers)
    assert skinny_gemm_amd.prepack_q4_k_size(4096, 12288) == 4096 * 12288 * 9 // 16
    assert L.prepack_q4_k_size(16, 128, ctypes.byref(n)) == -2
    assert L.prepack_q4_k_size(16, 256, None) == -1
    assert q4kp(L, M=9) == -4
    assert q4kp(L, M=8, y=0) == -1
    for K in (0, 128, 384):
        assert q4kp(L, K=K) == -2, K
        assert L.prepack_q4_k(V(A), V(A), 64, K, V(A), None) == -2, K
    for kw in ("w", "aq", "ad", "as_", "y"):
        assert q4kp(L, **{kw: 0}) == -1, kw
    assert L.prepack_q4_k(V(0), V(A), 64, 256, V(A), None) == -1
    assert L.prepack_q4_k(V(A), V(A + 8), 64, 256, V(A), None) == -3
    assert L.prepack_q4_k(V(A), V(A), 64, 256, V(A + 8), None) == -3
    for kw, off in (("w", 8), ("aq", 8), ("ad", 8), ("as_", 8), ("y", 2)):
        assert q4kp(L, **{kw: A + off}) == -3, kw
    assert q4kp(L, w=0, aq=0, ad=0, as_=0, y=0, M=0) == 0
    assert L.prepack_q4_k(V(0), V(0), 0, 256, V(0), None) == 0


def test_q6_k_packed_validation(L):
    import skinny_gemm_amd

    n = ctypes.c_size_t(0)
    for N, K, want in ((1, 256, 1024 * 2 + 1312), (17, 512, 2 * (1024 * 4 + 1312 * 2)), (0, 256, 0)):
        assert L.prepack_q6_k_size(N, K, ctypes.byref(n)) == 0
        assert n.value == want
        assert skinny_gemm_amd.prepack_q6_k_size(N, K) == want
    # whole tiles: exactly the canonical bytes (6.5625 bits per weight)
    assert skinny_gemm_amd.prepack_q6_k_size(4096, 12288) == 4096 * 12288 * 105 // 128
    assert L.prepack_q6_k_size(16, 128, ctypes.byref(n)) == -2
    assert L.prepack_q6_k_size(16, 256, None) == -1

    def q6p(w=A, N=64, K=256, aq=A, ad=A, M=1, y=A):
        return L.mmvq_q6_k_packed(V(w), N, K, V(aq), V(ad), M, V(y), None)

    def pre(ql=A, qh=A, sc=A, d=A, N=64, K=256, p=A):
        return L.prepack_q6_k(V(ql), V(qh), V(sc), V(d), N, K, V(p), None)

    assert q6p(M=9) == -4
    assert q6p(M=8, y=0) == -1
    for K in (0, 128, 384):
        assert q6p(K=K) == -2, K
        assert pre(K=K) == -2, K
    for kw in ("w", "aq", "ad", "y"):
        assert q6p(**{kw: 0}) == -1, kw
    for kw in ("ql", "qh", "sc", "d", "p"):
        assert pre(**{kw: 0}) == -1, kw
    for kw, off in (("w", 8), ("aq", 8), ("ad", 8), ("y", 2)):
        assert q6p(**{kw: A + off}) == -3, kw
    for kw, off in (("ql", 8), ("qh", 4), ("sc", 1), ("d", 1), ("p", 8)):
        assert pre(**{kw: A + off}) == -3, kw
    assert q6p(w=0, aq=0, ad=0, y=0, M=0) == 0
    assert pre(ql=0, qh=0, sc=0, d=0, p=0, N=0) == 0
