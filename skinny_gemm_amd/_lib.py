"""ctypes binding of libskinny_gemm.so.

Argument marshalling only: each function checks tensor dtypes, shapes,
device and contiguity, allocates outputs that were not supplied (torch is
used for device memory and streams, nothing else), and calls the C entry of
the same name with the tensors' device current, on that device's current
stream unless a stream is given.  Every step of the computation runs in
the library's HIP kernels.  A missing library raises immediately; there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libskinny_gemm.so")

OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_ALIGN = -3
ERR_M = -4
ERR_LAUNCH = -5

EXPORTS = ("skinny_status_string", "quantize_act_q8_1", "mmvq_q4_0", "mmvq_q4_0_f32act",
           "mmvq_q4_k", "mmvq_q6_k", "prepack_q4_0_size", "prepack_q4_0", "mmvq_q4_0_packed",
           "gemv_nvfp4_w4a16", "prepack_nvfp4_size", "prepack_nvfp4",
           "gemv_nvfp4_w4a16_packed", "gemv_fp8_w8a16", "prepack_fp8_size", "prepack_fp8",
           "gemv_fp8_w8a16_packed", "prepack_q4_k_size", "prepack_q4_k", "mmvq_q4_k_packed",
           "prepack_q6_k_size", "prepack_q6_k", "mmvq_q6_k_packed", "mmvq_iq4_xs",
           "prepack_iq4_xs_size", "prepack_iq4_xs", "mmvq_iq4_xs_packed")

_lib = None


class SkinnyError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__("%s failed with status %d (%s)" % (fn, status, text))
        self.status = status


def library_path() -> str:
    return LIB_PATH


def lib():
    """Load libskinny_gemm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libskinny_gemm.so is not built (%s); run "
                           "`python -m skinny_gemm_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L.skinny_status_string.argtypes = [I]
    L.skinny_status_string.restype = ctypes.c_char_p
    L.quantize_act_q8_1.argtypes = [P, I, I, P, P, P, P]
    L.quantize_act_q8_1.restype = I
    L.mmvq_q4_0.argtypes = [P, P, I, I, P, P, P, I, P, P]
    L.mmvq_q4_0.restype = I
    L.mmvq_q4_0_f32act.argtypes = [P, P, I, I, P, I, P, P]
    L.mmvq_q4_0_f32act.restype = I
    L.mmvq_q4_k.argtypes = [P, P, I, I, P, P, P, I, P, P]
    L.mmvq_q4_k.restype = I
    L.mmvq_q6_k.argtypes = [P, P, P, P, I, I, P, P, I, P, P]
    L.mmvq_q6_k.restype = I
    L.mmvq_iq4_xs.argtypes = [P, P, I, I, P, P, I, P, P]
    L.mmvq_iq4_xs.restype = I
    L.gemv_nvfp4_w4a16.argtypes = [P, P, ctypes.c_float, I, I, P, I, P, P]
    L.gemv_nvfp4_w4a16.restype = I
    L.prepack_q4_0_size.argtypes = [I, I, ctypes.POINTER(ctypes.c_size_t)]
    L.prepack_q4_0_size.restype = I
    L.prepack_q4_0.argtypes = [P, P, I, I, P, P]
    L.prepack_q4_0.restype = I
    L.mmvq_q4_0_packed.argtypes = [P, I, I, P, P, P, I, P, P]
    L.mmvq_q4_0_packed.restype = I
    L.prepack_q4_k_size.argtypes = [I, I, ctypes.POINTER(ctypes.c_size_t)]
    L.prepack_q4_k_size.restype = I
    L.prepack_q4_k.argtypes = [P, P, I, I, P, P]
    L.prepack_q4_k.restype = I
    L.mmvq_q4_k_packed.argtypes = [P, I, I, P, P, P, I, P, P]
    L.mmvq_q4_k_packed.restype = I
    L.prepack_iq4_xs_size.argtypes = [I, I, ctypes.POINTER(ctypes.c_size_t)]
    L.prepack_iq4_xs_size.restype = I
    L.prepack_iq4_xs.argtypes = [P, P, I, I, P, P]
    L.prepack_iq4_xs.restype = I
    L.mmvq_iq4_xs_packed.argtypes = [P, I, I, P, P, I, P, P]
    L.mmvq_iq4_xs_packed.restype = I
    L.prepack_q6_k_size.argtypes = [I, I, ctypes.POINTER(ctypes.c_size_t)]
    L.prepack_q6_k_size.restype = I
    L.prepack_q6_k.argtypes = [P, P, P, P, I, I, P, P]
    L.prepack_q6_k.restype = I
    L.mmvq_q6_k_packed.argtypes = [P, I, I, P, P, I, P, P]
    L.mmvq_q6_k_packed.restype = I
    L.prepack_nvfp4_size.argtypes = [I, I, ctypes.POINTER(ctypes.c_size_t)]
    L.prepack_nvfp4_size.restype = I
    L.prepack_nvfp4.argtypes = [P, P, I, I, P, P]
    L.prepack_nvfp4.restype = I
    L.gemv_nvfp4_w4a16_packed.argtypes = [P, ctypes.c_float, I, I, P, I, P, P]
    L.gemv_nvfp4_w4a16_packed.restype = I
    L.gemv_fp8_w8a16.argtypes = [P, P, I, I, P, I, P, P]
    L.gemv_fp8_w8a16.restype = I
    L.prepack_fp8_size.argtypes = [I, I, ctypes.POINTER(ctypes.c_size_t)]
    L.prepack_fp8_size.restype = I
    L.prepack_fp8.argtypes = [P, I, I, P, P]
    L.prepack_fp8.restype = I
    L.gemv_fp8_w8a16_packed.argtypes = [P, P, I, I, P, I, P, P]
    L.gemv_fp8_w8a16_packed.restype = I
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().skinny_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise SkinnyError(fn, status, status_string(status))


# ------------------------------------------------------------- marshalling

def _torch():
    import torch

    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run(fn: str, tensors, stream, *args) -> None:
    """Call C entry `fn` with `args` and the stream appended, with the
    tensors' device current (the library launches on, and sizes its LDS
    limits for, the current device).  Every tensor must be on that one
    device; `stream` defaults to its current stream and must belong to it."""
    torch = _torch()
    device = tensors[0].device
    for t in tensors[1:]:
        if t.device != device:
            raise ValueError("%s: tensors on %s and %s; all must be on one device"
                             % (fn, device, t.device))
    with torch.cuda.device(device):
        if stream is None:
            stream = torch.cuda.current_stream(device)
        elif stream.device != device:
            raise ValueError("%s: stream on %s, tensors on %s" % (fn, stream.device, device))
        _check(fn, getattr(lib(), fn)(*args, ctypes.c_void_p(stream.cuda_stream)))


def _req(t, name, dtypes, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s: dtype %s not in %s" % (name, t.dtype, dtypes))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t


def _f16_bits_dtypes():
    torch = _torch()
    return (torch.float16, torch.int16, torch.uint16)


def quantize_act_q8_1(x, qs=None, d=None, s=None, stream=None):
    """x float32 [M][K] -> (qs int8 [M][K], d, s binary16 [M][K/32])."""
    torch = _torch()
    _req(x, "x", (torch.float32,))
    M, K = x.shape
    if qs is None:
        qs = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((M, K // 32), dtype=torch.float16, device=x.device)
    if s is None:
        s = torch.empty((M, K // 32), dtype=torch.float16, device=x.device)
    _req(qs, "qs", (torch.int8,), (M, K))
    _req(d, "d", _f16_bits_dtypes(), (M, K // 32))
    _req(s, "s", _f16_bits_dtypes(), (M, K // 32))
    _run("quantize_act_q8_1", (x, qs, d, s), stream, _ptr(x), M, K, _ptr(qs), _ptr(d), _ptr(s))
    return qs, d, s


def mmvq_q4_0(w_qs, w_d, a_qs, a_d, a_s, y=None, stream=None):
    """Q4_0 weights [N][K/2] + [N][K/32], Q8_1 activations -> y float32 [M][N]."""
    torch = _torch()
    _req(w_qs, "w_qs", (torch.uint8,))
    N, K2 = w_qs.shape
    K = 2 * K2
    _req(w_d, "w_d", _f16_bits_dtypes(), (N, K // 32))
    _req(a_qs, "a_qs", (torch.int8,))
    M = a_qs.shape[0]
    _req(a_qs, "a_qs", (torch.int8,), (M, K))
    _req(a_d, "a_d", _f16_bits_dtypes(), (M, K // 32))
    _req(a_s, "a_s", _f16_bits_dtypes(), (M, K // 32))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=w_qs.device)
    _req(y, "y", (torch.float32,), (M, N))
    _run("mmvq_q4_0", (w_qs, w_d, a_qs, a_d, a_s, y), stream, _ptr(w_qs), _ptr(w_d), N, K,
         _ptr(a_qs), _ptr(a_d), _ptr(a_s), M, _ptr(y))
    return y


def mmvq_q4_0_f32act(w_qs, w_d, x, y=None, stream=None):
    """Q4_0 weights [N][K/2] + [N][K/32], float32 activations x [M][K] (M <= 2)
    quantized to Q8_1 inside the same launch -> y float32 [M][N]."""
    torch = _torch()
    _req(w_qs, "w_qs", (torch.uint8,))
    N, K2 = w_qs.shape
    K = 2 * K2
    _req(w_d, "w_d", _f16_bits_dtypes(), (N, K // 32))
    _req(x, "x", (torch.float32,))
    M = x.shape[0]
    _req(x, "x", (torch.float32,), (M, K))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=w_qs.device)
    _req(y, "y", (torch.float32,), (M, N))
    _run("mmvq_q4_0_f32act", (w_qs, w_d, x, y), stream, _ptr(w_qs), _ptr(w_d), N, K, _ptr(x), M,
         _ptr(y))
    return y


def mmvq_q4_k(w_qs, w_hdr, a_qs, a_d, a_s, y=None, stream=None):
    """Q4_K weights (qs [N][K/2], hdr [N][K/256][16]), Q8_1 activations
    -> y float32 [M][N]."""
    torch = _torch()
    _req(w_qs, "w_qs", (torch.uint8,))
    N, K2 = w_qs.shape
    K = 2 * K2
    _req(w_hdr, "w_hdr", (torch.uint8,), (N, K // 256, 16))
    _req(a_qs, "a_qs", (torch.int8,))
    M = a_qs.shape[0]
    _req(a_qs, "a_qs", (torch.int8,), (M, K))
    _req(a_d, "a_d", _f16_bits_dtypes(), (M, K // 32))
    _req(a_s, "a_s", _f16_bits_dtypes(), (M, K // 32))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=w_qs.device)
    _req(y, "y", (torch.float32,), (M, N))
    _run("mmvq_q4_k", (w_qs, w_hdr, a_qs, a_d, a_s, y), stream, _ptr(w_qs), _ptr(w_hdr), N, K,
         _ptr(a_qs), _ptr(a_d), _ptr(a_s), M, _ptr(y))
    return y


def mmvq_q6_k(w_ql, w_qh, w_sc, w_d, a_qs, a_d, y=None, stream=None):
    """Q6_K weights (ql [N][K/2], qh [N][K/4], sc int8 [N][K/16], d [N][K/256]),
    Q8_1 activations (codes and d8) -> y float32 [M][N]."""
    torch = _torch()
    _req(w_ql, "w_ql", (torch.uint8,))
    N, K2 = w_ql.shape
    K = 2 * K2
    _req(w_qh, "w_qh", (torch.uint8,), (N, K // 4))
    _req(w_sc, "w_sc", (torch.int8,), (N, K // 16))
    _req(w_d, "w_d", _f16_bits_dtypes(), (N, K // 256))
    _req(a_qs, "a_qs", (torch.int8,))
    M = a_qs.shape[0]
    _req(a_qs, "a_qs", (torch.int8,), (M, K))
    _req(a_d, "a_d", _f16_bits_dtypes(), (M, K // 32))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=w_ql.device)
    _req(y, "y", (torch.float32,), (M, N))
    _run("mmvq_q6_k", (w_ql, w_qh, w_sc, w_d, a_qs, a_d, y), stream, _ptr(w_ql), _ptr(w_qh),
         _ptr(w_sc), _ptr(w_d), N, K, _ptr(a_qs), _ptr(a_d), M, _ptr(y))
    return y


def mmvq_iq4_xs(w_qs, w_hdr, a_qs, a_d, y=None, stream=None):
    """IQ4_XS weights (qs [N][K/2], hdr [N][K/256][8]), Q8_1 activations
    (codes and d8) -> y float32 [M][N]."""
    torch = _torch()
    _req(w_qs, "w_qs", (torch.uint8,))
    N, K2 = w_qs.shape
    K = 2 * K2
    _req(w_hdr, "w_hdr", (torch.uint8,), (N, K // 256, 8))
    _req(a_qs, "a_qs", (torch.int8,))
    M = a_qs.shape[0]
    _req(a_qs, "a_qs", (torch.int8,), (M, K))
    _req(a_d, "a_d", _f16_bits_dtypes(), (M, K // 32))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=w_qs.device)
    _req(y, "y", (torch.float32,), (M, N))
    _run("mmvq_iq4_xs", (w_qs, w_hdr, a_qs, a_d, y), stream, _ptr(w_qs), _ptr(w_hdr), N, K,
         _ptr(a_qs), _ptr(a_d), M, _ptr(y))
    return y


def gemv_nvfp4_w4a16(w_codes, w_scales, global_scale, x, y=None, stream=None):
    """NVFP4 weights [N][K/2] codes + [N][K/16] E4M3 scales, binary16 x [M][K]
    -> binary16 y [M][N]."""
    torch = _torch()
    _req(w_codes, "w_codes", (torch.uint8,))
    N, K2 = w_codes.shape
    K = 2 * K2
    _req(w_scales, "w_scales", (torch.uint8, torch.float8_e4m3fn), (N, K // 16))
    _req(x, "x", _f16_bits_dtypes())
    M = x.shape[0]
    _req(x, "x", _f16_bits_dtypes(), (M, K))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _req(y, "y", _f16_bits_dtypes(), (M, N))
    _run("gemv_nvfp4_w4a16", (w_codes, w_scales, x, y), stream, _ptr(w_codes), _ptr(w_scales),
         float(global_scale), N, K, _ptr(x), M, _ptr(y))
    return y


def prepack_q4_0_size(N: int, K: int) -> int:
    """Bytes of the packed copy of an N x K Q4_0 matrix (K % 256 == 0)."""
    n = ctypes.c_size_t(0)
    _check("prepack_q4_0_size", lib().prepack_q4_0_size(int(N), int(K), ctypes.byref(n)))
    return n.value


def prepack_q4_0(w_qs, w_d, w_packed=None, stream=None):
    """Planar Q4_0 weights w_qs [N][K/2], w_d binary16 [N][K/32] -> the packed
    copy (uint8, prepack_q4_0_size(N, K) bytes)."""
    torch = _torch()
    _req(w_qs, "w_qs", (torch.uint8,))
    N, K2 = w_qs.shape
    K = 2 * K2
    _req(w_d, "w_d", _f16_bits_dtypes(), (N, K // 32))
    nbytes = prepack_q4_0_size(N, K)
    if w_packed is None:
        w_packed = torch.empty((nbytes,), dtype=torch.uint8, device=w_qs.device)
    _req(w_packed, "w_packed", (torch.uint8,), (nbytes,))
    _run("prepack_q4_0", (w_qs, w_d, w_packed), stream, _ptr(w_qs), _ptr(w_d), N, K,
         _ptr(w_packed))
    return w_packed


def mmvq_q4_0_packed(w_packed, N, K, a_qs, a_d, a_s, y=None, stream=None):
    """Packed Q4_0 weights (from prepack_q4_0, N x K) x Q8_1 activations
    -> float32 y [M][N]."""
    torch = _torch()
    N, K = int(N), int(K)
    _req(w_packed, "w_packed", (torch.uint8,), (prepack_q4_0_size(N, K),))
    _req(a_qs, "a_qs", (torch.int8,))
    M = a_qs.shape[0]
    _req(a_qs, "a_qs", (torch.int8,), (M, K))
    _req(a_d, "a_d", _f16_bits_dtypes(), (M, K // 32))
    _req(a_s, "a_s", _f16_bits_dtypes(), (M, K // 32))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=a_qs.device)
    _req(y, "y", (torch.float32,), (M, N))
    _run("mmvq_q4_0_packed", (w_packed, a_qs, a_d, a_s, y), stream, _ptr(w_packed), N, K,
         _ptr(a_qs), _ptr(a_d), _ptr(a_s), M, _ptr(y))
    return y


def prepack_nvfp4_size(N: int, K: int) -> int:
    """Bytes of the packed copy of an N x K NVFP4 matrix (K % 256 == 0)."""
    n = ctypes.c_size_t(0)
    _check("prepack_nvfp4_size", lib().prepack_nvfp4_size(int(N), int(K), ctypes.byref(n)))
    return n.value


def prepack_nvfp4(w_codes, w_scales, w_packed=None, stream=None):
    """Canonical NVFP4 weights [N][K/2] codes + [N][K/16] E4M3 scales -> the
    packed copy (uint8, prepack_nvfp4_size(N, K) bytes)."""
    torch = _torch()
    _req(w_codes, "w_codes", (torch.uint8,))
    N, K2 = w_codes.shape
    K = 2 * K2
    _req(w_scales, "w_scales", (torch.uint8, torch.float8_e4m3fn), (N, K // 16))
    nbytes = prepack_nvfp4_size(N, K)
    if w_packed is None:
        w_packed = torch.empty((nbytes,), dtype=torch.uint8, device=w_codes.device)
    _req(w_packed, "w_packed", (torch.uint8,), (nbytes,))
    _run("prepack_nvfp4", (w_codes, w_scales, w_packed), stream, _ptr(w_codes), _ptr(w_scales),
         N, K, _ptr(w_packed))
    return w_packed


def gemv_nvfp4_w4a16_packed(w_packed, N, K, global_scale, x, y=None, stream=None):
    """Packed NVFP4 weights (from prepack_nvfp4, N x K), binary16 x [M][K]
    -> binary16 y [M][N]."""
    torch = _torch()
    N, K = int(N), int(K)
    _req(w_packed, "w_packed", (torch.uint8,), (prepack_nvfp4_size(N, K),))
    _req(x, "x", _f16_bits_dtypes())
    M = x.shape[0]
    _req(x, "x", _f16_bits_dtypes(), (M, K))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _req(y, "y", _f16_bits_dtypes(), (M, N))
    _run("gemv_nvfp4_w4a16_packed", (w_packed, x, y), stream, _ptr(w_packed),
         float(global_scale), N, K, _ptr(x), M, _ptr(y))
    return y


def gemv_fp8_w8a16(w, channel_scale, x, y=None, stream=None):
    """FP8 E4M3 weights [N][K], float32 channel scales [N], binary16 x [M][K]
    -> binary16 y [M][N]."""
    torch = _torch()
    _req(w, "w", (torch.uint8, torch.float8_e4m3fn))
    N, K = w.shape
    _req(channel_scale, "channel_scale", (torch.float32,), (N,))
    _req(x, "x", _f16_bits_dtypes())
    M = x.shape[0]
    _req(x, "x", _f16_bits_dtypes(), (M, K))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _req(y, "y", _f16_bits_dtypes(), (M, N))
    _run("gemv_fp8_w8a16", (w, channel_scale, x, y), stream, _ptr(w), _ptr(channel_scale), N, K,
         _ptr(x), M, _ptr(y))
    return y


def prepack_fp8_size(N: int, K: int) -> int:
    """Bytes of the packed copy of an N x K FP8 matrix (K % 256 == 0)."""
    n = ctypes.c_size_t(0)
    _check("prepack_fp8_size", lib().prepack_fp8_size(int(N), int(K), ctypes.byref(n)))
    return n.value


def prepack_fp8(w, w_packed=None, stream=None):
    """E4M3 weights [N][K] -> the packed copy (uint8, prepack_fp8_size(N, K) bytes)."""
    torch = _torch()
    _req(w, "w", (torch.uint8, torch.float8_e4m3fn))
    N, K = w.shape
    nbytes = prepack_fp8_size(N, K)
    if w_packed is None:
        w_packed = torch.empty((nbytes,), dtype=torch.uint8, device=w.device)
    _req(w_packed, "w_packed", (torch.uint8,), (nbytes,))
    _run("prepack_fp8", (w, w_packed), stream, _ptr(w), N, K, _ptr(w_packed))
    return w_packed


def gemv_fp8_w8a16_packed(w_packed, N, K, channel_scale, x, y=None, stream=None):
    """Packed FP8 weights (from prepack_fp8, N x K), float32 channel scales
    [N], binary16 x [M][K] -> binary16 y [M][N]."""
    torch = _torch()
    N, K = int(N), int(K)
    _req(w_packed, "w_packed", (torch.uint8,), (prepack_fp8_size(N, K),))
    _req(channel_scale, "channel_scale", (torch.float32,), (N,))
    _req(x, "x", _f16_bits_dtypes())
    M = x.shape[0]
    _req(x, "x", _f16_bits_dtypes(), (M, K))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _req(y, "y", _f16_bits_dtypes(), (M, N))
    _run("gemv_fp8_w8a16_packed", (w_packed, channel_scale, x, y), stream, _ptr(w_packed),
         _ptr(channel_scale), N, K, _ptr(x), M, _ptr(y))
    return y


def prepack_q4_k_size(N: int, K: int) -> int:
    """Bytes of the packed copy of an N x K Q4_K matrix (K % 256 == 0)."""
    n = ctypes.c_size_t(0)
    _check("prepack_q4_k_size", lib().prepack_q4_k_size(int(N), int(K), ctypes.byref(n)))
    return n.value


def prepack_q4_k(w_qs, w_hdr, w_packed=None, stream=None):
    """Planar Q4_K weights w_qs [N][K/2], w_hdr [N][K/256][16] -> the packed
    copy (uint8, prepack_q4_k_size(N, K) bytes)."""
    torch = _torch()
    _req(w_qs, "w_qs", (torch.uint8,))
    N, K2 = w_qs.shape
    K = 2 * K2
    _req(w_hdr, "w_hdr", (torch.uint8,), (N, K // 256, 16))
    nbytes = prepack_q4_k_size(N, K)
    if w_packed is None:
        w_packed = torch.empty((nbytes,), dtype=torch.uint8, device=w_qs.device)
    _req(w_packed, "w_packed", (torch.uint8,), (nbytes,))
    _run("prepack_q4_k", (w_qs, w_hdr, w_packed), stream, _ptr(w_qs), _ptr(w_hdr), N, K,
         _ptr(w_packed))
    return w_packed


def mmvq_q4_k_packed(w_packed, N, K, a_qs, a_d, a_s, y=None, stream=None):
    """Packed Q4_K weights (from prepack_q4_k, N x K) x Q8_1 activations
    -> float32 y [M][N]."""
    torch = _torch()
    N, K = int(N), int(K)
    _req(w_packed, "w_packed", (torch.uint8,), (prepack_q4_k_size(N, K),))
    _req(a_qs, "a_qs", (torch.int8,))
    M = a_qs.shape[0]
    _req(a_qs, "a_qs", (torch.int8,), (M, K))
    _req(a_d, "a_d", _f16_bits_dtypes(), (M, K // 32))
    _req(a_s, "a_s", _f16_bits_dtypes(), (M, K // 32))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=a_qs.device)
    _req(y, "y", (torch.float32,), (M, N))
    _run("mmvq_q4_k_packed", (w_packed, a_qs, a_d, a_s, y), stream, _ptr(w_packed), N, K,
         _ptr(a_qs), _ptr(a_d), _ptr(a_s), M, _ptr(y))
    return y


def prepack_iq4_xs_size(N: int, K: int) -> int:
    """Bytes of the packed copy of an N x K IQ4_XS matrix (K % 256 == 0)."""
    n = ctypes.c_size_t(0)
    _check("prepack_iq4_xs_size", lib().prepack_iq4_xs_size(int(N), int(K), ctypes.byref(n)))
    return n.value


def prepack_iq4_xs(w_qs, w_hdr, w_packed=None, stream=None):
    """Planar IQ4_XS weights w_qs [N][K/2], w_hdr [N][K/256][8] -> the packed
    copy (uint8, prepack_iq4_xs_size(N, K) bytes)."""
    torch = _torch()
    _req(w_qs, "w_qs", (torch.uint8,))
    N, K2 = w_qs.shape
    K = 2 * K2
    _req(w_hdr, "w_hdr", (torch.uint8,), (N, K // 256, 8))
    nbytes = prepack_iq4_xs_size(N, K)
    if w_packed is None:
        w_packed = torch.empty((nbytes,), dtype=torch.uint8, device=w_qs.device)
    _req(w_packed, "w_packed", (torch.uint8,), (nbytes,))
    _run("prepack_iq4_xs", (w_qs, w_hdr, w_packed), stream, _ptr(w_qs), _ptr(w_hdr), N, K,
         _ptr(w_packed))
    return w_packed


def mmvq_iq4_xs_packed(w_packed, N, K, a_qs, a_d, y=None, stream=None):
    """Packed IQ4_XS weights (from prepack_iq4_xs, N x K) x Q8_1 activations
    (codes and d8) -> float32 y [M][N]."""
    torch = _torch()
    N, K = int(N), int(K)
    _req(w_packed, "w_packed", (torch.uint8,), (prepack_iq4_xs_size(N, K),))
    _req(a_qs, "a_qs", (torch.int8,))
    M = a_qs.shape[0]
    _req(a_qs, "a_qs", (torch.int8,), (M, K))
    _req(a_d, "a_d", _f16_bits_dtypes(), (M, K // 32))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=a_qs.device)
    _req(y, "y", (torch.float32,), (M, N))
    _run("mmvq_iq4_xs_packed", (w_packed, a_qs, a_d, y), stream, _ptr(w_packed), N, K,
         _ptr(a_qs), _ptr(a_d), M, _ptr(y))
    return y


def prepack_q6_k_size(N: int, K: int) -> int:
    """Bytes of the packed copy of an N x K Q6_K matrix (K % 256 == 0)."""
    n = ctypes.c_size_t(0)
    _check("prepack_q6_k_size", lib().prepack_q6_k_size(int(N), int(K), ctypes.byref(n)))
    return n.value


def prepack_q6_k(w_ql, w_qh, w_sc, w_d, w_packed=None, stream=None):
    """Planar Q6_K weights (ql [N][K/2], qh [N][K/4], sc int8 [N][K/16], d
    binary16 [N][K/256]) -> the packed copy (uint8, prepack_q6_k_size bytes)."""
    torch = _torch()
    _req(w_ql, "w_ql", (torch.uint8,))
    N, K2 = w_ql.shape
    K = 2 * K2
    _req(w_qh, "w_qh", (torch.uint8,), (N, K // 4))
    _req(w_sc, "w_sc", (torch.int8,), (N, K // 16))
    _req(w_d, "w_d", _f16_bits_dtypes(), (N, K // 256))
    nbytes = prepack_q6_k_size(N, K)
    if w_packed is None:
        w_packed = torch.empty((nbytes,), dtype=torch.uint8, device=w_ql.device)
    _req(w_packed, "w_packed", (torch.uint8,), (nbytes,))
    _run("prepack_q6_k", (w_ql, w_qh, w_sc, w_d, w_packed), stream, _ptr(w_ql), _ptr(w_qh),
         _ptr(w_sc), _ptr(w_d), N, K, _ptr(w_packed))
    return w_packed


def mmvq_q6_k_packed(w_packed, N, K, a_qs, a_d, y=None, stream=None):
    """Packed Q6_K weights (from prepack_q6_k, N x K) x Q8_1 activations
    (codes and d8) -> float32 y [M][N]."""
    torch = _torch()
    N, K = int(N), int(K)
    _req(w_packed, "w_packed", (torch.uint8,), (prepack_q6_k_size(N, K),))
    _req(a_qs, "a_qs", (torch.int8,))
    M = a_qs.shape[0]
    _req(a_qs, "a_qs", (torch.int8,), (M, K))
    _req(a_d, "a_d", _f16_bits_dtypes(), (M, K // 32))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=a_qs.device)
    _req(y, "y", (torch.float32,), (M, N))
    _run("mmvq_q6_k_packed", (w_packed, a_qs, a_d, y), stream, _ptr(w_packed), N, K,
         _ptr(a_qs), _ptr(a_d), M, _ptr(y))
    return y
