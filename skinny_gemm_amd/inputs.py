"""Seeded synthetic inputs for the quantized skinny-GEMV path.

This module only draws random numbers and stores them in the byte layouts the
library takes.  It holds none of the method's arithmetic: no quantizer, no
decode, no dot product.  Format encodings it needs to *produce* weights
(binary16 and E4M3 rounding of drawn reals) are library casts (numpy's
float16, torch's float8_e4m3fn), after clamping to the finite E4M3 range.
Both the GPU tests and the oracle side take their inputs from here.

Distributions (one per workload):
  * Q4_0 weights: 4-bit codes uniform over 0..15 (a uniform random byte is
    two independent uniform codes), scales d ~ U[0.002, 0.02] rounded to
    binary16.
  * Q8_1 source activations: float32 N(0, 1), one independent row per M.
  * NVFP4 weights: E2M1 codes uniform over all 16 code points (uniform
    bytes), one E4M3 scale per 16 elements with scale = e4m3(u / 6),
    u ~ U[0.01, 0.1], so the largest decodable magnitude 6 * scale spans
    U[0.01, 0.1]; per-tensor scale 1.0.
  * FP8 weights: E4M3 of N(0, 0.05) (clamped to +-448, round to nearest
    even); per-output-channel float32 scales ~ U[0.5, 2].
  * binary16 activations: N(0, 1) drawn in float64, rounded to binary16.
  * Q4_K weights: uniform random bytes for the 4-bit codes and for the 12
    packed scale/min bytes of each super-block (every 6-bit field uniform
    over 0..63); d and dmin ~ U[6.2e-5, 2e-4] rounded to binary16.
  * Q6_K weights: uniform random bytes for the low and high code bits (codes
    uniform over 0..63) and for the int8 sub-block scales; d ~ U[6.2e-5,
    2e-4] rounded to binary16.
  * IQ4_XS weights: uniform random bytes for the 4-bit table indices and for
    the 6 packed scale bytes of each super-block (every 6-bit scale uniform
    over 0..63); d ~ U[6.2e-5, 2e-4] rounded to binary16.

Seeds: ``seed(config, shape, tensor)`` = 1000*config + 10*shape + tensor,
tensor 0 = codes/weights, 1 = scales, 2 = activations.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def seed(config: int, shape: int, tensor: int) -> int:
    return 1000 * int(config) + 10 * int(shape) + int(tensor)


def _rng(s: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(s)))


def _e4m3_bytes(v: np.ndarray) -> np.ndarray:
    """Round reals to E4M3 (torch's round-to-nearest-even cast) after
    clamping to the finite range, returned as raw bytes."""
    import torch

    v = np.clip(np.asarray(v, np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


# ---------------------------------------------------------------- host (numpy)

def q4_0_weights(N: int, K: int, base_seed: int):
    """-> (w_qs uint8 [N][K/2], w_d uint16 [N][K/32] binary16 bits)."""
    w_qs = _rng(base_seed + 0).integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    d = _rng(base_seed + 1).uniform(0.002, 0.02, size=(N, K // 32))
    w_d = d.astype(np.float16).view(np.uint16)
    return w_qs, w_d


def normal_f32(M: int, K: int, s: int) -> np.ndarray:
    return _rng(s).standard_normal(size=(M, K), dtype=np.float32)


def normal_f16_bits(M: int, K: int, s: int, std: float = 1.0) -> np.ndarray:
    x = _rng(s).standard_normal(size=(M, K)) * std
    return x.astype(np.float16).view(np.uint16)


def nvfp4_weights(N: int, K: int, base_seed: int, global_scale: float = 1.0):
    """-> (codes uint8 [N][K/2], scales uint8 E4M3 [N][K/16], g float)."""
    codes = _rng(base_seed + 0).integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    u = _rng(base_seed + 1).uniform(0.01, 0.1, size=(N, K // 16))
    scales = _e4m3_bytes(u / 6.0)
    return codes, scales, float(global_scale)


def fp8_weights(N: int, K: int, base_seed: int):
    """-> (w uint8 E4M3 [N][K], cs float32 [N])."""
    w = _e4m3_bytes(_rng(base_seed + 0).normal(0.0, 0.05, size=(N, K)))
    cs = _rng(base_seed + 1).uniform(0.5, 2.0, size=(N,)).astype(np.float32)
    return w, cs


def q4_k_weights(N: int, K: int, base_seed: int):
    """-> (w_qs uint8 [N][K/2], w_hdr uint8 [N][K/256][16]: binary16 d and
    dmin in bytes 0-3, then 12 packed scale/min bytes)."""
    ns = K // 256
    w_qs = _rng(base_seed + 0).integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    r = _rng(base_seed + 1)
    hdr = np.empty((N, ns, 16), np.uint8)
    dd = r.uniform(6.2e-5, 2e-4, size=(N, ns, 2)).astype(np.float16)
    hdr[:, :, 0:4] = dd.view(np.uint8).reshape(N, ns, 4)
    hdr[:, :, 4:16] = r.integers(0, 256, size=(N, ns, 12), dtype=np.uint8)
    return w_qs, hdr


def q6_k_weights(N: int, K: int, base_seed: int):
    """-> (w_ql uint8 [N][K/2], w_qh uint8 [N][K/4], w_sc int8 [N][K/16],
    w_d uint16 [N][K/256] binary16 bits)."""
    r = _rng(base_seed + 0)
    w_ql = r.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    w_qh = r.integers(0, 256, size=(N, K // 4), dtype=np.uint8)
    r = _rng(base_seed + 1)
    w_sc = r.integers(-128, 128, size=(N, K // 16)).astype(np.int8)
    w_d = r.uniform(6.2e-5, 2e-4, size=(N, K // 256)).astype(np.float16).view(np.uint16)
    return w_ql, w_qh, w_sc, w_d


def iq4_xs_weights(N: int, K: int, base_seed: int):
    """-> (w_qs uint8 [N][K/2], w_hdr uint8 [N][K/256][8]: binary16 d in
    bytes 0-1, then 6 bytes of packed sub-block scale bits)."""
    ns = K // 256
    w_qs = _rng(base_seed + 0).integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    r = _rng(base_seed + 1)
    hdr = np.empty((N, ns, 8), np.uint8)
    d = r.uniform(6.2e-5, 2e-4, size=(N, ns)).astype(np.float16)
    hdr[:, :, 0:2] = d.view(np.uint8).reshape(N, ns, 2)
    hdr[:, :, 2:8] = r.integers(0, 256, size=(N, ns, 6), dtype=np.uint8)
    return w_qs, hdr


def q8_1_unit_scale_source(M: int, K: int, s: int, spread: int = 60) -> np.ndarray:
    """float32 integer-valued activations for the exact-integer gate.

    Every 32-block holds one entry of +-127 and 31 entries in [-spread,
    spread] (spread <= 60), so its Q8_1 scale is exactly 1, its codes equal
    the inputs, and the code sum (|sum| <= 127 + 31*60 = 1987) is an integer
    binary16 holds exactly.
    """
    assert 0 <= spread <= 60
    r = _rng(s)
    x = r.integers(-spread, spread + 1, size=(M, K)).astype(np.float32)
    nb = K // 32
    pos = r.integers(0, 32, size=(M, nb))
    sign = np.where(r.integers(0, 2, size=(M, nb)) == 0, -127.0, 127.0)
    rows = np.repeat(np.arange(M), nb)
    cols = (np.tile(np.arange(nb), M) * 32 + pos.ravel())
    x[rows, cols] = sign.ravel()
    return x


# ---------------------------------------------------------------- device (torch)

def q4_0_weights_torch(N: int, K: int, base_seed: int, device):
    """Device-side draw with the same distributions as ``q4_0_weights`` (a
    different stream of numbers), for weight sets too large to draw on the
    host.  -> (w_qs uint8 [N][K/2], w_d int16 [N][K/32] binary16 bits)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(base_seed))
    w_qs = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=device, generator=g)
    u = torch.rand((N, K // 32), dtype=torch.float32, device=device, generator=g)
    w_d = (0.002 + 0.018 * u).to(torch.float16).view(torch.int16)
    return w_qs, w_d


def q4_k_weights_torch(N: int, K: int, base_seed: int, device):
    """Device-side draw with the distributions of ``q4_k_weights``.
    -> (w_qs uint8 [N][K/2], w_hdr uint8 [N][K/256][16])."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(base_seed))
    ns = K // 256
    w_qs = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=device, generator=g)
    hdr = torch.randint(0, 256, (N, ns, 16), dtype=torch.uint8, device=device, generator=g)
    u = torch.rand((N, ns, 2), dtype=torch.float32, device=device, generator=g)
    dd = (6.2e-5 + 1.38e-4 * u).to(torch.float16)
    hdr[:, :, 0:4] = dd.view(torch.uint8).reshape(N, ns, 4)
    return w_qs, hdr


def q6_k_weights_torch(N: int, K: int, base_seed: int, device):
    """Device-side draw with the distributions of ``q6_k_weights``.
    -> (w_ql uint8 [N][K/2], w_qh uint8 [N][K/4], w_sc int8 [N][K/16],
    w_d int16 [N][K/256] binary16 bits)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(base_seed))
    w_ql = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=device, generator=g)
    w_qh = torch.randint(0, 256, (N, K // 4), dtype=torch.uint8, device=device, generator=g)
    w_sc = torch.randint(-128, 128, (N, K // 16), dtype=torch.int8, device=device, generator=g)
    u = torch.rand((N, K // 256), dtype=torch.float32, device=device, generator=g)
    w_d = (6.2e-5 + 1.38e-4 * u).to(torch.float16).view(torch.int16)
    return w_ql, w_qh, w_sc, w_d


def iq4_xs_weights_torch(N: int, K: int, base_seed: int, device):
    """Device-side draw with the distributions of ``iq4_xs_weights``.
    -> (w_qs uint8 [N][K/2], w_hdr uint8 [N][K/256][8])."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(base_seed))
    ns = K // 256
    w_qs = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=device, generator=g)
    hdr = torch.randint(0, 256, (N, ns, 8), dtype=torch.uint8, device=device, generator=g)
    u = torch.rand((N, ns), dtype=torch.float32, device=device, generator=g)
    d = (6.2e-5 + 1.38e-4 * u).to(torch.float16)
    hdr[:, :, 0:2] = d.view(torch.uint8).reshape(N, ns, 2)
    return w_qs, hdr


def normal_f32_torch(M: int, K: int, s: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(s))
    return torch.randn((M, K), dtype=torch.float32, device=device, generator=g)


def nvfp4_weights_torch(N: int, K: int, base_seed: int, device):
    """Device-side draw with the distributions of ``nvfp4_weights``.
    -> (codes uint8 [N][K/2], scales uint8 E4M3 [N][K/16])."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(base_seed))
    codes = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=device, generator=g)
    u = 0.01 + 0.09 * torch.rand((N, K // 16), dtype=torch.float32, device=device, generator=g)
    scales = (u / 6.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scales


def fp8_weights_torch(N: int, K: int, base_seed: int, device):
    """Device-side draw with the distributions of ``fp8_weights``.
    -> (w uint8 E4M3 [N][K], cs float32 [N])."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(base_seed))
    w = torch.randn((N, K), dtype=torch.float32, device=device, generator=g) * 0.05
    w = w.clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    cs = 0.5 + 1.5 * torch.rand((N,), dtype=torch.float32, device=device, generator=g)
    return w, cs


def normal_f16_torch(M: int, K: int, s: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(s))
    return torch.randn((M, K), dtype=torch.float32, device=device, generator=g).to(torch.float16)
