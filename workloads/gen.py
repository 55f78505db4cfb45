"""Counter-based, exactly reproducible pseudo-normal values.

Every element of every synthetic tensor is a pure function of
(seed, stream, flat index).  The same integer recipe runs on the host (NumPy)
and on the device (torch integer ops), and both produce bit-identical values,
so a multi-GB pool can be generated in HBM while the host regenerates any
slice of it for a check.

Recipe (all arithmetic on unsigned 32-bit words held in int64):
  * mix32(x): xor-shift / multiply finaliser
        x ^= x >> 16; x = x * 0x7FEB352D mod 2^32; x ^= x >> 15;
        x = x * 0x5BD1E995 mod 2^32; x ^= x >> 16
    Both multipliers are below 2^31, so no int64 product overflows.
  * For element i (lo = i mod 2^32, hi = i >> 32) and word r in {0,1,2}:
        w_r = mix32(mix32(lo ^ k_r) ^ ((hi * 0x27D4EB2F + k_r) mod 2^32))
    where k_r = key_for(seed, stream, r) is fixed per tensor.
  * S = sum of the 12 bytes of (w_0, w_1, w_2), S in [0, 3060].
  * value = (S - 1530) / 256.
The value is the Irwin-Hall approximation of N(0, 1) (sum of twelve uniforms
minus their mean): mean 0, variance 65535/65536, support [-5.98, 5.98].  It is
a multiple of 1/256 with |numerator| <= 1530 < 2^11, so it is exact in fp16,
fp32 and fp64 alike; no rounding ever differs between host and device.

Full-mantissa variant (full_values*): a fourth word w_3 adds a 24-bit
perturbation u = w_3 >> 8 below the 1/256 grid,
  value = ((S - 1530) * 2^24 + (u - 2^23)) / 2^32,
an integer over a power of two, exact in fp64 (|numerator| < 2^35).  Cast to
fp32 it rounds once (to nearest even), so almost every value uses all 24
mantissa bits and is NOT representable in fp16; host and device round the same
exact fp64 number and agree bit for bit.  Used for fp32 batches, so that an
fp32 path that silently went through fp16 would be seen.
"""

from __future__ import annotations

import numpy as np

M32 = 0xFFFFFFFF
_C1 = 0x7FEB352D
_C2 = 0x5BD1E995
_C3 = 0x27D4EB2F


def _mix32_py(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * _C1) & M32
    x ^= x >> 15
    x = (x * _C2) & M32
    x ^= x >> 16
    return x


def key_for(seed: int, stream: int, r: int) -> int:
    """Per-tensor key for word r; distinct (seed, stream, r) give distinct streams."""
    k = _mix32_py(seed * 0x9E3779B1 + 0x632BE5AB)
    k = _mix32_py(k ^ (stream * 0x85EBCA77 + 0x165667B1))
    k = _mix32_py(k ^ (r * 0xC2B2AE3D + 0x27D4EB2F))
    return k


def _mix32_np(x):
    x = x ^ (x >> 16)
    x = (x * _C1) & M32
    x = x ^ (x >> 15)
    x = (x * _C2) & M32
    x = x ^ (x >> 16)
    return x


def _byte_sum_np(w):
    t = (w & 0x00FF00FF) + ((w >> 8) & 0x00FF00FF)
    return (t & 0xFFFF) + (t >> 16)


def normal_values(seed: int, stream: int, index, dtype=np.float32):
    """Values at the given flat indices (int64 array-like) as `dtype` (exact)."""
    idx = np.asarray(index, dtype=np.int64)
    lo = idx & M32
    hi = idx >> 32
    s = np.zeros(idx.shape, dtype=np.int64)
    for r in range(3):
        k = key_for(seed, stream, r)
        w = _mix32_np(_mix32_np(lo ^ k) ^ ((hi * _C3 + k) & M32))
        s += _byte_sum_np(w)
    out = (s - 1530).astype(np.float64) / 256.0
    return out.astype(dtype)


def full_values(seed: int, stream: int, index, dtype=np.float32):
    """Full-mantissa values at the given flat indices: the normal value plus a 24-bit
    perturbation in [-2^-9, 2^-9), as an exact fp64 number rounded once to `dtype`."""
    idx = np.asarray(index, dtype=np.int64)
    lo = idx & M32
    hi = idx >> 32
    s = np.zeros(idx.shape, dtype=np.int64)
    for r in range(3):
        k = key_for(seed, stream, r)
        w = _mix32_np(_mix32_np(lo ^ k) ^ ((hi * _C3 + k) & M32))
        s += _byte_sum_np(w)
    k = key_for(seed, stream, 3)
    u = _mix32_np(_mix32_np(lo ^ k) ^ ((hi * _C3 + k) & M32)) >> 8
    num = (s - 1530) * (1 << 24) + (u - (1 << 23))
    out = num.astype(np.float64) / float(1 << 32)
    return out.astype(dtype)


def normal_array(seed: int, stream: int, shape, dtype=np.float32, offset: int = 0,
                 chunk: int = 1 << 22, full: bool = False):
    """A whole array of the given shape; element i has flat index offset + i.  full=True takes
    the full-mantissa variant."""
    fn = full_values if full else normal_values
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=dtype)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        out[a:b] = fn(seed, stream, np.arange(offset + a, offset + b, dtype=np.int64), dtype)
    return out.reshape(shape)


def _mix32_t(x):
    x = x ^ (x >> 16)
    x = (x * _C1) & M32
    x = x ^ (x >> 15)
    x = (x * _C2) & M32
    x = x ^ (x >> 16)
    return x


def _byte_sum_t(w):
    t = (w & 0x00FF00FF) + ((w >> 8) & 0x00FF00FF)
    return (t & 0xFFFF) + (t >> 16)


def values_at_torch(seed: int, stream: int, idx, full: bool = False):
    """The values at the flat indices `idx` (an int64 torch tensor on any device) as an exact
    float64 tensor: normal_values() (full=True: full_values()) computed with torch ops, which
    is faster on the host than NumPy for large index sets."""
    import torch

    lo = idx & M32
    hi = idx >> 32
    s = torch.zeros_like(idx)
    for r in range(3):
        k = key_for(seed, stream, r)
        w = _mix32_t(_mix32_t(lo ^ k) ^ ((hi * _C3 + k) & M32))
        s += _byte_sum_t(w)
    if not full:
        return (s - 1530).to(torch.float64) / 256.0
    k = key_for(seed, stream, 3)
    u = _mix32_t(_mix32_t(lo ^ k) ^ ((hi * _C3 + k) & M32)) >> 8
    return ((s - 1530) * (1 << 24) + (u - (1 << 23))).to(torch.float64) / float(1 << 32)


def normal_values_torch(seed: int, stream: int, out, offset: int = 0, chunk: int = 1 << 28,
                        full: bool = False):
    """Fill the contiguous torch tensor `out` (any float dtype, any device) in place.

    Element i of `out.view(-1)` receives the value for flat index offset + i, the
    same number normal_values() (full=True: full_values()) gives on the host.
    """
    import torch

    flat = out.view(-1)
    n = flat.numel()
    keys = [key_for(seed, stream, r) for r in range(3)]
    k3 = key_for(seed, stream, 3)
    if full:
        chunk = min(chunk, 1 << 26)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        idx = torch.arange(offset + a, offset + b, dtype=torch.int64, device=flat.device)
        lo = idx & M32
        hi = idx >> 32
        s = torch.zeros_like(idx)
        for k in keys:
            w = _mix32_t(_mix32_t(lo ^ k) ^ ((hi * _C3 + k) & M32))
            s += _byte_sum_t(w)
        if full:
            u = _mix32_t(_mix32_t(lo ^ k3) ^ ((hi * _C3 + k3) & M32)) >> 8
            num = (s - 1530) * (1 << 24) + (u - (1 << 23))
            del u
            flat[a:b] = (num.to(torch.float64) / float(1 << 32)).to(flat.dtype)
            del num
        else:
            flat[a:b] = ((s - 1530).to(torch.float32) / 256.0).to(flat.dtype)
        del idx, lo, hi, s
    return out
