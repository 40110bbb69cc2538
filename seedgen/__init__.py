"""Seeded synthetic inputs for the attention path and its fp64 oracle.

This module is the only code shared by the GPU path's tests/benchmark and the
CPU oracle. It holds no attention arithmetic: it draws i.i.d. Gaussian numbers
from a counter-based generator and rounds them to the storage dtype.

Recipe (one stream per (seed, tensor_id)):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the k-th 64-bit word of the stream is
  ``mix(key + (k + 1) * 0x9E3779B97F4A7C15)`` with ``key = seed * 2**32 + tensor_id``
  and ``mix`` the published finaliser (xor-shift 30/27/31 with multipliers
  0xBF58476D1CE4E5B9 and 0x94D049BB133111EB).
* Box-Muller (1958): words 2i and 2i+1 give ``u1 = (w >> 11 + 1) * 2**-53`` in
  (0, 1] and ``u2 = (w >> 11) * 2**-53`` in [0, 1); element 2i is
  ``sqrt(-2 ln u1) cos(2 pi u2)``, element 2i+1 the same with ``sin``.
* The fp64 value is multiplied by ``mul`` (1.0, or 0.5 for the 64K-token
  wide-head workload), rounded to fp32 (round to nearest even) and then to the
  storage dtype with round to nearest even (bf16 by the integer carry trick,
  fp16 by numpy's IEEE conversion).

Both sides receive the same stored bits: the GPU gets the bf16/fp16/fp32 tensor,
the oracle gets exactly those values widened to fp64.

Tensor ids: q=0, k=1, v=2, dO=3; 16 and up are free for test-local draws
(row samples, perturbations).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "splitmix64_words", "uniform01", "normal_f64", "round_f32_to_bf16_bits",
    "bf16_bits_to_f64", "draw", "Drawn", "TENSOR_Q", "TENSOR_K", "TENSOR_V",
    "TENSOR_DO", "choice_rows",
]

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO = 0, 1, 2, 3

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _key(seed: int, tensor_id: int) -> np.uint64:
    return np.uint64(((int(seed) << 32) + int(tensor_id)) & 0xFFFFFFFFFFFFFFFF)


def splitmix64_words(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of the SplitMix64 stream keyed by (seed, tensor_id)."""
    k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = _key(seed, tensor_id) + k * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, tensor_id: int, count: int) -> np.ndarray:
    """``count`` doubles in [0, 1) with 53 random bits each."""
    w = splitmix64_words(seed, tensor_id, 0, count)
    return (w >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal_f64(seed: int, tensor_id: int, count: int) -> np.ndarray:
    """``count`` standard normal doubles by Box-Muller over the SplitMix64 stream."""
    out = np.empty(count, dtype=np.float64)
    npairs = (count + 1) // 2
    for p0 in range(0, npairs, _CHUNK):
        p1 = min(npairs, p0 + _CHUNK)
        w = splitmix64_words(seed, tensor_id, 2 * p0, 2 * (p1 - p0))
        u1 = ((w[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
        u2 = (w[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        r = np.sqrt(-2.0 * np.log(u1))
        t = (2.0 * np.pi) * u2
        pair = np.empty(2 * (p1 - p0), dtype=np.float64)
        pair[0::2] = r * np.cos(t)
        pair[1::2] = r * np.sin(t)
        n = min(count - 2 * p0, pair.size)
        out[2 * p0: 2 * p0 + n] = pair[:n]
    return out


def round_f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even. No NaN inputs."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _e4m3_positive_values() -> np.ndarray:
    """Values of the e4m3 (OCP, 'fn') codes 0x00 .. 0x7E, increasing: 3 mantissa
    bits, exponent bias 7, subnormals below 2^-6, largest finite 448."""
    codes = np.arange(0x7F)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3 = _e4m3_positive_values()


def round_f32_to_e4m3_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> e4m3 codes (uint8), round to nearest, ties to the even code.
    Magnitudes above 448 (the largest finite value) are rejected."""
    x = np.asarray(x32, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 448.0) or np.any(np.isnan(a)):
        raise ValueError("value outside the e4m3 range")
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 1, 0x7E)
    lo = hi - 1
    dlo, dhi = a - _E4M3[lo], _E4M3[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == 0, 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of finite e4m3 codes to fp64."""
    b = np.asarray(bits, dtype=np.uint8)
    v = _E4M3[np.minimum(b & 0x7F, 0x7E)]
    return np.where(b & 0x80, -v, v)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


class Drawn:
    """A drawn tensor: ``stored`` holds the storage bits (uint16 for bf16/fp16,
    uint8 for fp8e4m3, float32 for fp32) and ``f64`` the same values widened
    exactly to fp64."""

    __slots__ = ("dtype", "shape", "stored", "f64")

    def __init__(self, dtype: str, shape, stored: np.ndarray, f64: np.ndarray):
        self.dtype, self.shape, self.stored, self.f64 = dtype, tuple(shape), stored, f64

    def torch(self, device="cpu"):
        """The stored values as a torch tensor of the storage dtype."""
        import torch
        if self.dtype == "bf16":
            t = torch.from_numpy(self.stored.view(np.int16).copy()).view(torch.bfloat16)
        elif self.dtype == "fp16":
            t = torch.from_numpy(self.stored.view(np.int16).copy()).view(torch.float16)
        elif self.dtype == "fp8e4m3":
            t = torch.from_numpy(self.stored.copy())  # the bytes, as uint8
        else:
            t = torch.from_numpy(self.stored.copy())
        return t.reshape(self.shape).to(device)


def draw(seed: int, tensor_id: int, shape, dtype: str, mul: float = 1.0,
         want_f64: bool = True) -> Drawn:
    """i.i.d. ``mul * N(0,1)`` values of ``shape``, stored as ``dtype`` in {bf16, fp16, fp32, fp8e4m3}."""
    count = int(np.prod(shape)) if len(shape) else 1
    x = normal_f64(seed, tensor_id, count)
    if mul != 1.0:
        x *= mul
    x32 = x.astype(np.float32)
    del x
    if dtype == "bf16":
        stored = round_f32_to_bf16_bits(x32)
        f64 = bf16_bits_to_f64(stored) if want_f64 else None
    elif dtype == "fp16":
        h = x32.astype(np.float16)
        stored = h.view(np.uint16)
        f64 = h.astype(np.float64) if want_f64 else None
    elif dtype == "fp32":
        stored = x32
        f64 = x32.astype(np.float64) if want_f64 else None
    elif dtype == "fp8e4m3":
        stored = round_f32_to_e4m3_bits(x32)
        f64 = e4m3_bits_to_f64(stored) if want_f64 else None
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    stored = stored.reshape(shape)
    if f64 is not None:
        f64 = f64.reshape(shape)
    return Drawn(dtype, shape, stored, f64)


def choice_rows(seed: int, tensor_id: int, n: int, count: int) -> np.ndarray:
    """``count`` distinct integers in [0, n), sorted, drawn from the seeded stream."""
    if count > n:
        raise ValueError("count > n")
    picked: list[int] = []
    seen = set()
    start = 0
    while len(picked) < count:
        w = splitmix64_words(seed, tensor_id, start, 4 * count)
        start += 4 * count
        for x in (w % np.uint64(n)).tolist():
            if x not in seen:
                seen.add(x)
                picked.append(x)
                if len(picked) == count:
                    break
    return np.array(sorted(picked), dtype=np.int64)


TENSOR_MASK = 8


def block_mask(seed: int, tensor_id: int, shape, density: float) -> np.ndarray:
    """uint8 array of ``shape`` whose entries are 1 with probability ``density``
    (independently, from the seeded stream) and 0 otherwise: a block mask for
    block-sparse attention."""
    n = int(np.prod(shape))
    return (uniform01(seed, tensor_id, n) < density).astype(np.uint8).reshape(shape)


TENSOR_LENS = 9


def lengths(seed: int, tensor_id: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` sequence lengths, independent and uniform over [lo, hi], from the
    seeded stream (int32): the length mix of a padded batch."""
    if not 0 <= lo <= hi:
        raise ValueError("need 0 <= lo <= hi")
    u = uniform01(seed, tensor_id, count)
    return np.minimum(lo + np.floor(u * (hi - lo + 1)).astype(np.int64), hi).astype(np.int32)
