"""Counter-based random numbers shared by every consumer of synthetic inputs.

Everything here is a pure function of (seed, index), so any element of any
tensor can be regenerated on its own: the host side (this file, numpy) and
the device fill kernel (``synth/csrc/fill.hip``) implement the same published
definitions and agree bit for bit.

* SplitMix64 (Steele, Lea and Flood, "Fast Splittable Pseudorandom Number
  Generators", OOPSLA 2014; output mixer as in Vigna's public-domain
  ``splitmix64.c``): draw ``i`` of stream ``seed`` is
  ``mix(seed + (i + 1) * 0x9E3779B97F4A7C15)`` with
  ``mix(z) = z ^ (z >> 31)`` after ``z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9``
  and ``z = (z ^ (z >> 27)) * 0x94D049BB133111EB`` (all mod 2**64).
* Normal(0, sigma): a 4-term Irwin-Hall sum of the draw's four 16-bit lanes,
  centred and scaled to standard deviation sigma:
  ``x = float32(2 * sum(u16) - 262140) * float32(sigma * sqrt(3) / 2**17)``.
  The integer is exact in fp32 and the product is one IEEE multiply, so host
  and device agree.  bf16 tensors then round that fp32 value to nearest-even.
* Uniform [0, 1): ``(draw >> 11) * 2**-53``.

This module holds no part of the N-gram method's arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
MIX1 = np.uint64(0xBF58476D1CE4E5B9)
MIX2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1


def _mix(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * MIX1
        z = (z ^ (z >> np.uint64(27))) * MIX2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, idx) -> np.ndarray:
    """Draw(s) ``idx`` (int or integer array) of the SplitMix64 stream ``seed``."""
    i = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & _MASK64) + (i + np.uint64(1)) * GOLDEN_GAMMA
    return _mix(z)


def splitmix64_int(seed: int, idx: int) -> int:
    """Scalar pure-Python SplitMix64 draw (for seeds and constants)."""
    z = (seed + (idx + 1) * 0x9E3779B97F4A7C15) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def sub_seed(seed: int, *path: int) -> int:
    """Derive an independent stream seed from ``seed`` and a path of ints."""
    s = seed & _MASK64
    for p in path:
        s = splitmix64_int(s, p)
    return s


def uniform01(seed: int, idx) -> np.ndarray:
    d = splitmix64(seed, idx)
    return (d >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal_scale(sigma: float) -> np.float32:
    """fp32 multiplier that turns the centred Irwin-Hall integer into N(0, sigma)."""
    return np.float32(sigma * math.sqrt(3.0) / 131072.0)


def normal_f32(seed: int, idx, sigma: float) -> np.ndarray:
    d = splitmix64(seed, idx)
    m = np.uint64(0xFFFF)
    s = ((d & m) + ((d >> np.uint64(16)) & m) + ((d >> np.uint64(32)) & m)
         + (d >> np.uint64(48))).astype(np.int64)
    centred = (2 * s - 262140).astype(np.float32)
    return (centred * normal_scale(sigma)).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite (the generators never produce inf/nan)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to OCP FP8 E4M3 (nearest, ties to even); uint8 codes.  Uses
    torch's float8_e4m3fn conversion; inputs stay within +-448."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def normal_values(seed: int, idx, sigma: float, dtype: str, inv_scale: float = 1.0) -> np.ndarray:
    """Normal draws stored as ``dtype``: 'f32' -> float32, 'bf16' -> uint16 bits,
    'fp8' -> uint8 E4M3 codes of draw * inv_scale (one fp32 multiply)."""
    x = normal_f32(seed, idx, sigma)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp8":
        return f32_to_fp8_e4m3_bits(x * np.float32(inv_scale))
    raise ValueError(f"unknown dtype {dtype!r}")
