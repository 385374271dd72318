"""Exact decoding of storage elements to float64 (oracle; test infrastructure only).

The kernels store K, V, q and out as binary32, binary16 or bfloat16 and accumulate in
binary32; the oracle widens every stored element to float64 exactly, so rounding of the
inputs is never counted as kernel error.

binary16 (IEEE 754): 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0
encodes zero and subnormals (fraction * 2^-24), exponent 31 encodes inf / NaN.
bfloat16: the upper 16 bits of a binary32 (1 sign, 8 exponent bits with bias 127, 7 fraction
bits), so it widens by shifting its bits 16 places left.
"""
from __future__ import annotations

import numpy as np


def decode_bits_f16(bits) -> np.ndarray:
    """binary16 bit patterns (uint16) -> float64, from the field definitions."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    exp = (b >> 10) & 0x1F
    frac = (b & 0x3FF).astype(np.float64)
    normal = sign * np.ldexp(1.0 + frac / 1024.0, (exp - 15).astype(np.int64))
    sub = sign * np.ldexp(frac, -24)
    special = np.where(frac == 0, sign * np.inf, np.nan)
    return np.where(exp == 0, sub, np.where(exp == 31, special, normal))


def decode_bits_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: place the bits in the top half of a
    binary32 and widen."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode(arr, dtype: str) -> np.ndarray:
    """Storage array (float32 / float16 / uint16-for-bf16) -> float64, exactly."""
    arr = np.asarray(arr)
    if dtype == "f32":
        assert arr.dtype == np.float32
        return arr.astype(np.float64)
    if dtype == "f16":
        assert arr.dtype in (np.float16, np.uint16)
        return decode_bits_f16(arr.view(np.uint16))
    if dtype == "bf16":
        assert arr.dtype in (np.uint16, np.int16)
        return decode_bits_bf16(arr.view(np.uint16))
    raise ValueError(dtype)
