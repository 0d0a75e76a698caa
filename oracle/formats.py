"""Exact decoders from storage formats to float64 (oracle; test infrastructure only).

Each decoder follows the format's published bit layout and is exact: every
fp16, bf16 and e4m3fn value is representable in float64.

* IEEE binary16: numpy's own float16 type.
* bfloat16: the upper 16 bits of an IEEE binary32.
* OCP 8-bit e4m3fn ("FP8 E4M3" in the GBSA article, "quantisation" section):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals when the
  exponent field is 0, no infinities, and S.1111.111 is NaN.
"""
from __future__ import annotations

import numpy as np


def f16_to_f64(bits_or_half: np.ndarray) -> np.ndarray:
    a = np.asarray(bits_or_half)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    assert a.dtype == np.float16
    return a.astype(np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 given as its uint16 bit pattern."""
    b = np.asarray(bits)
    assert b.dtype == np.uint16
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP e4m3fn given as uint8 bit patterns, decoded field by field."""
    b = np.asarray(bits)
    assert b.dtype == np.uint8
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    exp = ((b >> 3) & 0xF).astype(np.int64)
    man = (b & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + man / 8.0, exp - 7)
    subnormal = sign * np.ldexp(man / 8.0, -6)
    out = np.where(exp == 0, subnormal, normal)
    nan = (exp == 0xF) & ((b & 0x7) == 0x7)
    return np.where(nan, np.nan, out)


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f16_to_f64(x)
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "fp8":
        return e4m3fn_to_f64(x)
    raise ValueError(dtype)
