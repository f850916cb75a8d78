"""Comparison helpers shared by the tests (no method arithmetic here)."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_lines(name: str):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line


def f32_from_bits(u) -> np.ndarray:
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def bits_from_f32(f) -> np.ndarray:
    return np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)


def bf16_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_ordinal(b) -> np.ndarray:
    """Map bf16 bit patterns to integers that are monotone in value, with
    +0 and -0 both at 0, so |ord(a) - ord(b)| counts bf16 ulps between a, b."""
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_diff(a, b) -> np.ndarray:
    return np.abs(bf16_ordinal(a) - bf16_ordinal(b))


def f32_ulp(x) -> np.ndarray:
    """Spacing of fp32 numbers at |x| (x normal)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 23)
