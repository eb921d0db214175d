"""INT8 storage for an 8-bit KV cache (oracle side), the second 8-bit format beside E4M3.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name 8-bit KV caches (TurboMind's "8bit KV Cache" quantisation in the
AIGC interview book's LMDeploy section, its "8-bit integer quantisation" note, and
the linear INT8 mapping the same book discusses for deployment) but fix no format.
The reading taken for the integer variant: symmetric linear quantisation with one
float32 scale per cache (keys and values each), value = code * scale, codes the
signed integers -127 .. 127 stored as two's-complement bytes (the symmetric range,
so that negating a value negates its code; the byte 0x80 = -128 is never written
but decodes as -128).

Quantisation of a new key or value element x (stored in the model's 16-bit type):
y = x / scale in float32 (correctly rounded), then the nearest integer, ties to
even, clamped to [-127, 127]; a NaN element is written as code 0.
"""
from __future__ import annotations

import numpy as np

I8_MAX = 127


def i8_decode(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of INT8 codes (uint8 bytes, two's complement)."""
    b = np.asarray(bits).astype(np.int64)
    return np.where(b >= 128, b - 256, b).astype(np.float64)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """INT8 codes (as uint8 bytes) of x / scale: the division in float32, rounded to the nearest
    integer with ties to even, clamped to +-127; NaN gives 0."""
    y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    nan = np.isnan(y)
    q = np.clip(np.rint(np.where(nan, np.float32(0), y)), -I8_MAX, I8_MAX).astype(np.int64)
    return (q & 0xFF).astype(np.uint8)
