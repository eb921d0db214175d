"""FP8 E4M3 storage for an 8-bit KV cache (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name 8-bit KV caches (TurboMind's "8bit KV Cache" quantisation in the
AIGC interview book's LMDeploy section; FP8 among SGLang's quantisations) but
fix no format.  The reading taken: the OCP 8-bit floating-point format E4M3
(the one MI355X converts in hardware), one float32 scale per cache (keys and
values each), value = decode(code) * scale.

E4M3, from its definition: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
bits; exponent field 0 encodes subnormals m/8 * 2^-6; the all-ones pattern
S.1111.111 is NaN; there are no infinities, so the largest finite value is
1.75 * 2^8 = 448.

Quantisation of a new key or value element x (stored in the model's 16-bit
type): y = x / scale in float32 (correctly rounded), clamped to [-448, 448],
then rounded to the nearest E4M3 value, ties to even mantissa.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of E4M3 codes (uint8)."""
    b = np.asarray(bits).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    out = sign * mag
    return np.where((e == 15) & ((b & 7) == 7), np.nan, out)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code (ties to even) of values already within [-448, 448] (NaN -> NaN code)."""
    y = np.asarray(y, dtype=np.float64)
    nan = np.isnan(y)
    a = np.where(nan, 0.0, np.abs(y))
    assert np.all(a <= E4M3_MAX), "clamp before encoding"
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9; q == 8 is the smallest normal, whose code is also 8
    q_sub = np.rint(a / 2.0 ** -9).astype(np.int64)
    # normal range: a = 2^e (1 + f), f in [0, 1): mantissa = rint(8 f), a carry moves to e + 1
    e = np.floor(np.log2(np.where(sub, 1.0, a))).astype(np.int64)
    # guard the floor(log2) of values a hair below a power of two
    e = np.where(np.exp2(e.astype(np.float64)) > a, e - 1, e)
    e = np.where(np.exp2((e + 1).astype(np.float64)) <= a, e + 1, e)
    q = np.rint((a / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    code_norm = ((e + 7) << 3) | q
    code = np.where(sub, q_sub, code_norm)
    code = code | np.where(np.signbit(y) & ~nan, 0x80, 0)
    return np.where(nan, E4M3_NAN, code).astype(np.uint8)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes of x / scale: the division in float32, clamped to +-448, ties to even."""
    y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y)
