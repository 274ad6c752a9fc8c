"""Plain CPU definition of NVFP4 block quantisation (E2M1 elements, an E4M3
scale per 16 elements, an fp32 per-tensor scale), the second low-precision
form whose encoded values and scale buffers the pages fingerprint.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: French article, section "Méthodologie de débogage du
non-déterminisme": for MXFP8 and NVFP4 the encoded values and the scale
buffers are fingerprinted.  The pages do not define the format; this reading
follows NVIDIA's public description of NVFP4:
  * E2M1 elements: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit;
    magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN;
  * a block is 16 consecutive elements of a row, with one E4M3 scale;
  * a float32 scale for the whole tensor places the block scales in E4M3's
    range: g = amax / (6 * 448) (1 for an all-zero tensor).
The decisions are taken in float32 steps, written out here so that a kernel
can take the same ones (where float arithmetic decides a code, both sides
decide in the same precision):
  g  = f32(amax) / 2688                       (1 if that is 0: an all-zero
                                              tensor, or one so small that
                                              g underflows)
  t  = f32(6 * g);  x = f32(amax_b / t)       block scale code sb = E4M3(x)
  d  = f32(value(sb) * g)                     element code = E2M1(f32(v / d))
                                              (0 codes, sign kept, if d == 0)
Each E4M3 / E2M1 encoding picks the nearest value exactly (ties to the even
code) and saturates at 448 / 6.  Two element codes share a byte, the even
element in the low nibble.  Non-finite inputs are outside the definition.
"""
import bisect
from fractions import Fraction

import numpy as np

from .mx import e4m3_decode, e4m3_encode

BLOCK = 16
E2M1_MAX = 6.0


def e2m1_decode(code: int) -> float:
    """Value of a 4-bit E2M1 code."""
    code = int(code)
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * 0.5 * m
    return s * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


_POS = sorted((e2m1_decode(c), c) for c in range(8))
_POS_VALUES = [Fraction(v) for v, _ in _POS]


def e2m1_encode(a: Fraction, negative: bool) -> int:
    """E2M1 code of sign * a for the exact magnitude a >= 0: the nearest value
    (ties to the even code), saturated at 6; the sign is kept."""
    sign = 0x8 if negative else 0
    if a >= Fraction(E2M1_MAX):
        return sign | 0x7
    i = bisect.bisect_left(_POS_VALUES, a)
    cands = [j for j in (i - 1, i) if 0 <= j < len(_POS)]
    best = min(cands, key=lambda j: (abs(_POS_VALUES[j] - a), _POS[j][1] & 1))
    return sign | _POS[best][1]


def nvfp4_quantize(rows: np.ndarray):
    """rows: float32 array [n, k], k a multiple of 16.  Returns (packed codes
    uint8 [n, k/2], block scales uint8 [n, k/16], per-tensor scale float32)."""
    rows = np.asarray(rows, np.float32)
    n, k = rows.shape
    assert k % BLOCK == 0
    f32 = np.float32
    amax = f32(np.max(np.abs(rows))) if rows.size else f32(0)
    g = f32(amax / f32(2688.0))
    if not g > 0:
        g = f32(1.0)
    t = f32(f32(6.0) * g)
    codes = np.zeros((n, k), np.uint8)
    scales = np.zeros((n, k // BLOCK), np.uint8)
    for i in range(n):
        for b in range(k // BLOCK):
            blk = rows[i, b * BLOCK:(b + 1) * BLOCK]
            x = f32(f32(np.max(np.abs(blk))) / t)
            sb = e4m3_encode(Fraction(float(x)), False)
            scales[i, b] = sb
            d = f32(f32(e4m3_decode(sb)) * g)
            for j, v in enumerate(blk):
                neg = bool(np.signbit(v))
                y = f32(abs(v) / d) if d != 0 else f32(0.0)
                codes[i, b * BLOCK + j] = e2m1_encode(Fraction(float(y)), neg)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales, g


def nvfp4_dequantize(packed: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """Values E2M1(code) * E4M3(block scale) * g as float64."""
    packed = np.asarray(packed, np.uint8)
    n, h = packed.shape
    codes = np.zeros((n, 2 * h), np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    vals = np.vectorize(e2m1_decode)(codes)
    s = np.vectorize(e4m3_decode)(np.asarray(scales, np.uint8))
    return vals * np.repeat(s, BLOCK, axis=1) * float(g)
