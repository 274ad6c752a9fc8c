"""Plain CPU definition of MXFP8 block quantisation (E4M3 elements, E8M0
scales), the encoded form whose values and scale buffers the pages fingerprint.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: French article, section "Méthodologie de débogage du
non-déterminisme": for MXFP8 and NVFP4 the encoded values and the scale
buffers are fingerprinted.  The pages do not define the format; it is taken
from the published OCP Microscaling Formats (MX) Specification v1.0:
  * a block is 32 consecutive elements of a row; its shared scale is
    X = 2^(floor(log2(max |V_i|)) - emax_elem), emax_elem = 8 for E4M3
    (largest normal 1.75 * 2^8 = 448), stored as an E8M0 byte
    (biased exponent, bias 127); the exponent is clamped to [-127, 127]
    (an all-zero block takes the smallest scale, byte 0);
  * each element is V_i / X rounded to E4M3 (1 sign, 4 exponent bits with
    bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN)
    to nearest, ties to the even code, and saturated at +-448; the sign is
    kept, so -0 and negative values that round to zero encode as -0 (0x80).
Non-finite inputs are outside the definition.  Arithmetic is exact
(fractions / exact binary widening), and the rounding is done by choosing
the nearest of the enumerated E4M3 values, so it can be checked by eye.
"""
import bisect
from fractions import Fraction

import numpy as np

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_decode(code: int) -> float:
    """Value of an E4M3 code (NaN for S.1111.111)."""
    code = int(code)
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# the non-negative finite codes and their values, in increasing value order
_POS = sorted((e4m3_decode(c), c) for c in range(0x7F))
_POS_VALUES = [Fraction(v) for v, _ in _POS]


def e4m3_encode(a: Fraction, negative: bool) -> int:
    """E4M3 code of sign * a for the exact magnitude a >= 0: the nearest
    representable magnitude (ties to the even code), saturated at 448; the
    sign is kept (so -0 and negative values that round to zero give 0x80)."""
    sign = 0x80 if negative else 0
    if a >= Fraction(E4M3_MAX):
        return sign | 0x7E
    i = bisect.bisect_left(_POS_VALUES, a)        # _POS_VALUES[i-1] < a <= _POS_VALUES[i]
    cands = [j for j in (i - 1, i) if 0 <= j < len(_POS)]
    best = min(cands, key=lambda j: (abs(_POS_VALUES[j] - a), _POS[j][1] & 1))
    return sign | _POS[best][1]


def e8m0_decode(byte: int) -> float:
    return float("nan") if byte == 0xFF else 2.0 ** (byte - 127)


def shared_exponent(block) -> int:
    """floor(log2(max |v|)) - 8, clamped to [-127, 127]; -127 for an all-zero block."""
    amax = max(abs(Fraction(float(v))) for v in block)
    if amax == 0:
        return -127
    e = amax.numerator.bit_length() - amax.denominator.bit_length()
    if Fraction(2) ** e > amax:        # make 2^e <= amax < 2^(e+1)
        e -= 1
    return max(-127, min(127, e - 8))


def mx_quantize(rows: np.ndarray):
    """rows: float64 array [n, k] with k a multiple of 32 (exact values of the
    input).  Returns (codes uint8 [n, k], scales uint8 [n, k/32])."""
    rows = np.asarray(rows, np.float64)
    n, k = rows.shape
    assert k % BLOCK == 0
    codes = np.zeros((n, k), np.uint8)
    scales = np.zeros((n, k // BLOCK), np.uint8)
    for i in range(n):
        for b in range(k // BLOCK):
            blk = rows[i, b * BLOCK:(b + 1) * BLOCK]
            se = shared_exponent(blk)
            scales[i, b] = se + 127
            x = Fraction(2) ** se
            for j, v in enumerate(blk):
                codes[i, b * BLOCK + j] = e4m3_encode(abs(Fraction(float(v))) / x, bool(np.signbit(v)))
    return codes, scales


_DECODE = np.array([e4m3_decode(c) for c in range(256)])
_POS_F64 = np.array([v for v, _ in _POS])            # increasing magnitudes of codes 0..126
_POS_CODE = np.array([c for _, c in _POS], np.uint8)


def mx_quantize_fast(rows: np.ndarray):
    """mx_quantize in vectorised float64 (same definition, for large tensors;
    pinned against mx_quantize).  Exactness: v * 2^-se is a power-of-two scaling
    of a float32 value (exact in float64), and the two candidate magnitudes
    around it lie within a factor of two of it, so their distances to it are
    exact float64 differences."""
    rows = np.asarray(rows, np.float64)
    n, k = rows.shape
    assert k % BLOCK == 0
    blocks = rows.reshape(n, k // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=2)
    _, ex = np.frexp(amax)                           # amax = m * 2^ex, m in [0.5, 1)
    se = np.where(amax > 0, np.clip(ex - 1 - 8, -127, 127), -127).astype(np.int64)
    y = np.ldexp(np.abs(blocks), -se[:, :, None])
    i = np.searchsorted(_POS_F64, y, side="left")    # _POS_F64[i-1] < y <= _POS_F64[i]
    lo = np.clip(i - 1, 0, len(_POS_F64) - 1)
    hi = np.clip(i, 0, len(_POS_F64) - 1)
    dlo, dhi = y - _POS_F64[lo], _POS_F64[hi] - y
    clo, chi = _POS_CODE[lo], _POS_CODE[hi]
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (chi % 2 == 0) & (clo % 2 == 1))
    code = np.where(pick_hi, chi, clo)
    code = np.where(y >= E4M3_MAX, np.uint8(0x7E), code)
    code = code | np.where(np.signbit(blocks), np.uint8(0x80), np.uint8(0))
    return code.reshape(n, k).astype(np.uint8), (se + 127).astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values X * P_i as float64: the code's value times its block's scale
    (codes [..., k], scales [..., k/32])."""
    codes = np.asarray(codes, np.uint8)
    x = np.exp2(np.asarray(scales, np.float64) - 127.0)
    return _DECODE[codes] * np.repeat(x, BLOCK, axis=-1)


def mx_grouped_rows(a_codes, a_scales, b_codes, b_scales, offsets) -> np.ndarray:
    """out[r] = dequant(A)[r] . dequant(B_e)^T for the rows r of group e
    (offsets[e] <= r < offsets[e+1]); A [rows, K], B [groups, N, K]."""
    A = mx_dequantize(a_codes, a_scales)
    out = np.zeros((A.shape[0], b_codes.shape[1]))
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi] = A[lo:hi] @ mx_dequantize(b_codes[e], b_scales[e]).T
    return out
