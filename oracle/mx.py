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


# ------------------------------------------------------------ weight gradients
# The weight gradients contract over the routed rows of one expert,
#   dW1_e = X_e^T dH_e   and   dW2_e = A_e^T dY_e,   A = p relu(h)^2,
# where X_e and dY_e are the rows of the expert's tokens.  A block scale
# factors out of a product only if it is constant along the contraction, so
# these four operands are quantised along the rows: a block is 32
# consecutive routed rows of one expert in one column, the first block
# starting at the expert's first row and the last one completed with zero
# rows.  The pages name the format only; this layout is the reading of this
# library.  Each expert's rows are laid out in a multiple of MXW_PAD rows
# (two blocks: one 64-element step of the scaled product), zero past its
# count.

MXW_PAD = 64


def mx_pad_offsets(counts, pad: int = MXW_PAD) -> np.ndarray:
    """First padded row of each expert (and the total at the end): the row
    counts rounded up to a multiple of ``pad``, prefix-summed."""
    c = np.asarray(counts, np.int64)
    padded = (c + pad - 1) // pad * pad
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)


def mx_quantize_expert_rows(values: np.ndarray, offsets, pad: int = MXW_PAD):
    """MXFP8 of each expert's rows along the row axis.

    values: float64 [R, M], the exact input values of the routed rows,
    expert-major (rows offsets[e]..offsets[e+1] belong to expert e).
    Returns (codes uint8 [M, P], scales uint8 [M, P/32], poff): column j of
    expert e's range poff[e] <= j < poff[e+1] holds its routed row
    offsets[e] + (j - poff[e]), transposed; columns past its count are zero
    rows (code 0; a block of them alone takes scale byte 0)."""
    values = np.asarray(values, np.float64)
    offsets = np.asarray(offsets, np.int64)
    M = values.shape[1]
    poff = mx_pad_offsets(np.diff(offsets), pad)
    P = int(poff[-1])
    codes = np.zeros((M, P), np.uint8)
    scales = np.zeros((M, P // BLOCK), np.uint8)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        p0, p1 = int(poff[e]), int(poff[e + 1])
        if p1 == p0:
            continue
        block = np.zeros((M, p1 - p0))
        block[:, : hi - lo] = values[lo:hi].T
        c, s = mx_quantize_fast(block)
        codes[:, p0:p1] = c
        scales[:, p0 // BLOCK: p1 // BLOCK] = s
    return codes, scales, poff


def act_p_f32(h, p) -> np.ndarray:
    """p * relu(h)^2 as the weight-gradient quantiser forms it, in float32:
    r = h where h > 0, else +0; then r * r and that times p, each product
    rounded to float32 (p: one routing weight per row, h [rows, F])."""
    h = np.asarray(h, np.float32)
    p = np.asarray(p, np.float32).reshape(-1, 1)
    r = np.where(h > 0, h, np.float32(0.0)).astype(np.float32)
    return (p * (r * r)).astype(np.float32)


def mx_wgrad(a_codes, a_scales, b_codes, b_scales, poff, experts=None):
    """Yields (e, dW_e) with dW_e = dequant(A_e) dequant(B_e)^T in float64,
    A_e / B_e the columns poff[e]..poff[e+1] of the row-quantised operands
    ([M, P] and [N, P]); an expert without rows gets zeros."""
    poff = np.asarray(poff, np.int64)
    M, N = a_codes.shape[0], b_codes.shape[0]
    for e in (range(len(poff) - 1) if experts is None else experts):
        p0, p1 = int(poff[e]), int(poff[e + 1])
        if p1 == p0:
            yield e, np.zeros((M, N))
            continue
        a = mx_dequantize(a_codes[:, p0:p1], a_scales[:, p0 // BLOCK: p1 // BLOCK])
        b = mx_dequantize(b_codes[:, p0:p1], b_scales[:, p0 // BLOCK: p1 // BLOCK])
        yield e, a @ b.T
