"""Pins of the MXFP8 quantisation oracle against facts that do not come from
the oracle itself: the E4M3 and E8M0 code points that the OCP Microscaling
(MX) Specification v1.0 fixes, an exhaustive round trip and an exhaustive
ties-to-even check over every pair of neighbouring codes, saturation, the
shared-scale rule worked by hand, and a brute-force nearest-code search."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import mx


def test_e4m3_code_points_fixed_by_the_format():
    assert mx.e4m3_decode(0x7E) == 448.0              # largest normal, 1.75 * 2^8
    assert mx.e4m3_decode(0x08) == 2.0 ** -6          # smallest normal
    assert mx.e4m3_decode(0x01) == 2.0 ** -9          # smallest subnormal
    assert mx.e4m3_decode(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert mx.e4m3_decode(0x38) == 1.0                # exponent field 7 = bias
    assert np.isnan(mx.e4m3_decode(0x7F)) and np.isnan(mx.e4m3_decode(0xFF))
    assert mx.e4m3_decode(0x00) == 0.0 and np.signbit(mx.e4m3_decode(0x80))
    vals = [mx.e4m3_decode(c) for c in range(256) if c not in (0x7F, 0xFF)]
    assert len(set(vals)) == 253                      # 254 codes, +0 and -0 equal
    assert mx.e8m0_decode(127) == 1.0 and mx.e8m0_decode(0) == 2.0 ** -127 and np.isnan(mx.e8m0_decode(255))


def test_every_finite_code_round_trips():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        v = mx.e4m3_decode(c)
        assert mx.e4m3_encode(abs(Fraction(v)), bool(np.signbit(v))) == c, hex(c)


def test_midpoints_round_to_the_even_code():
    pos = sorted((mx.e4m3_decode(c), c) for c in range(0x7F))
    for (v0, c0), (v1, c1) in zip(pos, pos[1:]):
        mid = (Fraction(v0) + Fraction(v1)) / 2
        want = c0 if c0 % 2 == 0 else c1
        assert mx.e4m3_encode(mid, False) == want
        eps = Fraction(1, 1 << 40)
        assert mx.e4m3_encode(mid - eps, False) == c0 and mx.e4m3_encode(mid + eps, False) == c1


def test_saturation_at_448():
    assert mx.e4m3_encode(Fraction(463), False) == 0x7E            # below the 448/480 midpoint
    assert mx.e4m3_encode(Fraction(464), False) == 0x7E            # the midpoint: 448 has the even code
    assert mx.e4m3_encode(Fraction(500), True) == 0xFE
    assert mx.e4m3_encode(Fraction(10 ** 9), False) == 0x7E


def test_shared_scale_rule_by_hand():
    blk = np.zeros(32)
    blk[3] = 1.0                                       # amax = 1: exponent 0, shared 0 - 8
    codes, scales = mx.mx_quantize(blk[None, :])
    assert scales[0, 0] == 127 - 8
    assert codes[0, 3] == mx.e4m3_encode(Fraction(256), False) == 0x78     # 1 / 2^-8 = 256 = 1.0 * 2^8
    blk[5] = -1.9375                                   # amax in [1, 2): same exponent; 1.9375 * 256 = 496 saturates
    codes, scales = mx.mx_quantize(blk[None, :])
    assert scales[0, 0] == 119 and codes[0, 5] == 0xFE
    codes, scales = mx.mx_quantize(np.zeros((1, 32)))
    assert scales[0, 0] == 0 and not codes.any()
    tiny = np.full((1, 32), 2.0 ** -140)               # the exponent clamps at -127
    codes, scales = mx.mx_quantize(tiny)
    assert scales[0, 0] == 0 and codes[0, 0] == mx.e4m3_encode(Fraction(2) ** -13, False)


def _brute(block):
    amax = np.max(np.abs(block))
    se = -127 if amax == 0 else max(-127, min(127, int(np.floor(np.log2(amax))) - 8))
    x = 2.0 ** se
    out = []
    for v in block:
        best = None
        for c in range(256):
            if c in (0x7F, 0xFF):
                continue
            d = abs(mx.e4m3_decode(c) * x - v)
            if np.signbit(mx.e4m3_decode(c)) != np.signbit(v) and mx.e4m3_decode(c) == 0:
                continue
            key = (d, c & 1, c)
            if best is None or key < best[0]:
                best = (key, c)
        out.append(best[1])
    return se + 127, out


@pytest.mark.parametrize("seed", range(3))
def test_against_a_brute_force_search(seed):
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((4, 64)) * np.exp(rng.uniform(-20, 20, (4, 1)))
    rows[0, :32] = np.round(rows[0, :32] * 8) / 8      # some exact values and ties
    codes, scales = mx.mx_quantize(rows)
    for i in range(4):
        for b in range(2):
            s, cs = _brute(rows[i, 32 * b:32 * b + 32])
            assert scales[i, b] == s
            # the brute force clamps nothing, so compare where |V/X| < 448
            x = 2.0 ** (s - 127)
            for j, c in enumerate(cs):
                if abs(rows[i, 32 * b + j]) / x < 448:
                    assert codes[i, 32 * b + j] == c


def test_dequantised_error_within_half_an_e4m3_step():
    rng = np.random.default_rng(9)
    rows = rng.standard_normal((8, 128))
    codes, scales = mx.mx_quantize(rows)
    back = mx.mx_dequantize(codes, scales)
    x = np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)
    y = np.abs(rows) / x
    ok = (y < 448) & (y >= 2.0 ** -6)                  # normal, unsaturated
    assert np.all(np.abs(back - rows)[ok] <= np.abs(rows)[ok] * 2.0 ** -4)


def test_pins_catch_planted_mistakes(monkeypatch):
    blk = np.zeros((1, 32))
    blk[0, 0] = 1.0
    base = mx.shared_exponent
    monkeypatch.setattr(mx, "shared_exponent", lambda b: base(b) + 1)   # emax 7 instead of 8
    assert mx.mx_quantize(blk)[1][0, 0] != 127 - 8
    monkeypatch.setattr(mx, "shared_exponent", base)
    pos = sorted((mx.e4m3_decode(c), c) for c in range(0x7F))
    (v0, c0), (v1, c1) = pos[40], pos[41]
    mid = (Fraction(v0) + Fraction(v1)) / 2
    away = max(c0, c1)                                  # ties away from zero
    assert mx.e4m3_encode(mid, False) != away or away % 2 == 0


def test_vectorised_dequantise_equals_the_definition():
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    scales = np.array([[0], [1], [100], [126], [127], [128], [200], [254]], np.uint8)
    got = mx.mx_dequantize(codes, scales)
    for i in range(8):
        for j in range(32):
            want = mx.e4m3_decode(int(codes[i, j])) * mx.e8m0_decode(int(scales[i, 0]))
            assert (np.isnan(want) and np.isnan(got[i, j])) or got[i, j] == want


def test_grouped_rows_against_a_triple_loop():
    rng = np.random.default_rng(2)
    K, N = 64, 3
    a = rng.standard_normal((5, K))
    b = rng.standard_normal((2, N, K))
    ac, asc = mx.mx_quantize(a)
    bc, bsc = mx.mx_quantize(b.reshape(-1, K))
    bc, bsc = bc.reshape(2, N, K), bsc.reshape(2, N, K // 32)
    offsets = [0, 2, 5]
    out = mx.mx_grouped_rows(ac, asc, bc, bsc, offsets)
    for r in range(5):
        e = 0 if r < 2 else 1
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += (mx.e4m3_decode(int(ac[r, k])) * mx.e8m0_decode(int(asc[r, k // 32]))
                      * mx.e4m3_decode(int(bc[e, n, k])) * mx.e8m0_decode(int(bsc[e, n, k // 32])))
            assert abs(out[r, n] - s) <= 1e-12 * max(1.0, abs(s))


@pytest.mark.parametrize("seed", range(3))
def test_vectorised_quantise_equals_the_exact_one(seed):
    rng = np.random.default_rng(100 + seed)
    rows = (rng.standard_normal((16, 128)) * np.exp2(rng.uniform(-40, 40, (16, 1)))).astype(np.float32)
    pos = sorted(mx.e4m3_decode(c) for c in range(0x7F))
    mids = np.array([(u + v) / 2 for u, v in zip(pos, pos[1:])], np.float32)
    rows[0, :32] = mids[-32:] * np.float32(2.0 ** -8)
    rows[1, :32] = mids[:32] * np.float32(2.0 ** -8)
    rows[2, :32] = -0.0
    rows[3, :32] = np.float32(1.96875)
    rows[4, :32] = np.float32(2.0 ** -149)
    a, b = mx.mx_quantize(rows.astype(np.float64)), mx.mx_quantize_fast(rows.astype(np.float64))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
