"""Pins of the NVFP4 quantisation oracle against facts that do not come from
the oracle itself: the E2M1 code points, an exhaustive round trip and
ties-to-even check, saturation, a block worked by hand, a brute-force
nearest-code search over every E2M1 and E4M3 code, and the dequantisation
error bound."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import mx, nvfp4


def test_e2m1_code_points():
    assert [nvfp4.e2m1_decode(c) for c in range(8)] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [nvfp4.e2m1_decode(c) for c in range(9, 16)] == [-0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert nvfp4.e2m1_decode(8) == 0.0 and np.signbit(nvfp4.e2m1_decode(8))


def test_round_trip_and_ties_to_even():
    for c in range(16):
        v = nvfp4.e2m1_decode(c)
        assert nvfp4.e2m1_encode(abs(Fraction(v)), bool(np.signbit(v))) == c
    pos = [(nvfp4.e2m1_decode(c), c) for c in range(8)]
    for (v0, c0), (v1, c1) in zip(pos, pos[1:]):
        mid = (Fraction(v0) + Fraction(v1)) / 2
        assert nvfp4.e2m1_encode(mid, False) == (c0 if c0 % 2 == 0 else c1)
        eps = Fraction(1, 1 << 30)
        assert nvfp4.e2m1_encode(mid - eps, False) == c0 and nvfp4.e2m1_encode(mid + eps, False) == c1


def test_saturation():
    assert nvfp4.e2m1_encode(Fraction(5), False) == 0x6           # midpoint of 4 and 6: 4 has the even code
    assert nvfp4.e2m1_encode(Fraction(7), False) == 0x7
    assert nvfp4.e2m1_encode(Fraction(10 ** 6), True) == 0xF


def test_a_block_worked_by_hand():
    # amax 2688 = 6 * 448 gives g = 1; block amax 2688 gives x = 2688 / 6 =
    # 448, the E4M3 code 0x7E; d = 448 and each element is v / 448
    row = np.zeros((1, 16), np.float32)
    row[0, :6] = [2688.0, 448.0, -672.0, 224.0, 1120.0, 0.0]      # 6, 1, -1.5, 0.5, 2.5 -> 2 (even), 0
    packed, scales, g = nvfp4.nvfp4_quantize(row)
    assert g == np.float32(1.0) and scales[0, 0] == 0x7E
    codes = [(packed[0, i // 2] >> (4 * (i % 2))) & 0xF for i in range(6)]
    assert codes == [0x7, 0x2, 0xB, 0x1, 0x4, 0x0]
    # a second block of the same row with amax 3: x = 3 / 6 = 0.5 (E4M3 0x30)
    row2 = np.zeros((1, 32), np.float32)
    row2[0, :16] = row[0]
    row2[0, 16:18] = [3.0, -0.75]                                 # d = 0.5: 6 and -1.5
    packed, scales, g = nvfp4.nvfp4_quantize(row2)
    assert scales[0, 1] == 0x30 and mx.e4m3_decode(0x30) == 0.5
    assert packed[0, 8] == (0x7 | (0xB << 4))
    zero = nvfp4.nvfp4_quantize(np.zeros((2, 16), np.float32))
    assert zero[2] == np.float32(1.0) and not zero[0].any() and not zero[1].any()
    # a tensor whose scale amax / 2688 underflows: g = 1, and every code and
    # scale is zero (the sign bits kept)
    tiny = np.full((1, 16), np.float32(2.0 ** -140))
    tiny[0, 1] = -tiny[0, 1]
    t = nvfp4.nvfp4_quantize(tiny)
    assert t[2] == np.float32(1.0) and not t[1].any() and t[0][0, 0] == 0x80


def _brute(rows):
    """Same float32 steps, encoders replaced by a scan over every code."""
    f32 = np.float32
    amax = f32(np.max(np.abs(rows)))
    g = f32(amax / f32(2688.0))
    g = g if g > 0 else f32(1.0)
    t = f32(f32(6.0) * g)
    e4 = [(mx.e4m3_decode(c), c) for c in range(0x7F)]
    e2 = [(nvfp4.e2m1_decode(c), c) for c in range(8)]
    out_c, out_s = [], []
    for blk in rows.reshape(-1, 16):
        x = float(f32(f32(np.max(np.abs(blk))) / t))
        sb = min(e4, key=lambda vc: (abs(vc[0] - x), vc[1] & 1))[1] if x < 448 else 0x7E
        d = f32(f32(mx.e4m3_decode(sb)) * g)
        out_s.append(sb)
        for v in blk:
            y = float(f32(abs(v) / d)) if d != 0 else 0.0
            c = min(e2, key=lambda vc: (abs(vc[0] - y), vc[1] & 1))[1] if y < 6 else 0x7
            out_c.append(c | (0x8 if np.signbit(v) else 0))
    return np.array(out_c, np.uint8), np.array(out_s, np.uint8), g


@pytest.mark.parametrize("seed", range(3))
def test_against_a_brute_force_search(seed):
    rng = np.random.default_rng(seed)
    rows = (rng.standard_normal((4, 64)) * np.exp2(rng.uniform(-12, 12, (4, 1)))).astype(np.float32)
    rows[0, :16] = np.round(rows[0, :16] * 4) / 4
    packed, scales, g = nvfp4.nvfp4_quantize(rows)
    bc, bs, bg = _brute(rows)
    codes = np.zeros((4, 64), np.uint8)
    codes[:, 0::2], codes[:, 1::2] = packed & 0xF, packed >> 4
    assert g == bg
    np.testing.assert_array_equal(scales.ravel(), bs)
    np.testing.assert_array_equal(codes.ravel(), bc)


def test_dequantised_error_bound():
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((8, 64)).astype(np.float32)
    packed, scales, g = nvfp4.nvfp4_quantize(rows)
    back = nvfp4.nvfp4_dequantize(packed, scales, g)
    d = np.repeat(np.vectorize(mx.e4m3_decode)(scales), 16, axis=1) * float(g)
    # the widest gap between E2M1 magnitudes is 2 (4 to 6): error <= d,
    # and <= d / 4 where |v| / d <= 2 (gaps of 0.5)
    err = np.abs(back - rows)
    assert np.all(err <= d * (1 + 1e-6))
    small = np.abs(rows) / d <= 2
    assert np.all(err[small] <= d[small] * (0.25 + 1e-6))


def test_pins_catch_planted_mistakes(monkeypatch):
    base = nvfp4.e2m1_encode
    monkeypatch.setattr(nvfp4, "e2m1_encode",
                        lambda a, neg: base(a + Fraction(1, 1 << 20), neg))   # ties away from zero
    row = np.zeros((1, 16), np.float32)
    row[0, :2] = [2688.0, 1120.0]                                 # 2.5: the tie 2 / 3
    packed, _, _ = nvfp4.nvfp4_quantize(row)
    assert (packed[0, 0] >> 4) != 0x4
