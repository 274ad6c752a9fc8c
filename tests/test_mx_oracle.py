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


# ------------------------------------------------------------ weight gradients
def _blocks_by_hand(values, lo, hi, pad):
    """Codes and scales of one expert built block by block with the exact
    quantiser: block b of column m is rows lo + 32 b .. of column m, zeros
    past hi."""
    n = hi - lo
    P = (n + pad - 1) // pad * pad
    M = values.shape[1]
    codes = np.zeros((M, P), np.uint8)
    scales = np.zeros((M, P // 32), np.uint8)
    for m in range(M):
        for b in range(P // 32):
            blk = [values[lo + 32 * b + j, m] if 32 * b + j < n else 0.0 for j in range(32)]
            c, s = mx.mx_quantize(np.array([blk]))
            codes[m, 32 * b: 32 * b + 32] = c[0]
            scales[m, b] = s[0, 0]
    return codes, scales


def test_pad_offsets():
    np.testing.assert_array_equal(mx.mx_pad_offsets([0, 1, 64, 65, 128, 0]), [0, 0, 64, 128, 256, 384, 384])
    np.testing.assert_array_equal(mx.mx_pad_offsets([5, 40], pad=32), [0, 32, 96])


def test_expert_rows_one_expert_is_the_transposed_row_quantiser():
    rng = np.random.default_rng(31)
    v = rng.standard_normal((128, 48)) * np.exp2(rng.integers(-10, 10, (128, 48)))
    codes, scales, poff = mx.mx_quantize_expert_rows(v, [0, 128])
    rc, rs = mx.mx_quantize_fast(v.T)
    np.testing.assert_array_equal(poff, [0, 128])
    np.testing.assert_array_equal(codes, rc)
    np.testing.assert_array_equal(scales, rs)


def test_expert_rows_blocks_start_at_each_experts_first_row():
    rng = np.random.default_rng(32)
    counts = [5, 0, 40, 64, 1, 70]
    off = np.concatenate([[0], np.cumsum(counts)])
    v = rng.standard_normal((off[-1], 3)) * np.exp2(rng.integers(-6, 6, (off[-1], 1)))
    codes, scales, poff = mx.mx_quantize_expert_rows(v, off)
    for e in range(len(counts)):
        c, s = _blocks_by_hand(v, off[e], off[e + 1], 64)
        np.testing.assert_array_equal(codes[:, poff[e]:poff[e + 1]], c, err_msg=str(e))
        np.testing.assert_array_equal(scales[:, poff[e] // 32: poff[e + 1] // 32], s, err_msg=str(e))
    # a block shifted by one row (blocks counted from the start of all rows
    # instead of the expert's) gives other bytes
    shifted = _blocks_by_hand(v, off[2] - 1, off[3] - 1, 64)
    assert not np.array_equal(codes[:, poff[2]:poff[3]], shifted[0])


def test_expert_rows_depend_only_on_their_own_rows():
    rng = np.random.default_rng(33)
    off = np.array([0, 30, 100, 101])
    v = rng.standard_normal((101, 8))
    c0, s0, poff = mx.mx_quantize_expert_rows(v, off)
    w = v.copy()
    w[30:100] *= 1000.0
    c1, s1, _ = mx.mx_quantize_expert_rows(w, off)
    keep = np.r_[poff[0]:poff[1], poff[2]:poff[3]]
    np.testing.assert_array_equal(c0[:, keep], c1[:, keep])
    np.testing.assert_array_equal(s0[:, keep[::32] // 32], s1[:, keep[::32] // 32])
    assert not np.array_equal(s0[:, poff[1] // 32: poff[2] // 32], s1[:, poff[1] // 32: poff[2] // 32])


def test_padding_rows_are_zero_codes_and_an_empty_block_takes_scale_zero():
    v = np.full((3, 4), 5.0)
    codes, scales, poff = mx.mx_quantize_expert_rows(v, [0, 3])
    assert codes.shape == (4, 64) and scales.shape == (4, 2)
    assert np.all(codes[:, 3:] == 0) and np.all(scales[:, 1] == 0)
    assert np.all(scales[:, 0] == 127 + 2 - 8)             # floor(log2 5) - 8
    assert np.all(mx.mx_dequantize(codes, scales)[:, :3] == 5.0)


def _small_ints(rng, shape):
    """Integers in [-8, 8]: with any block maximum among them, every element
    times 2^-scale is an E4M3 value, so quantisation is exact."""
    return rng.integers(-8, 9, shape).astype(np.float64)


@pytest.mark.parametrize("seed", range(2))
def test_wgrad_equals_the_exact_product_on_representable_values(seed):
    rng = np.random.default_rng(40 + seed)
    counts = [37, 0, 64, 100]
    off = np.concatenate([[0], np.cumsum(counts)])
    R, D, F = int(off[-1]), 32, 48
    x = _small_ints(rng, (R, D)) * 2.0 ** -7
    dh = _small_ints(rng, (R, F)) * 2.0 ** 5
    xc, xs, poff = mx.mx_quantize_expert_rows(x, off)
    hc, hs, _ = mx.mx_quantize_expert_rows(dh, off)
    np.testing.assert_array_equal(mx.mx_dequantize(xc, xs)[:, poff[0]:poff[0] + 37], x[:37].T)
    for e, dw in mx.mx_wgrad(xc, xs, hc, hs, poff):
        lo, hi = off[e], off[e + 1]
        want = x[lo:hi].T @ dh[lo:hi]                        # exact: small dyadic integers
        assert dw.shape == (D, F)
        np.testing.assert_array_equal(dw, want, err_msg=str(e))
    # planted mistakes: blocks of another expert, or the operands swapped
    bad = poff.copy()
    bad[2:] += 32
    bad[-1] = min(bad[-1], xc.shape[1])
    assert not np.array_equal(dict(mx.mx_wgrad(xc, xs, hc, hs, bad))[2], x[off[2]:off[3]].T @ dh[off[2]:off[3]])
    assert dict(mx.mx_wgrad(hc, hs, xc, xs, poff))[0].shape == (F, D)


def test_wgrad_within_the_quantisation_bound_on_gaussian_rows():
    rng = np.random.default_rng(44)
    off = np.array([0, 150])
    a, b = rng.standard_normal((150, 16)), rng.standard_normal((150, 16))
    ac, as_, poff = mx.mx_quantize_expert_rows(a, off)
    bc, bs, _ = mx.mx_quantize_expert_rows(b, off)
    dw = dict(mx.mx_wgrad(ac, as_, bc, bs, poff))[0]
    exact = a.T @ b

    def elem_bound(v, sc):
        # half an E4M3 step: 2^-4 relative for normals, 2^-10 of the block
        # scale for subnormals
        x = np.repeat(2.0 ** (sc.astype(np.int64) - 127), 32, axis=1)[:, :150].T
        return np.abs(v) * 2.0 ** -4 + x * 2.0 ** -10

    ea, eb = elem_bound(a, as_), elem_bound(b, bs)
    bound = ea.T @ np.abs(b) + np.abs(a).T @ eb + ea.T @ eb
    assert np.all(np.abs(dw - exact) <= bound * (1 + 1e-12))


def test_act_p_f32():
    h = np.array([[2.0 ** -3, -1.0, -0.0, 0.0, 3.0]], np.float32)
    p = np.array([0.25], np.float32)
    a = mx.act_p_f32(h, p)
    np.testing.assert_array_equal(a, [[2.0 ** -8, 0.0, 0.0, 0.0, 2.25]])
    assert not np.any(np.signbit(a))                         # relu gives +0
    rng = np.random.default_rng(45)
    h = rng.standard_normal((64, 32)).astype(np.float32)
    p = rng.uniform(0.01, 1.0, 64).astype(np.float32)
    a = mx.act_p_f32(h, p).astype(np.float64)
    exact = p.astype(np.float64)[:, None] * np.maximum(h.astype(np.float64), 0.0) ** 2
    assert np.all(np.abs(a - exact) <= exact * 2.0 ** -23)   # two float32 roundings
    assert a.dtype == np.float64 and mx.act_p_f32(h, p).dtype == np.float32


def test_act_p_f32_squares_before_scaling():
    """The order of the two roundings is fixed (it decides codes): r * r
    first, then times p; find inputs where the other order differs."""
    rng = np.random.default_rng(46)
    h = rng.uniform(0.5, 2.0, 4096).astype(np.float32)
    p = rng.uniform(0.1, 1.0, 4096).astype(np.float32)
    other = (p * h) * h
    a = mx.act_p_f32(h.reshape(-1, 1), p)[:, 0]
    differ = a != other
    assert differ.any()
    r64 = h.astype(np.float64) ** 2
    sq = r64.astype(np.float32).astype(np.float64)             # r * r rounded once
    np.testing.assert_array_equal(a, (sq * p.astype(np.float64)).astype(np.float32))
