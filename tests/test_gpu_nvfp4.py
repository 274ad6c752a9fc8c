"""NVFP4 quantisation (moe_nvfp4_quantize) against the CPU oracle, byte for
byte: packed E2M1 codes, E4M3 block scales and the float32 tensor scale, on
random rows across many binades, constructed E2M1 and E4M3 ties, bf16 input,
zero and underflowing tensors; and bit-identical under shuffled launch
orders."""
import numpy as np
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
import oracle
from synth.inputs import f32_to_bf16_bits, bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def _check(rows_f32, dev_tensor):
    c, s, g = moe.moe_nvfp4_quantize(dev_tensor)
    torch.cuda.synchronize()
    rc, rs, rg = oracle.nvfp4_quantize(rows_f32)
    assert np.float32(g.item()) == rg
    np.testing.assert_array_equal(s.cpu().numpy().reshape(rs.shape), rs)
    np.testing.assert_array_equal(c.cpu().numpy().reshape(rc.shape), rc)


def _ties():
    """Tensor scale 1 (amax 2688); block 0 amax 2688 (d = 448) holding every
    E2M1 midpoint and value times 448; further blocks whose amax / 6 is an
    E4M3 midpoint."""
    rows = np.zeros((4, 64), np.float32)
    e2 = sorted(oracle.e2m1_decode(c) for c in range(8))
    mids = [(a + b) / 2 for a, b in zip(e2, e2[1:])]
    vals = [6.0] + mids + e2[1:8]
    rows[0, :15] = np.array(vals[:15], np.float32) * 448
    rows[0, 1::2] *= -1
    e4 = sorted(oracle.e4m3_decode(c) for c in range(0x7F))
    e4m = [(a + b) / 2 for a, b in zip(e4, e4[1:])]
    picks = np.array(e4m[::8][:12], np.float64)
    for b, m in enumerate(picks):
        r, c0 = 1 + b // 4, 16 * (b % 4)
        rows[r, c0] = np.float32(6 * m)
        rows[r, c0 + 1:c0 + 16] = np.float32(6 * m) * np.linspace(-1, 1, 15, dtype=np.float32)
    rows[3, 63] = 2688.0
    return rows


@pytest.mark.parametrize("case", ["binades", "near_binades", "ties", "zero", "tiny", "subnormal_g"])
def test_nvfp4_f32_bytes_equal_the_oracle(case):
    """binades: row scales over 60 binades (rows far below the tensor amax
    get block scale 0); near_binades: row scales within 2^12 of the tensor
    amax, so every row reaches the E2M1 encoder; subnormal_g: amax near
    2^-120, so the tensor scale g = amax / 2688 and the decode scales are
    float32 subnormals."""
    print(f"nvfp4 {case}", flush=True)
    rng = np.random.default_rng(11)
    if case == "binades":
        rows = (rng.standard_normal((64, 512)) * np.exp2(rng.uniform(-30, 30, (64, 1)))).astype(np.float32)
    elif case == "near_binades":
        rows = (rng.standard_normal((64, 512)) * np.exp2(rng.uniform(-12, 0, (64, 1)) + 5)).astype(np.float32)
    elif case == "subnormal_g":
        rows = (rng.standard_normal((16, 64)) * np.exp2(rng.uniform(-8, 0, (16, 1)) - 122)).astype(np.float32)
        g = np.float32(np.abs(rows).max()) / np.float32(2688)
        assert 0 < g < np.finfo(np.float32).tiny
    elif case == "ties":
        rows = _ties()
    elif case == "zero":
        rows = np.zeros((8, 64), np.float32)
        rows[2, 5] = -0.0
    else:
        rows = (rng.standard_normal((8, 64)) * 2.0 ** -140).astype(np.float32)
    _check(rows, torch.from_numpy(rows).cuda())


def test_nvfp4_bf16_bytes_equal_the_oracle():
    rng = np.random.default_rng(12)
    bits = f32_to_bf16_bits((rng.standard_normal((96, 1024)) * 0.01).astype(np.float32))
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    _check(bf16_bits_to_f32(bits), t)


def test_nvfp4_bits_identical_under_shuffles():
    rng = np.random.default_rng(13)
    t = torch.from_numpy(rng.standard_normal((4096, 2048)).astype(np.float32)).cuda()
    ref = None
    for seed in (0, 5, 0xABCD):
        c, s, g = moe.moe_nvfp4_quantize(t, shuffle_seed=seed)
        fps = (moe.moe_fingerprint(c)[1], moe.moe_fingerprint(s)[1], moe.moe_fingerprint(g)[1])
        ref = fps if ref is None else ref
        assert fps == ref, seed
