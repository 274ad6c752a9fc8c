"""MXFP8 block quantisation on the GPU against the CPU oracle, byte for byte
(codes and scales), on random rows across 60 binades, constructed ties,
saturating blocks, all-zero and all-subnormal blocks, signed zeros, and the
layer's own dh tensor; plus bit-identical fingerprints of the encoded values
and scale buffers under shuffled launch orders."""
import numpy as np
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
import oracle
from oracle import mx
from synth.inputs import f32_to_bf16_bits, bf16_bits_to_f32
from harness import device_inputs, run_layer
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def _rows(seed, n, k):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((n, k)) * np.exp2(rng.uniform(-30, 30, (n, 1)))).astype(np.float32)
    # constructed blocks: exact E4M3 midpoints after scaling, saturation, zeros, signed zeros
    pos = sorted(mx.e4m3_decode(c) for c in range(0x7F))
    mids = [(u + v) / 2 for u, v in zip(pos, pos[1:])]
    a[0, :32] = np.array(mids[-32:], np.float32) * 2.0 ** -8          # amax in [256, 512) * 2^-8
    a[1, :32] = 0.0
    a[1, 32:64] = -0.0
    a[2, :32] = np.float32(1.96875) * np.sign(rng.standard_normal(32))   # saturates to +-448
    a[3, :32] = np.array(mids[:32], np.float32) * 2.0 ** -8            # subnormal-code midpoints
    return a


def _check(a_host, dtype, shuffle=0):
    if dtype == "bf16":
        bits = f32_to_bf16_bits(a_host)
        t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        ref_in = bf16_bits_to_f32(bits).astype(np.float64)
    else:
        t = torch.from_numpy(a_host).cuda()
        ref_in = a_host.astype(np.float64)
    codes, scales = moe.moe_mx_quantize(t, shuffle_seed=shuffle)
    torch.cuda.synchronize()
    rc, rs = mx.mx_quantize(ref_in.reshape(-1, a_host.shape[-1]))
    np.testing.assert_array_equal(scales.cpu().numpy().reshape(rs.shape), rs)
    np.testing.assert_array_equal(codes.cpu().numpy().reshape(rc.shape), rc)
    return codes, scales


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(37, 256), (8, 32), (5, 96)])
def test_mx_quantize_bit_exact(dtype, shape):
    print(f"mx quantize {dtype} {shape}", flush=True)
    a = _rows(sum(shape), max(shape[0], 4), shape[1]) if shape[1] >= 64 else _rows(3, shape[0], shape[1])
    _check(a[: shape[0]], dtype)


def test_mx_quantize_subnormal_block():
    a = np.zeros((2, 64), np.float32)
    sub = f32_to_bf16_bits(np.float32(1.5) * np.float32(2.0 ** -130) * np.arange(1, 33, dtype=np.float32))
    a[0, :32] = bf16_bits_to_f32(sub)                  # every value a bf16 subnormal
    a[1, 32:] = np.float32(2.0 ** -149)                # the smallest float32 subnormal
    _check(a, "bf16")
    _check(a, "f32")


def test_mx_quantize_layer_tensor_and_fingerprints():
    cfg = CONFIGS["bf16_e8k2"]
    di = device_inputs(cfg)
    out = run_layer(moe.Problem.from_config(cfg), di)
    dh = out["dh"][: out["routing"].rows].contiguous()
    codes, scales = moe.moe_mx_quantize(dh)
    torch.cuda.synchronize()
    rows = np.random.default_rng(4).choice(dh.shape[0], 24, replace=False)
    hd = dh[torch.as_tensor(rows, device="cuda")].float().cpu().numpy().astype(np.float64)
    rc, rs = mx.mx_quantize(hd)
    np.testing.assert_array_equal(codes[torch.as_tensor(rows, device="cuda")].cpu().numpy(), rc)
    np.testing.assert_array_equal(scales[torch.as_tensor(rows, device="cuda")].cpu().numpy(), rs)
    ref = (moe.moe_fingerprint(codes)[1], moe.moe_fingerprint(scales)[1])
    for seed in (1, 0xBEEF):
        c2, s2 = moe.moe_mx_quantize(dh, shuffle_seed=seed)
        assert (moe.moe_fingerprint(c2)[1], moe.moe_fingerprint(s2)[1]) == ref


def test_mx_quantize_rejects_bad_shapes():
    t = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="status 2"):
        moe.moe_mx_quantize(t)
