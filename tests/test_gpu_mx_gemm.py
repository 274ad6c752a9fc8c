"""MXFP8 fc1 data gradient (moe_mx_dgrad_fc1) against the CPU oracle: both
sides quantise the same seeded dh and W1 themselves (GPU moe_mx_quantize,
oracle mx_quantize; their bytes agree exactly, see test_gpu_mx.py) and the
oracle multiplies the dequantised values in float64 per expert.  The output is
bf16, so the bound is the bf16 rel-L2 tolerance; the bits are identical under
shuffled launch orders."""
import numpy as np
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
import oracle
from synth import CONFIGS
from synth.inputs import f32_to_bf16_bits, bf16_bits_to_f32
from harness import device_inputs, rel_l2, to_host
from test_gpu_parity import EDGE

pytestmark = pytest.mark.gpu


def _case(name):
    cfg = CONFIGS.get(name) or EDGE[name]
    di = device_inputs(cfg)
    prob = moe.Problem.from_config(cfg)
    routing, _, _ = moe.moe_fwd(prob, di.logits, di.x, di.w1, di.w2)
    rng = np.random.default_rng([cfg.seed, 77])
    dh_bits = f32_to_bf16_bits((rng.standard_normal((prob.rows_cap, cfg.d_ffn)) * 0.01).astype(np.float32))
    dh = torch.from_numpy(dh_bits.view(np.int16)).cuda().view(torch.bfloat16)
    return cfg, di, prob, routing, dh_bits, dh


@pytest.mark.parametrize("name", ["ragged_bf16", "many_experts_bf16", "bf16_e8k2"])
def test_mx_dgrad_fc1_parity(name):
    print(f"mx dgrad fc1 {name}", flush=True)
    cfg, di, prob, routing, dh_bits, dh = _case(name)
    D, F, el = cfg.d_model, cfg.d_ffn, cfg.num_local
    dmx = moe.moe_mx_quantize(dh)
    wmx = moe.moe_mx_quantize(di.w1.reshape(el * D, F))
    wmx = (wmx[0].reshape(el, D, F), wmx[1].reshape(el, D, F // 32))
    out = moe.moe_mx_dgrad_fc1(prob, routing, dmx, wmx)
    torch.cuda.synchronize()
    idx, _ = oracle.route(di.host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, cfg.num_local)
    R = int(perm["offsets"][-1])
    ac, asc = oracle.mx_quantize_fast(bf16_bits_to_f32(dh_bits[:R]).astype(np.float64))
    w1 = oracle.decode(di.host["w1"], "bf16").reshape(el * D, F)
    bc, bsc = oracle.mx_quantize_fast(w1)
    ref = oracle.mx_grouped_rows(ac, asc, bc.reshape(el, D, F), bsc.reshape(el, D, F // 32), perm["offsets"])
    err = rel_l2(to_host(out[:R]), ref)
    print(f"  rel-L2 {err:.3e}", flush=True)
    assert err <= 2e-2


def test_mx_dgrad_fc1_bits_identical_under_shuffles():
    cfg, di, prob, routing, dh_bits, dh = _case("bf16_e8k2")
    D, F, el = cfg.d_model, cfg.d_ffn, cfg.num_local
    dmx = moe.moe_mx_quantize(dh)
    wmx = moe.moe_mx_quantize(di.w1.reshape(el * D, F))
    wmx = (wmx[0].reshape(el, D, F), wmx[1].reshape(el, D, F // 32))
    R = routing.rows
    ref = None
    for seed in (0, 3, 0xBEEF):
        out = moe.moe_mx_dgrad_fc1(prob.with_seed(seed), routing, dmx, wmx)
        fp = moe.moe_fingerprint(out[:R].contiguous())[1]
        ref = fp if ref is None else ref
        assert fp == ref, seed
