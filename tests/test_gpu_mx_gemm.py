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
from compare import MX_REL_TOL, MX_TERM_BOUND
from harness import device_inputs, rel_l2, to_host
from test_gpu_parity import EDGE

pytestmark = pytest.mark.gpu

# the float32 dprob of the MXFP8 path: tests/compare.py MX_TERM_BOUND (per
# slot, of its sum of |terms|) and MX_REL_TOL (rel-L2)
MX_DPROB_TOL = MX_REL_TOL


def _case(name):
    cfg = CONFIGS.get(name) or EDGE[name]
    di = device_inputs(cfg)
    prob = moe.Problem.from_config(cfg)
    routing, _, _ = moe.moe_fwd(prob, di.logits, di.x, di.w1, di.w2)
    rng = np.random.default_rng([cfg.seed, 77])
    dh_bits = f32_to_bf16_bits((rng.standard_normal((prob.rows_cap, cfg.d_ffn)) * 0.01).astype(np.float32))
    dh = torch.from_numpy(dh_bits.view(np.int16)).cuda().view(torch.bfloat16)
    return cfg, di, prob, routing, dh_bits, dh


@pytest.mark.parametrize("name", ["ragged_bf16", "many_experts_bf16", "rows192_bf16", "single_token_bf16",
                                  "no_tokens_bf16", "max_experts_bf16", "bf16_e8k2"])
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


def test_mx_dgrad_fc1_codes_beyond_2gib():
    """dh codes past 2 GiB (600000 tokens top-2 of 64 experts at d_ffn
    2048: 2.5 GB of codes, read from each tile's first row): the first
    expert's and the last two experts' dx rows against the oracle.  dh rows
    repeat one seeded 4096-row block."""
    from synth import Config
    cfg = Config("mx_fc1_2gib_e64k2", 600000, 256, 2048, 64, 2, 0, 64, "bf16", 1, 36)
    di = device_inputs(cfg)
    prob = moe.Problem.from_config(cfg)
    routing = moe.moe_route(prob, di.logits)
    D, F, el, rc = cfg.d_model, cfg.d_ffn, cfg.num_local, prob.rows_cap
    rng = np.random.default_rng([cfg.seed, 77])
    reps = (rc + 4095) // 4096
    dh_bits = np.tile(f32_to_bf16_bits((rng.standard_normal((4096, F)) * 0.01).astype(np.float32)), (reps, 1))[:rc]
    dh = torch.from_numpy(dh_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dmx = moe.moe_mx_quantize(dh)
    wmx = moe.moe_mx_quantize(di.w1.reshape(el * D, F))
    wmx = (wmx[0].reshape(el, D, F), wmx[1].reshape(el, D, F // 32))
    out = moe.moe_mx_dgrad_fc1(prob, routing, dmx, wmx)
    torch.cuda.synchronize()
    idx, _ = oracle.route(di.host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, el)
    off = perm["offsets"]
    assert int(off[-2]) * F > (2 << 30)
    w1 = oracle.decode(di.host["w1"], "bf16")
    for e in (0, el - 2, el - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        ac, asc = oracle.mx_quantize_fast(bf16_bits_to_f32(dh_bits[lo:hi]).astype(np.float64))
        bc, bsc = oracle.mx_quantize_fast(w1[e])
        ref = oracle.mx_grouped_rows(ac, asc, bc[None], bsc[None], np.array([0, hi - lo]))
        err = rel_l2(to_host(out[lo:hi]), ref)
        print(f"  expert {e} rows {lo}..{hi} rel-L2 {err:.3e}", flush=True)
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


# ---------------------------------------------------------------- fc2 dgrad
# The MXFP8 fc2 data gradient is the layer backward with dy and W2 replaced by
# their MXFP8 values, so the oracle is oracle.backward on the oracle's own
# dequantised operands; h is a seeded input shared by both sides.
def _fc2_case(name):
    cfg = CONFIGS.get(name) or EDGE[name]
    di = device_inputs(cfg)
    prob = moe.Problem.from_config(cfg)
    routing, _, _ = moe.moe_fwd(prob, di.logits, di.x, di.w1, di.w2)
    rng = np.random.default_rng([cfg.seed, 78])
    h_bits = f32_to_bf16_bits((rng.standard_normal((prob.rows_cap, cfg.d_ffn)) * 0.5).astype(np.float32))
    h = torch.from_numpy(h_bits.view(np.int16)).cuda().view(torch.bfloat16)
    D, F, el = cfg.d_model, cfg.d_ffn, cfg.num_local
    dymx = moe.moe_mx_quantize(di.dy)
    wq = moe.moe_mx_quantize(di.w2.reshape(el * F, D))
    w2mx = (wq[0].reshape(el, F, D), wq[1].reshape(el, F, D // 32))
    return cfg, di, prob, routing, h_bits, h, dymx, w2mx


def _fc2_oracle(cfg, di, h_bits):
    D, F, el, k = cfg.d_model, cfg.d_ffn, cfg.num_local, cfg.top_k
    idx, topk_prob = oracle.route(di.host["logits"], k)
    perm = oracle.permute(idx, cfg.expert_begin, el)
    R = int(perm["offsets"][-1])
    deq = lambda a: oracle.mx_dequantize(*oracle.mx_quantize_fast(a))  # noqa: E731
    dy = deq(oracle.decode(di.host["dy"], "bf16"))
    w2 = deq(oracle.decode(di.host["w2"], "bf16").reshape(el * F, D)).reshape(el, F, D)
    x = oracle.decode(di.host["x"], "bf16")
    w1 = oracle.decode(di.host["w1"], "bf16")
    h = bf16_bits_to_f32(h_bits[:R]).astype(np.float64)
    ref = oracle.backward(x, w1, w2, h, dy, topk_prob, perm, k, combine=False)
    # sum over f and k of |dy[tok, k] W2[f, k] relu(h[f])^2| per slot: the
    # scale of dprob's rounding bound
    off, row_tok = perm["offsets"], perm["row_tok"]
    a = np.maximum(h, 0.0) ** 2
    mag = np.zeros(R)
    for e in range(el):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            mag[lo:hi] = np.sum((np.abs(dy[row_tok[lo:hi]]) @ np.abs(w2[e]).T) * a[lo:hi], axis=1)
    ref["dprob_mag"] = np.zeros(cfg.tokens * k)
    ref["dprob_mag"][perm["row_src"]] = mag
    return R, ref


@pytest.mark.parametrize("name,mode", [("ragged_bf16", moe.DETERMINISTIC), ("ragged_bf16", moe.ATOMIC),
                                       ("shard_bf16", moe.DETERMINISTIC), ("empty_experts_bf16", moe.DETERMINISTIC),
                                       ("single_token_bf16", moe.DETERMINISTIC), ("no_tokens_bf16", moe.DETERMINISTIC),
                                       ("rows192_bf16", moe.ATOMIC), ("max_experts_bf16", moe.DETERMINISTIC),
                                       ("bf16_e8k2", moe.DETERMINISTIC), ("bf16_e8k2", moe.ATOMIC)])
def test_mx_dgrad_fc2_parity(name, mode):
    print(f"mx dgrad fc2 {name} mode {mode}", flush=True)
    cfg, di, prob, routing, h_bits, h, dymx, w2mx = _fc2_case(name)
    dprob, dh = moe.moe_mx_dgrad_fc2(prob, routing, dymx, w2mx, h, mode)
    torch.cuda.synchronize()
    R, ref = _fc2_oracle(cfg, di, h_bits)
    e_dprob = rel_l2(dprob.cpu().numpy(), ref["dprob"])
    e_dh = rel_l2(to_host(dh[:R]), ref["dh"])
    print(f"  rel-L2 dprob {e_dprob:.3e} dh {e_dh:.3e}", flush=True)
    assert e_dh <= 2e-2
    assert e_dprob <= MX_DPROB_TOL
    err = np.abs(dprob.cpu().numpy().astype(np.float64).ravel() - ref["dprob"].ravel())
    assert np.all(err <= MX_TERM_BOUND * ref["dprob_mag"] + 1e-30), float(np.max(err / (ref["dprob_mag"] + 1e-30)))
    # slots routed to non-local experts are exactly 0
    local = (ref["dprob"] != 0)
    assert np.all(dprob.cpu().numpy()[~local] == 0)


def test_mx_dgrad_fc2_bits_identical_under_shuffles():
    cfg, di, prob, routing, h_bits, h, dymx, w2mx = _fc2_case("bf16_e8k2")
    R = routing.rows
    ref = None
    for seed in (0, 3, 0xBEEF):
        dprob, dh = moe.moe_mx_dgrad_fc2(prob.with_seed(seed), routing, dymx, w2mx, h)
        fps = tuple(moe.moe_fingerprint(t.contiguous())[1] for t in (dprob, dh[:R]))
        ref = fps if ref is None else ref
        assert fps == ref, seed
