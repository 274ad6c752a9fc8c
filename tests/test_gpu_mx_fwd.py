"""MXFP8 forward GEMMs (moe_mx_fwd_fc1, moe_mx_fwd_fc2) and the transposing
quantiser they read the weights through (moe_mx_quantize_t), against the CPU
oracle.

Both sides quantise the same seeded tensors themselves (GPU moe_mx_quantize /
moe_mx_quantize_t, oracle mx_quantize_fast on the matrix or its transpose;
the bytes are compared exactly) and the oracle multiplies its own dequantised
values in float64, one expert at a time.  Outputs are bf16, so every row is
held to the bf16 bounds of tests/compare.py; the bits are identical under
shuffled launch orders."""
import numpy as np
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
import oracle
from compare import Piecewise, tol_for
from harness import device_inputs, rel_l2, to_host
from synth import CONFIGS
from synth.inputs import bf16_bits_to_f32, f32_to_bf16_bits
from test_gpu_parity import EDGE

pytestmark = pytest.mark.gpu

SMALL = ["ragged_bf16", "many_experts_bf16", "rows192_bf16", "single_token_bf16", "no_tokens_bf16",
         "empty_experts_bf16", "shard_bf16", "max_experts_bf16", "bf16_e8k2"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()


def _u8(t):
    return t.cpu().numpy().astype(np.uint8)


@pytest.mark.parametrize("shape,dtype", [((3, 64, 96), "bf16"), ((2, 32, 512), "f32"), ((1, 256, 256), "bf16"),
                                         ((5, 96, 40), "f32")])
def test_mx_quantize_t_bytes_equal_the_oracle(shape, dtype):
    """Codes and scales of each matrix's transpose, byte for byte (values
    across many binades, and one all-zero column block)."""
    g, rows, cols = shape
    rng = np.random.default_rng([g, rows, cols])
    v = (rng.standard_normal(shape) * np.exp2(rng.integers(-20, 20, size=shape))).astype(np.float32)
    v[:, :32, 0] = 0.0
    if dtype == "bf16":
        bits = f32_to_bf16_bits(v)
        t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        vals = bf16_bits_to_f32(bits).astype(np.float64)
    else:
        t = torch.from_numpy(v).cuda()
        vals = v.astype(np.float64)
    codes, scales = moe.moe_mx_quantize_t(t)
    for e in range(g):
        rc, rs = oracle.mx_quantize_fast(vals[e].T)
        assert np.array_equal(_u8(codes[e]), rc), e
        assert np.array_equal(_u8(scales[e]), rs), e
    # shuffled launch order: the same bytes
    c2, s2 = moe.moe_mx_quantize_t(t, shuffle_seed=0xC0DE)
    assert torch.equal(c2, codes) and torch.equal(s2, scales)


def _setup(cfg):
    di = device_inputs(cfg)
    prob = moe.Problem.from_config(cfg)
    routing, _, _ = moe.moe_fwd(prob, di.logits, di.x, di.w1, di.w2)
    return di, prob, routing


def _oracle_perm(cfg, host):
    idx, p = oracle.route(host["logits"], cfg.top_k)
    return idx, p, oracle.permute(idx, cfg.expert_begin, cfg.num_local)


def _dequant_weights_t(host_w, experts, pool):
    """The oracle's dequantised MXFP8 of each expert's transposed weight
    (quantised along the contraction axis), computed on a thread pool."""
    def one(e):
        return e, oracle.mx_dequantize(*oracle.mx_quantize_fast(oracle.decode(host_w[e], "bf16").T))
    return dict(pool.map(one, experts))


def _batches(cfg, perm, label):
    """Non-empty local experts in batches of 64, with a progress line each."""
    off = perm["offsets"]
    live = [e for e in range(cfg.num_local) if off[e + 1] > off[e]]
    for i in range(0, len(live), 64):
        if len(live) > 64:
            print(f"  {label}: experts {i}..{min(i + 64, len(live)) - 1} of {len(live)}", flush=True)
        yield live[i:i + 64]


def _fc1_check(cfg, di, prob, routing, perm, h, act):
    """Every routed row of h and act against the oracle, expert by expert."""
    from concurrent.futures import ThreadPoolExecutor
    x = oracle.decode(di.host["x"], "bf16")
    xq = oracle.mx_dequantize(*oracle.mx_quantize_fast(x))
    off, row_tok = perm["offsets"], perm["row_tok"]
    tol = tol_for("bf16")
    ch, ca = Piecewise("h", tol), Piecewise("act", tol)
    with ThreadPoolExecutor(16) as pool:
        for batch in _batches(cfg, perm, "oracle fc1"):
            wq = _dequant_weights_t(di.host["w1"], batch, pool)     # [F, D] per expert
            for e in batch:
                s, t = int(off[e]), int(off[e + 1])
                href = xq[row_tok[s:t]] @ wq[e].T
                ch.add(to_host(h[s:t]), href, ("expert", e))
                ca.add(to_host(act[s:t]), np.maximum(href, 0.0) ** 2, ("expert", e))
    fails = ch.failures() + ca.failures()
    assert not fails, fails
    return dict(h=ch.rel(), act=ca.rel(), h_worst_row=ch.worst, act_worst_row=ca.worst)


@pytest.mark.parametrize("name", SMALL)
def test_mx_fwd_fc1_parity(name):
    print(f"mx fwd fc1 {name}", flush=True)
    cfg = CONFIGS.get(name) or EDGE[name]
    di, prob, routing = _setup(cfg)
    el, D, F = cfg.num_local, cfg.d_model, cfg.d_ffn
    xmx = moe.moe_mx_quantize(di.x)
    w1t = moe.moe_mx_quantize_t(di.w1)
    h, act = moe.moe_mx_fwd_fc1(prob, routing, xmx, w1t)
    torch.cuda.synchronize()
    _, _, perm = _oracle_perm(cfg, di.host)
    print(" ", _fc1_check(cfg, di, prob, routing, perm, h, act), flush=True)


def _act_input(cfg, prob):
    """A seeded bf16 act [rows_cap, F] (relu(h)^2 of a seeded h), shared input of both sides."""
    rng = np.random.default_rng([cfg.seed, 81])
    hh = (rng.standard_normal((prob.rows_cap, cfg.d_ffn)) * 0.05).astype(np.float32)
    bits = f32_to_bf16_bits(np.maximum(hh, 0) ** 2)
    return bits, torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def _fc2_ref(cfg, di, perm, p, act_bits):
    """Oracle o rows and (full layer) y from its own MXFP8 act and W2^T."""
    from concurrent.futures import ThreadPoolExecutor
    R = int(perm["offsets"][-1])
    aq = oracle.mx_dequantize(*oracle.mx_quantize_fast(bf16_bits_to_f32(act_bits[:R]).astype(np.float64)))
    off = perm["offsets"]
    o = np.zeros((R, cfg.d_model))
    with ThreadPoolExecutor(16) as pool:
        for batch in _batches(cfg, perm, "oracle fc2"):
            wq = _dequant_weights_t(di.host["w2"], batch, pool)     # [D, F] per expert
            for e in batch:
                s, t = int(off[e]), int(off[e + 1])
                o[s:t] = aq[s:t] @ wq[e].T
    if cfg.combine:
        return o, oracle.combine_rows(o, perm["slot_row"], p, cfg.tokens, cfg.top_k)
    return o, None


@pytest.mark.parametrize("name,mode", [(n, moe.DETERMINISTIC) for n in SMALL] +
                                      [("ragged_bf16", moe.ATOMIC), ("bf16_e8k2", moe.ATOMIC)])
def test_mx_fwd_fc2_parity(name, mode):
    print(f"mx fwd fc2 {name} mode {mode}", flush=True)
    cfg = CONFIGS.get(name) or EDGE[name]
    di, prob, routing = _setup(cfg)
    act_bits, act = _act_input(cfg, prob)
    amx = moe.moe_mx_quantize(act)
    w2t = moe.moe_mx_quantize_t(di.w2)
    y = moe.moe_mx_fwd_fc2(prob, routing, amx, w2t, mode)
    torch.cuda.synchronize()
    _, p, perm = _oracle_perm(cfg, di.host)
    R = int(perm["offsets"][-1])
    o_ref, y_ref = _fc2_ref(cfg, di, perm, p, act_bits)
    tol = tol_for("bf16")
    if cfg.combine:
        c = Piecewise("y", tol).add(to_host(y), y_ref, "token")
    else:
        c = Piecewise("o_rows", tol).add(to_host(y[:R]), o_ref, "row")
    print(f"  rel-L2 {c.rel():.3e} worst row {c.worst:.3e}", flush=True)
    assert not c.failures(), c.failures()


def test_mx_fwd_bits_identical_under_shuffles():
    cfg = CONFIGS["bf16_e8k2"]
    di, prob, routing = _setup(cfg)
    R = routing.rows
    xmx, w1t, w2t = moe.moe_mx_quantize(di.x), moe.moe_mx_quantize_t(di.w1), moe.moe_mx_quantize_t(di.w2)
    ref = None
    for seed in (0, 5, 0xFACE):
        ps = prob.with_seed(seed)
        h, act = moe.moe_mx_fwd_fc1(ps, routing, xmx, w1t)
        y = moe.moe_mx_fwd_fc2(ps, routing, moe.moe_mx_quantize(act), w2t)
        fps = tuple(moe.moe_fingerprint(t.contiguous())[1] for t in (h[:R], act[:R], y))
        ref = fps if ref is None else ref
        assert fps == ref, seed


def test_mx_fwd_full_size_latent():
    """The 512-expert top-22 layer: every routed row of h and act (fc1), and
    every token of y from a seeded act (fc2), against the oracle streamed one
    expert at a time."""
    cfg = CONFIGS["latent_e512k22"]
    print("[latent mx fwd] inputs", flush=True)
    di, prob, routing = _setup(cfg)
    xmx = moe.moe_mx_quantize(di.x)
    w1t = moe.moe_mx_quantize_t(di.w1)
    h, act = moe.moe_mx_fwd_fc1(prob, routing, xmx, w1t)
    del w1t
    # fc2 on a seeded act, an input of both sides
    act_bits, act_in = _act_input(cfg, prob)
    w2t = moe.moe_mx_quantize_t(di.w2)
    y = moe.moe_mx_fwd_fc2(prob, routing, moe.moe_mx_quantize(act_in), w2t)
    torch.cuda.synchronize()
    del w2t
    _, p, perm = _oracle_perm(cfg, di.host)
    print("[latent mx fwd] oracle fc1", flush=True)
    errs = _fc1_check(cfg, di, prob, routing, perm, h, act)
    print("[latent mx fwd] oracle fc2", flush=True)
    _, y_ref = _fc2_ref(cfg, di, perm, p, act_bits)
    c = Piecewise("y", tol_for("bf16")).add(to_host(y), y_ref, "token")
    errs.update(y=c.rel(), y_worst_row=c.worst)
    print(f"[latent mx fwd] {errs}", flush=True)
    assert not c.failures(), c.failures()
