"""Full-size workloads (LatentMoE 512 experts top-22, the skewed-routing
variant, and one GPU's 4-expert shard of a 16384-token layer) against the
oracle, over every element of every output.

The float64 oracle of a whole 512-expert layer would hold 34 GB of weights,
so it runs one expert at a time on the same inputs (oracle.expert_forward and
oracle.expert_backward on the expert's rows), and the comparison accumulates:
  * routing state (top-k indices, counts, offsets, row maps) for the whole
    layer, bit-exact; probabilities to 1e-5;
  * h and dh: every routed row (whole-tensor and worst-row rel-L2);
  * dW1 and dW2: every expert's complete matrices, every row;
  * dprob: every slot, against its own rounding scale (tests/compare.py),
    exact zeros off the shard;
  * y and dx of the token-layout workloads: every token, from the oracle's
    rows combined over each token's k slots; the shard's o and dx rows;
  * empty experts exact zero dW;
  * the homogeneity identities (o is homogeneous of degree 2 in (x, W1) and
    of degree 1 in W2), evaluated from the outputs alone;
  * bit-identical outputs (fingerprints) over 20 repeated runs and under four
    shuffled workgroup orders.
"""
import time

import numpy as np
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
import oracle
from compare import Piecewise, SlotBound, dprob_term_scale, tol_for
from synth import CONFIGS, make_inputs, make_router_inputs
from harness import (DeviceInputs, LayerRunner, compare_routing, determinism_runs, rel_l2, to_dev, to_host)

pytestmark = pytest.mark.gpu

LARGE = ["latent_e512k22", "skewed_e512k22", "shard_e512k22_l4"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()


def _weights(cfg, host, e_local):
    """float64 weights of local expert e_local."""
    return oracle.decode(host["w1"][e_local], cfg.dtype), oracle.decode(host["w2"][e_local], cfg.dtype)


def _stream_check(cfg, host, perm, prob, out) -> dict:
    """Every expert's rows and weight gradients against the oracle, one
    expert at a time; the token-layout outputs from the oracle's rows
    combined over the k slots of each token."""
    tol = tol_for(cfg.dtype)
    x = oracle.decode(host["x"], cfg.dtype)
    dy = oracle.decode(host["dy"], cfg.dtype)
    off, row_tok, row_src, slot_row = perm["offsets"], perm["row_tok"], perm["row_src"], perm["slot_row"]
    R, D, F, el = int(off[-1]), cfg.d_model, cfg.d_ffn, cfg.num_local
    p_rows = prob.reshape(-1)[row_src]
    chk = {n: Piecewise(n, tol) for n in ("h", "dh", "dw1", "dw2")}
    if cfg.combine:
        o_all, dx_all = np.zeros((R, D)), np.zeros((R, D))
    else:
        chk["o_rows"], chk["dx_rows"] = Piecewise("o_rows", tol), Piecewise("dx_rows", tol)
    dprob_rows, scale = np.zeros(R), np.zeros(R)
    t0 = time.time()
    for e in range(el):
        s, t = int(off[e]), int(off[e + 1])
        g_dw1, g_dw2 = to_host(out["dw1"][e]), to_host(out["dw2"][e])
        if t == s:
            assert np.all(g_dw1 == 0) and np.all(g_dw2 == 0), f"empty expert {e} must have exact zero dW"
            continue
        w1, w2 = _weights(cfg, host, e)
        xr, dyr = x[row_tok[s:t]], dy[row_tok[s:t]]
        h, o = oracle.expert_forward(xr, w1, w2)
        b = oracle.expert_backward(xr, dyr, p_rows[s:t], h, w1, w2)
        chk["h"].add(to_host(out["h"][s:t]), h, ("expert", e))
        chk["dh"].add(to_host(out["dh"][s:t]), b["dh"], ("expert", e))
        chk["dw1"].add(g_dw1, b["dw1"], ("expert", e))
        chk["dw2"].add(g_dw2, b["dw2"], ("expert", e))
        dprob_rows[s:t] = b["dprob"]
        scale[s:t] = dprob_term_scale(b["dh"], h, p_rows[s:t])
        if cfg.combine:
            o_all[s:t], dx_all[s:t] = o, b["dx_rows"]
        else:
            chk["o_rows"].add(to_host(out["y"][s:t]), o, ("expert", e))
            chk["dx_rows"].add(to_host(out["dx"][s:t]), b["dx_rows"], ("expert", e))
        if e % 64 == 63:
            print(f"  oracle: {e + 1}/{el} experts, {time.time() - t0:.1f} s", flush=True)
    sb = SlotBound(cfg.dtype, max(D, F))
    gd = to_host(out["dprob"]).reshape(-1)
    sb.add(gd[row_src], dprob_rows, scale, "row")
    sb.add_zero(gd[slot_row < 0])
    rd = np.zeros(cfg.tokens * cfg.top_k)
    rd[row_src] = dprob_rows
    chk["dprob"] = Piecewise("dprob", tol).add(gd, rd, rows=False)
    if cfg.combine:
        T, k = cfg.tokens, cfg.top_k
        chk["y"] = Piecewise("y", tol).add(to_host(out["y"]), oracle.combine_rows(o_all, slot_row, prob, T, k), "token")
        chk["dx"] = Piecewise("dx", tol).add(to_host(out["dx"]),
                                            oracle.combine_rows(dx_all, slot_row, np.ones((T, k)), T, k), "token")
    fails = [f for c in chk.values() for f in c.failures()] + sb.failures()
    errs = {n: c.rel() for n, c in chk.items()}
    errs.update({f"{n}_worst_row": c.worst for n, c in chk.items() if n != "dprob"})
    errs["dprob_worst_z"] = sb.worst
    assert not fails, f"{fails} (all: {errs})"
    return errs


def _euler(cfg, di, out, routing):
    """Homogeneity identities over every expert (and token), evaluated in
    float64 on the device from the outputs alone."""
    R = routing.rows
    counts = routing.counts.long()
    offs = routing.offsets.long()
    dprob_rows = out["dprob"].reshape(-1)[routing.row_src[:R].long()].double()
    lp = dprob_rows * routing.row_prob[:R].double()
    seg = torch.repeat_interleave(torch.arange(cfg.num_local, device=lp.device), counts)
    L_e = torch.zeros(cfg.num_local, dtype=torch.float64, device=lp.device).index_add_(0, seg, lp)
    assert int(offs[-1]) == R
    lhs1 = torch.empty(cfg.num_local, dtype=torch.float64, device=lp.device)
    lhs2 = torch.empty_like(lhs1)
    for e in range(cfg.num_local):
        lhs1[e] = (out["dw1"][e].double() * di.w1[e].double()).sum()
        lhs2[e] = (out["dw2"][e].double() * di.w2[e].double()).sum()
    res = dict(euler_w1=rel_l2(lhs1.cpu().numpy(), 2 * L_e.cpu().numpy()),
               euler_w2=rel_l2(lhs2.cpu().numpy(), L_e.cpu().numpy()))
    if cfg.combine:
        xdx = (out["dx"].double() * di.x.double()).sum(dim=1)
        pdp = 2 * (routing.topk_prob.double() * out["dprob"].double()).sum(dim=1)
        res["euler_x"] = rel_l2(xdx.cpu().numpy(), pdp.cpu().numpy())
    return res


@pytest.mark.parametrize("name", LARGE)
def test_large_full_parity_and_determinism(name):
    cfg = CONFIGS[name]
    print(f"[{name}] drawing inputs", flush=True)
    host = make_inputs(cfg)
    di = DeviceInputs(cfg, host)
    prob = moe.Problem.from_config(cfg)
    print(f"[{name}] HIP path (deterministic)", flush=True)
    runner = LayerRunner(prob, di)
    out = runner.run(0)
    r = out["routing"]

    # routing, whole layer, bit-exact
    idx, p = oracle.route(host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, cfg.num_local)
    compare_routing(r, dict(topk_idx=idx, topk_prob=p, perm=perm))
    R = int(perm["offsets"][-1])
    assert R == r.rows
    if cfg.combine:
        assert R == cfg.tokens * cfg.top_k
    empty = np.nonzero(perm["counts"] == 0)[0]
    if name == "skewed_e512k22":
        # max/mean load about 12 (mean 176 rows) and some experts without rows
        assert len(empty) > 0 and perm["counts"].max() > 8 * 176, "skewed workload must be skewed and hold empty experts"

    print(f"[{name}] oracle over all {cfg.num_local} experts ({R} rows)", flush=True)
    errs = _stream_check(cfg, host, perm, p, out)
    errs.update(_euler(cfg, di, out, r))
    print(f"[{name}] errors {errs}", flush=True)
    bad = {k: v for k, v in errs.items() if k.startswith("euler") and not v <= 2e-2}
    assert not bad, f"identities off by more than 2e-2: {bad}"

    # router backward at full size (full-layer workloads): seeded dprob and
    # router weights, the layer's routing, whole tensors against the oracle
    if cfg.combine and cfg.num_local == cfg.num_experts:
        ri = make_router_inputs(cfg)
        dl, dwr, dxr = moe.moe_router_bwd(prob, r, torch.from_numpy(ri["dprob"]).cuda(), di.x,
                                          to_dev(ri["wr"], cfg.dtype))
        torch.cuda.synchronize()
        ref = oracle.router_backward(idx, p, ri["dprob"], oracle.decode(host["x"], cfg.dtype),
                                     oracle.decode(ri["wr"], cfg.dtype))
        rerr = {"router_dlogits": rel_l2(to_host(dl), ref["dlogits"]), "router_dwr": rel_l2(to_host(dwr), ref["dwr"]),
                "router_dx": rel_l2(to_host(dxr), ref["dx"])}
        print(f"[{name}] router rel-L2 {rerr}", flush=True)
        assert rerr["router_dlogits"] <= 1e-5 and rerr["router_dwr"] <= 1e-5 and rerr["router_dx"] <= 2e-2, rerr
        del dl, dwr, dxr

    # bit identity: 20 repeats, then four shuffled workgroup orders (twice each)
    print(f"[{name}] repeats and shuffled launch orders", flush=True)
    n = determinism_runs(runner, cfg.combine, label=name)
    print(f"[{name}] {n} runs bit-identical to the first", flush=True)


def test_routed_rows_beyond_2gib():
    """A layer whose arrays of routed rows exceed 2 GiB (80000 tokens top-2 of
    8 experts at d_ffn 8192: h, dh and act_p are 2.6 GB each), so that rows
    past the first 2 GiB are reached only through the tiles' own base
    addresses: every routed row, every dW element (each expert's 20000 rows
    split into ordered K chunks) and every token against the oracle, then
    bit identity over repeats and shuffled launch orders."""
    from synth import Config
    cfg = Config("rows_2gib_e8k2", 80000, 256, 8192, 8, 2, 0, 8, "bf16", 1, 31)
    prob = moe.Problem.from_config(cfg)
    assert prob.rows_cap * cfg.d_ffn * 2 > (2 << 30)
    print("[rows > 2 GiB] drawing inputs", flush=True)
    host = make_inputs(cfg)
    di = DeviceInputs(cfg, host)
    runner = LayerRunner(prob, di)
    out = runner.run(0)
    idx, p = oracle.route(host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, cfg.num_local)
    compare_routing(out["routing"], dict(topk_idx=idx, topk_prob=p, perm=perm))
    assert int(perm["offsets"][-1]) == cfg.tokens * cfg.top_k
    # the last expert's rows start past 2 GiB of h
    assert int(perm["offsets"][-2]) * cfg.d_ffn * 2 > (2 << 30)
    print("[rows > 2 GiB] oracle over all experts", flush=True)
    errs = _stream_check(cfg, host, perm, p, out)
    errs.update(_euler(cfg, di, out, out["routing"]))
    print(f"[rows > 2 GiB] errors {errs}", flush=True)
    assert errs["euler_w1"] <= 2e-2 and errs["euler_w2"] <= 2e-2 and errs["euler_x"] <= 2e-2, errs
    n = determinism_runs(runner, cfg.combine, repeats=4, label="rows > 2 GiB")
    print(f"[rows > 2 GiB] {n} runs bit-identical to the first", flush=True)


def test_large_mx_data_gradients_streamed():
    """The MXFP8 data gradients at LatentMoE size (512 experts, 2 GiB of W1
    codes): every routed row of every expert against the oracle on its own
    dequantised operands, one expert at a time.  h and dh are seeded inputs
    of both sides; dprob is held to the MXFP8 tolerance (compare.py
    MX_REL_TOL), dh and dx_rows to the bf16 bounds row by row."""
    from concurrent.futures import ThreadPoolExecutor
    from compare import MX_REL_TOL
    cfg = CONFIGS["latent_e512k22"]
    print("[latent mx] drawing inputs", flush=True)
    host = make_inputs(cfg)
    di = DeviceInputs(cfg, host)
    prob = moe.Problem.from_config(cfg)
    D, F, el = cfg.d_model, cfg.d_ffn, cfg.num_local
    routing, _, _ = moe.moe_fwd(prob, di.logits, di.x, di.w1, di.w2)
    rng = np.random.default_rng([cfg.seed, 79])
    from synth.inputs import f32_to_bf16_bits, bf16_bits_to_f32
    h_bits = f32_to_bf16_bits((rng.standard_normal((prob.rows_cap, F)) * 0.5).astype(np.float32))
    dh_bits = f32_to_bf16_bits((rng.standard_normal((prob.rows_cap, F)) * 0.01).astype(np.float32))
    up = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    h, dh = up(h_bits), up(dh_bits)
    print("[latent mx] HIP path", flush=True)
    dymx = moe.moe_mx_quantize(di.dy)
    wq2 = moe.moe_mx_quantize(di.w2.reshape(el * F, D))
    dprob, g_dh = moe.moe_mx_dgrad_fc2(prob, routing, dymx, (wq2[0].reshape(el, F, D),
                                                            wq2[1].reshape(el, F, D // 32)), h)
    del wq2
    wq1 = moe.moe_mx_quantize(di.w1.reshape(el * D, F))
    dx_rows = moe.moe_mx_dgrad_fc1(prob, routing, moe.moe_mx_quantize(dh), (wq1[0].reshape(el, D, F),
                                                                           wq1[1].reshape(el, D, F // 32)))
    torch.cuda.synchronize()
    del wq1

    idx, p = oracle.route(host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, el)
    off, row_tok, row_src = perm["offsets"], perm["row_tok"], perm["row_src"]
    p_rows = p.reshape(-1)[row_src]
    deq = lambda a: oracle.mx_dequantize(*oracle.mx_quantize_fast(a))  # noqa: E731
    x = oracle.decode(host["x"], "bf16")
    dy = oracle.decode(host["dy"], "bf16")
    g_dprob = to_host(dprob).reshape(-1)
    tol = tol_for("bf16")
    c_dh, c_dx = Piecewise("dh", tol), Piecewise("dx_rows", tol)
    got_p, ref_p = [], []

    def oracle_expert(e):
        s, t = int(off[e]), int(off[e + 1])
        if t == s:
            return e, None
        w1, w2 = _weights(cfg, host, e)
        hr = bf16_bits_to_f32(h_bits[s:t]).astype(np.float64)
        b = oracle.expert_backward(x[row_tok[s:t]], deq(dy[row_tok[s:t]]), p_rows[s:t], hr, w1, deq(w2))
        dhq = deq(bf16_bits_to_f32(dh_bits[s:t]).astype(np.float64))
        return e, (b["dprob"], b["dh"], dhq @ deq(w1).T)

    with ThreadPoolExecutor(16) as pool:
        for b0 in range(0, el, 64):
            print(f"[latent mx] oracle experts {b0}..{b0 + 63}", flush=True)
            for e, r in pool.map(oracle_expert, range(b0, min(b0 + 64, el))):
                if r is None:
                    continue
                s, t = int(off[e]), int(off[e + 1])
                got_p.append(g_dprob[row_src[s:t]])
                ref_p.append(np.asarray(r[0]).ravel())
                c_dh.add(to_host(g_dh[s:t]), r[1], ("expert", e))
                c_dx.add(to_host(dx_rows[s:t]), r[2], ("expert", e))
    errs = {"dprob": rel_l2(np.concatenate(got_p), np.concatenate(ref_p)), "dh": c_dh.rel(), "dx_rows": c_dx.rel(),
            "dh_worst_row": c_dh.worst, "dx_rows_worst_row": c_dx.worst}
    print(f"[latent mx] {errs}", flush=True)
    assert errs["dprob"] <= MX_REL_TOL
    fails = c_dh.failures() + c_dx.failures()
    assert not fails, fails
