"""MXFP8 weight gradients: the row-quantised operands (moe_mx_quantize_wgrad)
and the grouped GEMM (moe_mx_wgrad) against the CPU oracle.

Inputs of both sides: the seeded x, dY of the layer, seeded h and dH rows,
and seeded routing weights p per routed row (written into the routing's
row_prob, so that p relu(h)^2 is formed from the same float32 values on
both sides: its float32 value decides the codes).  Each side routes and
quantises by itself; the codes and scale bytes are compared exactly.  The
oracle multiplies its own dequantised operands in float64.  Both sides
multiply the same values, so the GEMM differs from the oracle only by its
accumulation, which the scaled MFMA does not do in exact float32 steps:
every element is held to tests/compare.py mx_block_bound (a fraction of
each block's largest representable product) plus the float32 bound of
adding the expert's K / 64 instruction results (fp32_sum_bound), and each
dW to MX_REL_TOL in rel-L2."""
import numpy as np
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
import oracle
from compare import MX_REL_TOL, ElementBound, Piecewise, fp32_sum_bound, mx_block_bound
from harness import device_inputs, to_host
from synth import CONFIGS, Config
from synth.inputs import bf16_bits_to_f32, f32_to_bf16_bits
from test_gpu_parity import EDGE

pytestmark = pytest.mark.gpu

# two experts of about 2500 rows each: 40 slices of K per tile, no chunk limit
LONG_K = Config("long_k_bf16", 5000, 256, 512, 2, 1, 0, 2, "bf16", 1, 31)
SMALL = ["ragged_bf16", "many_experts_bf16", "single_token_bf16", "no_tokens_bf16", "empty_experts_bf16",
         "shard_bf16", "rows192_bf16", "split_k_bf16", "max_experts_bf16", "bf16_e8k2", "long_k_bf16"]
KINDS = {"x": moe.MXW_TOKEN, "dy": moe.MXW_TOKEN, "dh": moe.MXW_ROW, "act": moe.MXW_ACT_P}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()


def _cfg(name):
    return LONG_K if name == "long_k_bf16" else (CONFIGS.get(name) or EDGE[name])


def _bits_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


class Case:
    """Seeded inputs of both sides, the HIP routing and the oracle's permutation."""

    def __init__(self, cfg, shuffle_seed=0):
        self.cfg = cfg
        self.di = device_inputs(cfg)
        self.prob = moe.Problem.from_config(cfg, shuffle_seed)
        self.routing, _, _ = moe.moe_fwd(self.prob, self.di.logits, self.di.x, self.di.w1, self.di.w2)
        rc, F = self.prob.rows_cap, cfg.d_ffn
        rng = np.random.default_rng([cfg.seed, 84])
        self.h_bits = f32_to_bf16_bits((rng.standard_normal((rc, F)) * 0.5).astype(np.float32))
        self.dh_bits = f32_to_bf16_bits((rng.standard_normal((rc, F)) * 0.01).astype(np.float32))
        self.p = rng.uniform(0.02, 1.0, rc).astype(np.float32)
        self.routing.row_prob.copy_(torch.from_numpy(self.p).cuda())
        self.h, self.dh = _bits_dev(self.h_bits), _bits_dev(self.dh_bits)
        idx, _ = oracle.route(self.di.host["logits"], cfg.top_k)
        self.perm = oracle.permute(idx, cfg.expert_begin, cfg.num_local)
        self.R = int(self.perm["offsets"][-1])

    def src(self, name):
        return {"x": self.di.x, "dy": self.di.dy, "dh": self.dh, "act": self.h}[name]

    def gpu(self, name, prob=None):
        return moe.moe_mx_quantize_wgrad(prob or self.prob, self.routing, self.src(name), KINDS[name])

    def oracle_values(self, name, rows=None):
        """Exact values of the routed rows (all, or the slice ``rows``) of operand ``name``."""
        rows = slice(0, self.R) if rows is None else rows
        tok = self.perm["row_tok"][rows]
        if name in ("x", "dy"):
            return oracle.decode(self.di.host[name][tok], "bf16")
        if name == "dh":
            return bf16_bits_to_f32(self.dh_bits[rows]).astype(np.float64)
        return oracle.act_p_f32(bf16_bits_to_f32(self.h_bits[rows]), self.p[rows]).astype(np.float64)


def _slice_major(a, per):
    """Oracle codes [cols, P] (per = 64) or scales [cols, P/32] (per = 2) ->
    the library's slice-major [P/64, cols, per]."""
    return a.reshape(a.shape[0], -1, per).transpose(1, 0, 2)


def _u8(t):
    return t.cpu().numpy().astype(np.uint8)


@pytest.mark.parametrize("name", SMALL)
def test_mx_quantize_wgrad_bytes_equal_the_oracle(name):
    print(f"mx wgrad quantise {name}", flush=True)
    case = Case(_cfg(name))
    off = case.perm["offsets"]
    for op in ("x", "dy", "dh", "act"):
        codes, scales = case.gpu(op)
        torch.cuda.synchronize()
        rc, rs, poff = oracle.mx_quantize_expert_rows(case.oracle_values(op), off)
        P = int(poff[-1])
        assert P // 64 <= codes.shape[0]
        assert np.array_equal(_u8(codes[: P // 64]), _slice_major(rc, 64)), op
        assert np.array_equal(_u8(scales[: P // 64]), _slice_major(rs, 2)), op


def _expert_check(checks, e, got1, got2, enc, p0, p1):
    """dW1_e and dW2_e against the oracle (operands ``enc``: columns p0..p1
    of the oracle's row-quantised encodings): the float32 accumulation
    bound per element, and the rel-L2 pieces."""
    def deq(op):
        c, sc = enc[op][0], enc[op][1]
        return oracle.mx_dequantize(c[:, p0:p1], sc[:, p0 // 32: p1 // 32])
    k = p1 - p0
    for name, got, a, b in (("dw1", got1, "x", "dh"), ("dw2", got2, "act", "dy")):
        ref = dict(oracle.mx_wgrad(enc[a][0][:, p0:p1], enc[a][1][:, p0 // 32: p1 // 32],
                                   enc[b][0][:, p0:p1], enc[b][1][:, p0 // 32: p1 // 32], [0, k]))[0]
        abs_terms = np.abs(deq(a)) @ np.abs(deq(b)).T
        got = to_host(got)
        bound = mx_block_bound(enc[a][1][:, p0 // 32: p1 // 32], enc[b][1][:, p0 // 32: p1 // 32]) + \
            fp32_sum_bound(abs_terms, k // 64)
        checks[name].add(got, ref, bound, ("expert", e))
        checks[name + "_l2"].add(got, ref, ("expert", e))


def _new_checks():
    return {"dw1": ElementBound("dw1"), "dw2": ElementBound("dw2"),
            "dw1_l2": Piecewise("dw1", MX_REL_TOL, row_tol=1.0), "dw2_l2": Piecewise("dw2", MX_REL_TOL, row_tol=1.0)}


def _report(checks, label):
    print(f"  {label} dw1 rel-L2 {checks['dw1_l2'].rel():.3e}, worst error / bound {checks['dw1'].worst:.3f}; "
          f"dw2 rel-L2 {checks['dw2_l2'].rel():.3e}, worst error / bound {checks['dw2'].worst:.3f}", flush=True)
    fails = [f for n in ("dw1", "dw2", "dw1_l2", "dw2_l2") for f in checks[n].failures()]
    assert not fails, fails


def _wgrad_check(case, dw1, dw2, label=""):
    """dW1 / dW2 of every local expert against the oracle."""
    off = case.perm["offsets"]
    enc = {op: oracle.mx_quantize_expert_rows(case.oracle_values(op), off) for op in KINDS}
    poff = enc["x"][2]
    checks = _new_checks()
    for e in range(case.prob.local):
        _expert_check(checks, e, dw1[e], dw2[e], enc, int(poff[e]), int(poff[e + 1]))
    _report(checks, label)


@pytest.mark.parametrize("name", SMALL)
def test_mx_wgrad_parity(name):
    print(f"mx wgrad {name}", flush=True)
    case = Case(_cfg(name))
    ops = [case.gpu(op) for op in ("x", "dh", "act", "dy")]
    dw1 = torch.full((case.prob.local, case.cfg.d_model, case.cfg.d_ffn), float("nan"), device="cuda")
    dw2 = torch.full((case.prob.local, case.cfg.d_ffn, case.cfg.d_model), float("nan"), device="cuda")
    moe.moe_mx_wgrad(case.prob, case.routing, *ops, dw1=dw1, dw2=dw2)
    torch.cuda.synchronize()
    # every element written (empty experts: zeros)
    assert not torch.isnan(dw1).any() and not torch.isnan(dw2).any()
    _wgrad_check(case, dw1, dw2, label=name)


def test_mx_wgrad_bits_identical_under_shuffles_and_poisoned_buffers():
    """Codes, scales and both dW bit for bit under shuffled launch orders,
    with every output pre-filled with garbage."""
    cfg = CONFIGS["bf16_e8k2"]
    case = Case(cfg)
    ref = None
    for seed, fill in ((0, 0), (5, 171), (0xFACE, 255), (0x9E3779B97F4A7C15, 7)):
        ps = case.prob.with_seed(seed)
        ops = []
        for op in ("x", "dh", "act", "dy"):
            cols = cfg.d_model if op in ("x", "dy") else cfg.d_ffn
            rp = moe.moe_mx_wgrad_rows(ps)
            c = torch.full((rp // 64, cols, 64), fill, dtype=torch.uint8, device="cuda")
            s = torch.full((rp // 64, cols, 2), fill, dtype=torch.uint8, device="cuda")
            ops.append(moe.moe_mx_quantize_wgrad(ps, case.routing, case.src(op), KINDS[op], c, s))
        dw1 = torch.full((ps.local, cfg.d_model, cfg.d_ffn), float(fill), device="cuda")
        dw2 = torch.full((ps.local, cfg.d_ffn, cfg.d_model), float(fill), device="cuda")
        moe.moe_mx_wgrad(ps, case.routing, *ops, dw1=dw1, dw2=dw2)
        P = int(oracle.mx_pad_offsets(case.perm["counts"])[-1])
        fps = [moe.moe_fingerprint(c[: P // 64].contiguous())[1] for c, _ in ops]
        fps += [moe.moe_fingerprint(s[: P // 64].contiguous())[1] for _, s in ops]
        fps += [moe.moe_fingerprint(dw1)[1], moe.moe_fingerprint(dw2)[1]]
        ref = fps if ref is None else ref
        assert fps == ref, seed


def test_mx_wgrad_encodings_beyond_2gib():
    """Encodings of routed rows past 2 GiB (160000 tokens top-2 of 64 experts
    at d_ffn 8192: the dh and act codes are 2.6 GB each): the quantiser's
    bytes and dW1 / dW2 of the first expert and of the last two, whose
    slices start past 2 GiB, against the oracle.  h and dh rows repeat one
    seeded 4096-row block (both sides read the same rows)."""
    cfg = Config("mx_2gib_e64k2", 160000, 256, 8192, 64, 2, 0, 64, "bf16", 1, 35)
    prob = moe.Problem.from_config(cfg)
    di = device_inputs(cfg)
    routing = moe.moe_route(prob, di.logits)
    rc, F = prob.rows_cap, cfg.d_ffn
    rng = np.random.default_rng([cfg.seed, 85])
    reps = (rc + 4095) // 4096
    h_bits = np.tile(f32_to_bf16_bits((rng.standard_normal((4096, F)) * 0.5).astype(np.float32)), (reps, 1))[:rc]
    dh_bits = np.tile(f32_to_bf16_bits((rng.standard_normal((4096, F)) * 0.01).astype(np.float32)), (reps, 1))[:rc]
    p = rng.uniform(0.02, 1.0, rc).astype(np.float32)
    routing.row_prob.copy_(torch.from_numpy(p).cuda())
    h, dh = _bits_dev(h_bits), _bits_dev(dh_bits)
    print("[mx > 2 GiB] HIP path", flush=True)
    ops = {op: moe.moe_mx_quantize_wgrad(prob, routing, {"x": di.x, "dy": di.dy, "dh": dh, "act": h}[op], KINDS[op])
           for op in ("x", "dh", "act", "dy")}
    dw1, dw2 = moe.moe_mx_wgrad(prob, routing, ops["x"], ops["dh"], ops["act"], ops["dy"])
    torch.cuda.synchronize()
    idx, _ = oracle.route(di.host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, cfg.num_local)
    off = perm["offsets"].astype(np.int64)
    poff = oracle.mx_pad_offsets(perm["counts"].astype(np.int64))
    assert int(poff[-1]) * F > (2 << 30) and int(poff[-2]) * F > (2 << 30)

    def values(op, lo, hi):
        tok = perm["row_tok"][lo:hi]
        if op in ("x", "dy"):
            return oracle.decode(di.host[op][tok], "bf16")
        if op == "dh":
            return bf16_bits_to_f32(dh_bits[lo:hi]).astype(np.float64)
        return oracle.act_p_f32(bf16_bits_to_f32(h_bits[lo:hi]), p[lo:hi]).astype(np.float64)

    checks = _new_checks()
    for e in (0, cfg.num_local - 2, cfg.num_local - 1):
        print(f"[mx > 2 GiB] expert {e}", flush=True)
        lo, hi = int(off[e]), int(off[e + 1])
        p0, p1 = int(poff[e]), int(poff[e + 1])
        enc = {op: oracle.mx_quantize_expert_rows(values(op, lo, hi), np.array([0, hi - lo])) for op in KINDS}
        for op in KINDS:
            c, s = ops[op]
            assert np.array_equal(_u8(c[p0 // 64: p1 // 64]), _slice_major(enc[op][0], 64)), (e, op)
            assert np.array_equal(_u8(s[p0 // 64: p1 // 64]), _slice_major(enc[op][1], 2)), (e, op)
        _expert_check(checks, e, dw1[e], dw2[e], enc, 0, p1 - p0)
    _report(checks, "[mx > 2 GiB]")


def test_mx_wgrad_full_size_latent_streamed():
    """The 512-expert top-22 layer at its full size, in the launch the bench
    times: every expert's operand bytes and dW1 / dW2 against the oracle,
    which encodes and multiplies one expert's rows at a time."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = CONFIGS["latent_e512k22"]
    print("[latent mx wgrad] inputs", flush=True)
    case = Case(cfg)
    ops = {op: case.gpu(op) for op in ("x", "dh", "act", "dy")}
    dw1, dw2 = moe.moe_mx_wgrad(case.prob, case.routing, ops["x"], ops["dh"], ops["act"], ops["dy"])
    torch.cuda.synchronize()
    counts = case.perm["counts"].astype(np.int64)
    off = case.perm["offsets"].astype(np.int64)
    poff = oracle.mx_pad_offsets(counts)
    P = int(poff[-1])
    host = {op: (_u8(c[: P // 64]), _u8(s[: P // 64])) for op, (c, s) in ops.items()}
    checks = _new_checks()

    def oracle_expert(e):
        lo, hi = int(off[e]), int(off[e + 1])
        one = np.array([0, hi - lo])
        return e, {op: oracle.mx_quantize_expert_rows(case.oracle_values(op, slice(lo, hi)), one) for op in KINDS}

    with ThreadPoolExecutor(16) as pool:
        for b0 in range(0, cfg.num_local, 64):
            print(f"[latent mx wgrad] experts {b0}..{b0 + 63}", flush=True)
            for e, enc in pool.map(oracle_expert, range(b0, min(b0 + 64, cfg.num_local))):
                p0, p1 = int(poff[e]), int(poff[e + 1])
                for op in KINDS:
                    assert np.array_equal(host[op][0][p0 // 64: p1 // 64], _slice_major(enc[op][0], 64)), (e, op)
                    assert np.array_equal(host[op][1][p0 // 64: p1 // 64], _slice_major(enc[op][1], 2)), (e, op)
                _expert_check(checks, e, dw1[e], dw2[e], enc, 0, p1 - p0)
    _report(checks, "[latent mx wgrad]")
