"""Deterministic train steps of the layer with the progressive tracer:
independent runs are bit-identical at every step and every traced tensor, a
resumed run equals the continuous one, the localiser finds a planted
divergence at the step and the op where it enters (also when it never reaches
the loss), and one step agrees with the CPU oracle (router logits, the SGD
update and the runtime copies)."""
import fractions

import numpy as np
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
import oracle
from bitwise_deterministic_moe_amd import trace
from synth import CONFIGS, make_batch, make_router_inputs
from synth.inputs import f32_to_bf16_bits
from test_gpu_parity import EDGE
from harness import rel_l2, to_host

pytestmark = pytest.mark.gpu

CASES = ["tiny_fp32", "ragged_bf16"]


def _cfg(name):
    return CONFIGS.get(name) or EDGE[name]


@pytest.mark.parametrize("name", CASES)
def test_independent_runs_are_bit_identical_at_every_op(name):
    cfg = _cfg(name)
    print(f"trace reproducibility {name}", flush=True)
    _, a = trace.run(cfg, 4, "ops")
    _, b = trace.run(cfg, 4, "ops")
    assert len(a.records) > 4 * 20
    assert trace.first_divergence(a.records, b.records) is None


@pytest.mark.parametrize("name", CASES)
def test_resume_from_checkpoint_equals_the_continuous_run(name, tmp_path):
    cfg = _cfg(name)
    print(f"trace resume {name}", flush=True)
    full_st, full = trace.run(cfg, 4, "phases")
    st, _ = trace.run(cfg, 2, "phases")
    ck = str(tmp_path / "ck.npz")
    st.save(ck)
    del st
    torch.cuda.empty_cache()
    st2 = trace.TrainState.load(ck, moe.Problem.from_config(cfg))
    assert st2.step == 2
    st2, tail = trace.run(cfg, 4, "phases", st=st2)
    ref = [r for r in full.records if r.step >= 2]
    assert trace.first_divergence(ref, tail.records) is None
    for n in ("w1", "w2", "wr"):
        assert moe.moe_fingerprint(st2.master[n])[1] == moe.moe_fingerprint(full_st.master[n])[1]
        assert moe.moe_fingerprint(st2.runtime[n])[1] == moe.moe_fingerprint(full_st.runtime[n])[1]


def _flip_runtime_w1(step_at):
    def hook(step, where, st):
        if step == step_at and where == "before_forward":
            w = st.runtime["w1"].view(-1)
            bits = w.view(torch.int16) if w.dtype == torch.bfloat16 else w.view(torch.int32)
            bits[5] ^= 1 << 6                      # a mantissa bit of one weight of expert 0
    return hook


def _flip_master_w2_low_bit(step_at):
    def hook(step, where, st):
        if step == step_at and where == "before_forward":
            st.master["w2"].view(-1).view(torch.int32)[3] ^= 1   # below the bf16 runtime copy's precision
    return hook


def test_localiser_finds_the_step_and_op_of_a_planted_flip():
    cfg = EDGE["ragged_bf16"]
    out = trace.localise(cfg, 4, hook_b=_flip_runtime_w1(2))
    print(out, flush=True)
    assert out["metric"]["step"] == 2
    assert out["phase"]["step"] == 2 and out["phase"]["name"] == "y"
    assert out["op"]["step"] == 2 and out["op"]["name"] == "h"      # the first tensor computed from W1


def test_localiser_finds_a_divergence_that_precedes_the_loss():
    # a one-ulp change of an fp32 master below the bf16 runtime precision:
    # the runtime weights and the loss stay equal; the optimizer's master is
    # the first (and here only) divergent tensor
    cfg = EDGE["ragged_bf16"]
    out = trace.localise(cfg, 3, hook_b=_flip_master_w2_low_bit(1))
    print(out, flush=True)
    assert out["metric"] is None
    assert out["phase"]["step"] == 1 and out["phase"]["name"] == "master_w2"


def test_one_step_against_the_oracle():
    cfg = EDGE["ragged_bf16"]
    prob = moe.Problem.from_config(cfg)
    st = trace.initial_state(cfg)
    w0 = {n: st.master[n].cpu().numpy().ravel().copy() for n in st.master}
    # the step's gradients, recomputed from the initial state with the same
    # calls (the step is deterministic, so these are the ones it applies)
    b = make_batch(cfg, 0)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)  # noqa
    x, dy = up(b["x"]), up(b["dy"])
    R = st.runtime
    logits = moe.moe_router_fwd(prob, x, R["wr"])
    routing, h, _ = moe.moe_fwd(prob, logits, x, R["w1"], R["w2"])
    _, dprob, dh = moe.moe_bwd_dgrad_dprob(prob, routing, dy, R["w1"], R["w2"], h)
    dw1, dw2 = moe.moe_bwd_wgrad(prob, routing, x, dy, h, dh)
    _, dwr, _ = moe.moe_router_bwd(prob, routing, dprob, x, R["wr"])
    torch.cuda.synchronize()
    grads = {n: t.cpu().numpy().ravel().copy() for n, t in (("w1", dw1), ("w2", dw2), ("wr", dwr))}
    # router logits against the oracle (fp32 dot products against fp64)
    ref = oracle.router_logits(oracle.decode(b["x"], cfg.dtype), oracle.decode(make_router_inputs(cfg)["wr"], cfg.dtype))
    assert rel_l2(to_host(logits), ref) <= 1e-5

    st, _ = trace.run(cfg, 1, "phases", st=st)
    lr = fractions.Fraction(np.float32(st.lr).item())
    rng = np.random.default_rng(7)
    for n in ("w1", "w2", "wr"):
        m1 = st.master[n].cpu().numpy().ravel()
        for i in rng.choice(m1.size, 200, replace=False):
            exact = fractions.Fraction(w0[n][i].item()) - lr * fractions.Fraction(grads[n][i].item())
            assert _rne32(exact) == m1[i], (n, int(i))
        rt = st.runtime[n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()
        assert np.array_equal(rt, f32_to_bf16_bits(m1))


def _rne32(q: fractions.Fraction) -> np.float32:
    """Round a rational to the nearest float32, ties to even (exact)."""
    lo = np.float32(float(q))
    cands = [lo, np.nextafter(lo, np.float32(np.inf)), np.nextafter(lo, np.float32(-np.inf))]
    best = min(cands, key=lambda c: (abs(fractions.Fraction(c.item()) - q),
                                     int(np.array([c], np.float32).view(np.int32)[0]) & 1))
    return best


def test_mx_train_steps_are_bit_identical_and_fingerprint_the_encoded_buffers():
    cfg = EDGE["ragged_bf16"]
    print("trace mx reproducibility", flush=True)
    _, a = trace.run(cfg, 3, "ops", mx=True)
    _, b = trace.run(cfg, 3, "ops", mx=True)
    assert trace.first_divergence(a.records, b.records) is None
    def names(op):
        return {r.name for r in a.records if r.op == op}

    def both(*ns):
        return {f"{n}_{k}" for n in ns for k in ("codes", "scales")}

    assert names("moe_mx_quantize") == both("x", "act", "dy", "w2", "dh", "w1")
    assert names("moe_mx_quantize_t") == both("w1t", "w2t")
    assert names("moe_mx_quantize_wgrad") == both("x", "dh", "act", "dy")
    assert names("moe_mx_fwd_fc1") == {"h"} and names("moe_mx_fwd_fc2") == {"y"}
    assert names("moe_mx_wgrad") == {"dw1", "dw2"} and not names("moe_fwd") - {
        "topk_idx", "topk_prob", "counts", "offsets", "row_src", "slot_row"}
    assert not names("moe_bwd_wgrad") and not names("moe_bwd_dgrad_dprob")
    assert all(r.dtype == "u8" for r in a.records if r.op.startswith("moe_mx_quantize"))
    nv = [r.name for r in a.records if r.op == "moe_nvfp4_quantize" and r.step == 0]
    assert nv == ["dh_codes", "dh_scales", "dh_tensor_scale"]
    # a different computation from the bf16 step: the traces part at step 0's
    # forward (same routing, then the MXFP8 encodings)
    _, c = trace.run(cfg, 3, "ops")
    d = trace.first_divergence(a.records, c.records)
    assert d is not None and d[1].step == 0 and d[1].phase == "forward"
