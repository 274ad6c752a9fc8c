"""The comparison used by the GPU parity tests catches single-row and
single-slot mistakes that a whole-tensor rel-L2 lets through, and accepts the
rounding the path is allowed to make.

Every case runs on the CPU: "got" is the oracle's own output, either with the
storage-type rounding of the path applied (must pass) or with one planted
mistake (must fail)."""
import copy

import numpy as np
import pytest

import oracle
from compare import compare_full, tol_for
from synth import Config, make_inputs
from synth.inputs import bf16_bits_to_f32, f32_to_bf16_bits

# 8192 tokens: one wrong token row moves the whole-tensor rel-L2 of y or dx
# by about sqrt(2 / 8192) = 1.6e-2, below the 2e-2 bf16 bound
CFG = Config("compare_bf16", 8192, 256, 512, 8, 2, 0, 8, "bf16", 1, 31)
SHARD = Config("compare_shard_bf16", 600, 256, 256, 16, 4, 3, 4, "bf16", 0, 32)


def _bf16(a):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, dtype=np.float32))).astype(np.float64)


def _layer(cfg):
    host = make_inputs(cfg)
    idx, p = oracle.route(host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, cfg.num_local)
    x, w1, w2, dy = (oracle.decode(host[n], cfg.dtype) for n in ("x", "w1", "w2", "dy"))
    f = oracle.forward(x, w1, w2, p, perm, cfg.top_k, combine=bool(cfg.combine))
    b = oracle.backward(x, w1, w2, f["h"], dy, p, perm, cfg.top_k, combine=bool(cfg.combine))
    ref = dict(topk_prob=p, perm=perm, **f, **b)
    # what the path computes: h rounded to bf16 once, the backward on that h,
    # bf16 rounding of every storage-type output (dprob and dW stay float32)
    hb = _bf16(f["h"])
    bb = oracle.backward(x, w1, w2, hb, dy, p, perm, cfg.top_k, combine=bool(cfg.combine))
    got = dict(h=hb, dh=_bf16(bb["dh"]), dprob=bb["dprob"].astype(np.float32), dw1=bb["dw1"].astype(np.float32),
               dw2=bb["dw2"].astype(np.float32))
    if cfg.combine:
        got["y"], got["dx"] = _bf16(f["y"]), _bf16(bb["dx"])
    else:
        got["y"], got["dx"] = _bf16(f["o_rows"]), _bf16(bb["dx_rows"])
    return cfg, got, ref, (x, w1, w2, dy)


@pytest.fixture(scope="module")
def layer():
    return _layer(CFG)


@pytest.fixture(scope="module")
def shard():
    return _layer(SHARD)


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def test_rounded_oracle_passes(layer, shard):
    for cfg, got, ref, _ in (layer, shard):
        errs = compare_full(cfg.dtype, got, ref, bool(cfg.combine), cfg.top_k)
        # the rounding the path makes stays far inside every bound
        assert errs["dprob_worst_z"] < 6, errs
        assert max(v for n, v in errs.items() if n.endswith("worst_row")) < 1e-2, errs


@pytest.mark.parametrize("name", ["y", "dx"])
def test_one_wrong_token_row_fails(layer, name):
    cfg, got, ref, _ = layer
    bad = copy.deepcopy(got)
    bad[name][100] = bad[name][101]
    # the whole-tensor figure alone would let it through ...
    assert _rel(bad[name], ref[name]) < tol_for("bf16")
    # ... the per-row bound does not
    with pytest.raises(AssertionError, match=f"{name}: worst row"):
        compare_full(cfg.dtype, bad, ref, True, cfg.top_k)


@pytest.mark.parametrize("name", ["h", "dh"])
def test_one_wrong_routed_row_fails(layer, name):
    cfg, got, ref, _ = layer
    bad = copy.deepcopy(got)
    bad[name][7] = bad[name][8]
    assert _rel(bad[name], ref[name]) < tol_for("bf16")
    with pytest.raises(AssertionError, match=f"{name}: worst row"):
        compare_full(cfg.dtype, bad, ref, True, cfg.top_k)


def test_one_wrong_weight_gradient_row_fails(layer):
    cfg, got, ref, _ = layer
    bad = copy.deepcopy(got)
    bad["dw1"][3, 17] *= 1.3
    assert _rel(bad["dw1"], ref["dw1"]) < tol_for("bf16")
    with pytest.raises(AssertionError, match="dw1: worst row"):
        compare_full(cfg.dtype, bad, ref, True, cfg.top_k)


def test_swapped_dprob_slots_fail(layer):
    cfg, got, ref, _ = layer
    bad = copy.deepcopy(got)
    bad["dprob"][5, 0], bad["dprob"][5, 1] = got["dprob"][5, 1], got["dprob"][5, 0]
    assert _rel(bad["dprob"], ref["dprob"]) < tol_for("bf16")
    with pytest.raises(AssertionError, match="dprob: worst slot"):
        compare_full(cfg.dtype, bad, ref, True, cfg.top_k)


def test_dprob_slot_missing_one_n_tile_fails(layer):
    """A slot whose first 256-column N-tile partial was never added (the
    fault class the private slots guard against)."""
    cfg, got, ref, (x, w1, w2, dy) = layer
    perm, p = ref["perm"], ref["topk_prob"]
    t, j = 9, 1
    r = int(perm["slot_row"][t * cfg.top_k + j])
    e = int(np.searchsorted(perm["offsets"], r, side="right") - 1)
    g = dy[t] @ w2[e].T
    part0 = float(np.sum(g[:256] * np.maximum(ref["h"][r, :256], 0.0) ** 2))
    bad = copy.deepcopy(got)
    bad["dprob"][t, j] -= part0
    assert _rel(bad["dprob"], ref["dprob"]) < tol_for("bf16")
    with pytest.raises(AssertionError, match="dprob: worst slot"):
        compare_full(cfg.dtype, bad, ref, True, cfg.top_k)


def test_nonlocal_slot_must_be_zero(shard):
    cfg, got, ref, _ = shard
    bad = copy.deepcopy(got)
    i = int(np.nonzero(ref["perm"]["slot_row"] < 0)[0][0])
    bad["dprob"].reshape(-1)[i] = 1e-30
    with pytest.raises(AssertionError, match="non-local"):
        compare_full(cfg.dtype, bad, ref, False, cfg.top_k)


def test_shard_row_outputs_checked_per_row(shard):
    cfg, got, ref, _ = shard
    bad = copy.deepcopy(got)
    bad["dx"][3] *= 1.5
    with pytest.raises(AssertionError, match="dx: worst row"):
        compare_full(cfg.dtype, bad, ref, False, cfg.top_k)


def _f32_accumulate(terms, truncate=False):
    """Sequential float32 accumulation (round to nearest, or toward zero)."""
    s = np.float32(0.0)
    for t in terms:
        exact = float(s) + float(t)
        r = np.float32(exact)
        if truncate and abs(float(r)) > abs(exact):
            r = np.nextafter(r, np.float32(0.0))
        s = r
    return float(s)


def test_fp32_sum_bound_covers_nearest_and_truncating_accumulation():
    from compare import fp32_sum_bound
    rng = np.random.default_rng(7)
    for k in (1, 2, 64, 700):
        terms = (rng.standard_normal(k) * np.exp2(rng.integers(-8, 8, k))).astype(np.float32)
        exact = float(np.sum(terms.astype(np.float64)))
        bound = float(fp32_sum_bound(np.sum(np.abs(terms.astype(np.float64))), k))
        for trunc in (False, True):
            assert abs(_f32_accumulate(terms, trunc) - exact) <= bound, (k, trunc)
    # a missing block of 32 terms out of 700 breaks it
    terms = np.abs(rng.standard_normal(700)).astype(np.float32)
    bound = float(fp32_sum_bound(np.sum(terms.astype(np.float64)), 700))
    assert abs(_f32_accumulate(terms[32:]) - float(np.sum(terms.astype(np.float64)))) > bound


def test_element_bound_reports_the_worst_ratio():
    from compare import ElementBound
    c = ElementBound("t")
    c.add([1.0, 2.0], [1.0, 2.5], [0.1, 1.0], "a")
    assert not c.failures() and abs(c.worst - 0.5) < 1e-12
    c.add([0.0, 1.0], [0.0, 0.0], [0.0, 0.5], "b")
    assert c.failures() and c.worst_at[0] == "b"


def test_mx_block_bound_by_hand():
    from compare import MX_BLOCK_TAU, mx_block_bound
    a = np.array([[127, 130]], np.uint8)          # scales 2^0, 2^3
    b = np.array([[127, 125], [0, 0]], np.uint8)  # 2^0, 2^-2; 2^-127 twice
    got = mx_block_bound(a, b)
    want0 = MX_BLOCK_TAU * 448.0 ** 2 * (1.0 + 2.0 ** 1)
    assert got.shape == (1, 2) and abs(got[0, 0] - want0) <= 1e-12 * want0
    assert 0 < got[0, 1] < 1e-30
