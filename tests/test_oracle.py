"""Pins of the CPU oracle against facts that do not come from the oracle itself:
brute force on tiny inputs, closed forms, finite differences, invariants and
homogeneity (Euler) identities.  A planted mistake in the oracle must fail at
least one of them (see the mutation tests at the end)."""
import math

import numpy as np
import pytest

import oracle
from oracle import moe as om
from synth import CONFIGS, make_inputs


def _rand_problem(rng, T=7, D=6, F=10, E=4, k=2, scale=1.0):
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, D)) * scale
    w1 = rng.standard_normal((E, D, F)) * scale
    w2 = rng.standard_normal((E, F, D)) * scale
    dy = rng.standard_normal((T, D))
    return logits, x, w1, w2, dy


# ------------------------------------------------------------------ routing
def _route_brute(logits, k):
    T, E = logits.shape
    idx = np.zeros((T, k), np.int32)
    prob = np.zeros((T, k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        sel = order[:k]
        idx[t] = sel
        m = max(float(logits[t, e]) for e in sel)
        w = [math.exp(float(logits[t, e]) - m) for e in sel]
        prob[t] = [v / sum(w) for v in w]
    return idx, prob


@pytest.mark.parametrize("seed", range(5))
def test_route_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    T, E, k = 40, 9, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # constructed exact ties, +-0 pairs and a repeated maximum
    logits[0, :] = 1.0
    logits[1, 2], logits[1, 5] = logits[1, 5], logits[1, 5]
    logits[2, :] = 0.0
    logits[2, 1] = -0.0
    logits[2, 4] = -0.0
    logits[3, 7] = logits[3, 3] = 10.0
    idx, prob = om.route(logits, k)
    bidx, bprob = _route_brute(logits, k)
    np.testing.assert_array_equal(idx, bidx)
    np.testing.assert_allclose(prob, bprob, rtol=1e-14, atol=0)
    np.testing.assert_allclose(prob.sum(1), 1.0, rtol=1e-14)


def test_route_negative_zero_is_equal_to_zero():
    logits = np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32)
    idx, prob = om.route(logits, 3)
    assert idx.tolist() == [[0, 1, 3]]
    np.testing.assert_allclose(prob, [[1 / 3] * 3], rtol=1e-15)


def test_route_full_softmax_when_k_equals_e():
    from scipy.special import softmax
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((16, 6)).astype(np.float32) * 3
    idx, prob = om.route(logits, 6)
    ref = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(prob, np.take_along_axis(ref, idx, 1), rtol=1e-13)
    # slot order is descending probability
    assert np.all(np.diff(prob, axis=1) <= 0)


# ------------------------------------------------------------------ permute
def _permute_brute(topk_idx, eb, el):
    T, k = topk_idx.shape
    lists = [[] for _ in range(el)]
    for t in range(T):
        for j in range(k):
            e = int(topk_idx[t, j])
            if eb <= e < eb + el:
                lists[e - eb].append(t * k + j)
    return lists


@pytest.mark.parametrize("eb,el", [(0, 6), (2, 3), (5, 1)])
def test_permute_brute_force_and_invariants(eb, el):
    rng = np.random.default_rng(3)
    T, E, k = 50, 6, 3
    idx, _ = om.route(rng.standard_normal((T, E)).astype(np.float32), k)
    p = om.permute(idx, eb, el)
    lists = _permute_brute(idx, eb, el)
    assert p["counts"].tolist() == [len(l) for l in lists]
    assert p["row_src"].tolist() == [i for l in lists for i in l]
    off = p["offsets"]
    assert off[0] == 0 and np.all(np.diff(off) == p["counts"])
    R = int(off[-1])
    assert np.all(p["slot_row"][p["row_src"]] == np.arange(R))
    assert np.sum(p["slot_row"] >= 0) == R
    for e in range(el):  # stability: flat index increasing inside each expert
        assert np.all(np.diff(p["row_src"][off[e]:off[e + 1]]) > 0)
    assert np.all(p["counts"] <= T)
    np.testing.assert_array_equal(p["row_tok"], p["row_src"] // k)
    if el == E:
        assert R == T * k


# ------------------------------------------------------------------ forward
def _forward_per_token(x, w1, w2, idx, prob):
    T, k = idx.shape
    y = np.zeros_like(x)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            h = x[t] @ w1[e]
            y[t] += prob[t, j] * (np.maximum(h, 0) ** 2 @ w2[e])
    return y


def test_forward_matches_per_token_evaluation():
    rng = np.random.default_rng(5)
    logits, x, w1, w2, _ = _rand_problem(rng, T=12, E=5, k=3)
    idx, prob = om.route(logits, 3)
    perm = om.permute(idx, 0, 5)
    out = om.forward(x, w1, w2, prob, perm, 3)
    np.testing.assert_allclose(out["y"], _forward_per_token(x, w1, w2, idx, prob), rtol=1e-12, atol=1e-12)


def test_forward_single_expert_is_dense_mlp():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((9, 4))
    w1 = rng.standard_normal((1, 4, 8))
    w2 = rng.standard_normal((1, 8, 4))
    idx, prob = om.route(np.zeros((9, 1), np.float32), 1)
    assert np.all(prob == 1.0)
    perm = om.permute(idx, 0, 1)
    y = om.forward(x, w1, w2, prob, perm, 1)["y"]
    h = x @ w1[0]
    ref = np.where(h > 0, h * h, 0.0) @ w2[0]
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_permute_then_unpermute_is_identity():
    rng = np.random.default_rng(7)
    T, E, k = 30, 7, 4
    idx, prob = om.route(rng.standard_normal((T, E)).astype(np.float32), k)
    perm = om.permute(idx, 0, E)
    x = rng.standard_normal((T, 5))
    rows = x[perm["row_tok"]]
    np.testing.assert_allclose(om.combine_rows(rows, perm["slot_row"], prob, T, k), x, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(om.combine_rows(rows, perm["slot_row"], np.ones((T, k)), T, k), k * x)


# ------------------------------------------------------------------ backward
def _setup_small(seed=8, T=6, D=5, F=7, E=3, k=2):
    rng = np.random.default_rng(seed)
    logits, x, w1, w2, dy = _rand_problem(rng, T=T, D=D, F=F, E=E, k=k)
    idx, prob = om.route(logits, k)
    perm = om.permute(idx, 0, E)
    fwd = om.forward(x, w1, w2, prob, perm, k)
    bwd = om.backward(x, w1, w2, fwd["h"], dy, prob, perm, k)
    return x, w1, w2, dy, idx, prob, perm, fwd, bwd


def _fd(f, arr, eps):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + eps
        fp = f()
        arr[i] = old - eps
        fm = f()
        arr[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_dprob_finite_difference_exact():
    x, w1, w2, dy, idx, prob, perm, fwd, bwd = _setup_small()
    k = prob.shape[1]
    p = prob.copy()
    g = _fd(lambda: om.layer_loss(x, w1, w2, p, perm, k, dy), p, 0.5)  # L is linear in p
    np.testing.assert_allclose(bwd["dprob"], g, rtol=1e-10, atol=1e-12)
    # identity: sum_{t,j} p * dprob = L
    L = om.layer_loss(x, w1, w2, prob, perm, k, dy)
    assert abs(np.sum(prob * bwd["dprob"]) - L) <= 1e-12 * max(1, abs(L))


@pytest.mark.parametrize("name", ["x", "w1", "w2"])
def test_gradients_finite_difference(name):
    x, w1, w2, dy, idx, prob, perm, fwd, bwd = _setup_small()
    k = prob.shape[1]
    arrs = dict(x=x, w1=w1, w2=w2)
    g = _fd(lambda: om.layer_loss(x, w1, w2, prob, perm, k, dy), arrs[name], 1e-6)
    ref = dict(x=bwd["dx"], w1=bwd["dw1"], w2=bwd["dw2"])[name]
    np.testing.assert_allclose(ref, g, rtol=1e-6, atol=1e-7)


def test_act_p_gives_dw2():
    """dW2 of an expert equals act_p^T dy over its rows, act_p = p relu(h)^2."""
    x, w1, w2, dy, idx, prob, perm, fwd, bwd = _setup_small(seed=13)
    off = perm["offsets"]
    p_rows = prob.reshape(-1)[perm["row_src"]]
    np.testing.assert_allclose(bwd["act_p"], p_rows[:, None] * np.maximum(fwd["h"], 0) ** 2, rtol=1e-14)
    for e in range(w1.shape[0]):
        s, t = off[e], off[e + 1]
        np.testing.assert_allclose(bwd["act_p"][s:t].T @ dy[perm["row_tok"][s:t]], bwd["dw2"][e], rtol=1e-12,
                                   atol=1e-14)


def test_dx_rows_sum_to_dx_and_empty_expert_zero():
    rng = np.random.default_rng(9)
    T, E, k = 10, 5, 2
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 4] = -100.0                     # expert 4 never selected
    x, w1, w2, dy = (rng.standard_normal((T, 4)), rng.standard_normal((E, 4, 6)),
                     rng.standard_normal((E, 6, 4)), rng.standard_normal((T, 4)))
    idx, prob = om.route(logits, k)
    perm = om.permute(idx, 0, E)
    assert perm["counts"][4] == 0
    fwd = om.forward(x, w1, w2, prob, perm, k)
    bwd = om.backward(x, w1, w2, fwd["h"], dy, prob, perm, k)
    assert np.all(bwd["dw1"][4] == 0) and np.all(bwd["dw2"][4] == 0)


def test_euler_identities():
    """o is homogeneous of degree 2 in (W1) and in (x), degree 1 in W2."""
    rng = np.random.default_rng(10)
    logits, x, w1, w2, dy = _rand_problem(rng, T=40, D=8, F=12, E=5, k=2)
    idx, prob = om.route(logits, 2)
    perm = om.permute(idx, 0, 5)
    fwd = om.forward(x, w1, w2, prob, perm, 2)
    bwd = om.backward(x, w1, w2, fwd["h"], dy, prob, perm, 2)
    p_rows = prob.reshape(-1)[perm["row_src"]]
    dprob_rows = bwd["dprob"].reshape(-1)[perm["row_src"]]
    off = perm["offsets"]
    for e in range(5):
        Le = np.sum(p_rows[off[e]:off[e + 1]] * dprob_rows[off[e]:off[e + 1]])
        np.testing.assert_allclose(np.sum(bwd["dw1"][e] * w1[e]), 2 * Le, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(np.sum(bwd["dw2"][e] * w2[e]), Le, rtol=1e-10, atol=1e-12)
    lhs = np.sum(bwd["dx"] * x, axis=1)
    rhs = 2 * np.sum(prob * bwd["dprob"], axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10, atol=1e-12)


def test_shard_equals_slice_of_full_layer():
    """An expert shard computes exactly the full layer's rows of its experts."""
    rng = np.random.default_rng(12)
    logits, x, w1, w2, dy = _rand_problem(rng, T=20, E=6, k=3)
    idx, prob = om.route(logits, 3)
    full = om.permute(idx, 0, 6)
    shard = om.permute(idx, 2, 2)
    ff = om.forward(x, w1, w2, prob, full, 3)
    fb = om.backward(x, w1, w2, ff["h"], dy, prob, full, 3)
    sf = om.forward(x, w1[2:4], w2[2:4], prob, shard, 3, combine=False)
    sb = om.backward(x, w1[2:4], w2[2:4], sf["h"], dy, prob, shard, 3, combine=False)
    lo, hi = full["offsets"][2], full["offsets"][4]
    np.testing.assert_array_equal(shard["row_src"], full["row_src"][lo:hi])
    np.testing.assert_allclose(sf["o_rows"], ff["o_rows"][lo:hi], rtol=1e-13)
    np.testing.assert_allclose(sb["dx_rows"], fb["dx_rows"][lo:hi], rtol=1e-13)
    np.testing.assert_allclose(sb["dw1"], fb["dw1"][2:4], rtol=1e-13)
    local = (idx >= 2) & (idx < 4)
    np.testing.assert_allclose(sb["dprob"][local], fb["dprob"][local], rtol=1e-13)
    assert np.all(sb["dprob"][~local] == 0)


def test_decode_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x0001], np.uint16)
    v = om.decode(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 0.0 and math.copysign(1, v[3]) == -1
    assert v[4] == 3.140625 and v[5] == 2.0 ** -133


# ------------------------------------------------------------------ workloads
def test_tiny_config_end_to_end_consistency():
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg)
    idx, prob = om.route(inp["logits"], cfg.top_k)
    perm = om.permute(idx, 0, cfg.num_experts)
    x, w1, w2, dy = (om.decode(inp[n], "f32") for n in ("x", "w1", "w2", "dy"))
    fwd = om.forward(x, w1, w2, prob, perm, cfg.top_k)
    np.testing.assert_allclose(fwd["y"], _forward_per_token(x, w1, w2, idx, prob), rtol=1e-12, atol=1e-18)
    assert int(perm["offsets"][-1]) == cfg.tokens * cfg.top_k


# ------------------------------------------------------------------ mutation
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle and check a pin fails."""
    base_act_grad = om._act_grad

    def check_grads():
        x, w1, w2, dy, idx, prob, perm, fwd, bwd = _setup_small(seed=21)
        k = prob.shape[1]
        g = _fd(lambda: om.layer_loss(x, w1, w2, prob, perm, k, dy), x, 1e-6)
        return np.allclose(bwd["dx"], g, rtol=1e-6, atol=1e-7)

    assert check_grads()
    monkeypatch.setattr(om, "_act_grad", lambda h: np.maximum(h, 0.0))     # dropped factor 2
    assert not check_grads()
    monkeypatch.setattr(om, "_act_grad", lambda h: 2.0 * h)                # dropped the ReLU mask
    assert not check_grads()
    monkeypatch.setattr(om, "_act_grad", base_act_grad)
    assert check_grads()
