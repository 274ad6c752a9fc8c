"""Pins of the router-backward oracle against facts that do not come from the
oracle itself: central finite differences of the routing loss through
logits = x wr^T (the loss is smooth in the logits while the selection stays
fixed), the zero row sums of the softmax Jacobian, the k = 1 and k = E special
cases, and an independent automatic differentiation (torch, float64, CPU).
The mutation test at the end plants plausible mistakes in the oracle and
checks that a pin fails."""
import numpy as np
import pytest
import torch

import oracle
from oracle import router as orr


def _problem(seed, T=6, D=5, E=7, k=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D))
    dprob = rng.standard_normal((T, k))
    logits = orr.router_logits(x, wr)
    idx, _ = oracle.route(logits.astype(np.float32), k)
    p = orr.router_probs(logits, idx)
    return x, wr, dprob, logits, np.asarray(idx, np.int64), p


def _fd(f, a, eps=1e-6):
    g = np.zeros_like(a)
    for i in np.ndindex(a.shape):
        old = a[i]
        a[i] = old + eps
        fp = f()
        a[i] = old - eps
        fm = f()
        a[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("seed", range(4))
def test_dlogits_matches_finite_differences(seed):
    x, wr, dprob, logits, idx, p = _problem(seed)
    dl = orr.router_dlogits(idx, p, dprob, wr.shape[0])
    lg = logits.copy()
    g = _fd(lambda: orr.router_loss(lg, idx, dprob), lg)
    np.testing.assert_allclose(dl, g, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("seed", range(3))
def test_dwr_and_dx_match_finite_differences(seed):
    x, wr, dprob, logits, idx, p = _problem(seed)
    out = orr.router_backward(idx, p, dprob, x, wr)
    xx, ww = x.copy(), wr.copy()
    loss = lambda: orr.router_loss(orr.router_logits(xx, ww), idx, dprob)
    np.testing.assert_allclose(out["dwr"], _fd(loss, ww), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(out["dx"], _fd(loss, xx), rtol=1e-6, atol=1e-8)


def test_dlogits_rows_sum_to_zero_and_vanish_off_selection():
    x, wr, dprob, logits, idx, p = _problem(11, T=50, E=16, k=5)
    dl = orr.router_dlogits(idx, p, dprob, 16)
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-14)
    mask = np.zeros_like(dl, bool)
    np.put_along_axis(mask, idx, True, axis=1)
    assert np.all(dl[~mask] == 0.0)


def test_single_expert_selection_has_no_router_gradient():
    # softmax over one logit is the constant 1
    x, wr, dprob, logits, idx, p = _problem(5, k=1)
    out = orr.router_backward(idx, p, dprob, x, wr)
    assert np.all(out["dlogits"] == 0.0) and np.all(out["dwr"] == 0.0) and np.all(out["dx"] == 0.0)


@pytest.mark.parametrize("k", [2, 7])  # k = 7 = E: the full softmax
def test_matches_torch_autograd(k):
    x, wr, dprob, logits, idx, p = _problem(21, T=9, D=4, E=7, k=k)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(wr, requires_grad=True)
    lt = xt @ wt.T
    sel = torch.gather(lt, 1, torch.tensor(idx))
    loss = (torch.softmax(sel, dim=1) * torch.tensor(dprob)).sum()
    lt.retain_grad()
    loss.backward()
    out = orr.router_backward(idx, p, dprob, x, wr)
    np.testing.assert_allclose(out["dlogits"], lt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["dwr"], wt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_router_pins_catch_planted_mistakes(monkeypatch):
    x, wr, dprob, logits, idx, p = _problem(3)
    lg = logits.copy()
    fd = _fd(lambda: orr.router_loss(lg, idx, dprob), lg)
    xx, ww = x.copy(), wr.copy()
    loss = lambda: orr.router_loss(orr.router_logits(xx, ww), idx, dprob)
    fd_w, fd_x = _fd(loss, ww), _fd(loss, xx)
    base = orr.router_dlogits

    def dropped_mean(idx_, p_, g_, E):          # forgot the - sum_i p_i dprob_i term
        out = np.zeros((idx_.shape[0], E))
        np.put_along_axis(out, np.asarray(idx_, np.int64), np.asarray(p_) * np.asarray(g_), axis=1)
        return out

    def flipped_sign(idx_, p_, g_, E):
        return -base(idx_, p_, g_, E)

    for bad in (dropped_mean, flipped_sign):
        monkeypatch.setattr(orr, "router_dlogits", bad)
        assert not np.allclose(orr.router_dlogits(idx, p, dprob, wr.shape[0]), fd, rtol=1e-6, atol=1e-8)
    monkeypatch.setattr(orr, "router_dlogits", base)
    # transposed / wrong-operand products
    good = orr.router_backward(idx, p, dprob, x, wr)
    dl = good["dlogits"]
    assert not np.allclose(dl.T @ np.ones_like(x), fd_w, rtol=1e-6, atol=1e-8)
    assert not np.allclose(dl @ np.abs(wr), fd_x, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(good["dwr"], fd_w, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(good["dx"], fd_x, rtol=1e-6, atol=1e-8)
