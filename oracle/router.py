"""Plain fp64 CPU definition of the router backward: the step directly upstream
of dprob.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Written for a reader to
check by eye; no blocking, fusion or reordering.

Source: "Trillion-Parameter Pretraining Goes Bitwise-Deterministic" (English
digest), section "Interpretation": the grouped-GEMM epilogue produces dprob,
one value per (token, selected expert); the router is what consumes it.  The
pages do not describe the router itself; the readings used here are:
  * a linear router without bias: logits[t, e] = <x_t, wr_e>, with router
    weights wr [E, D] (one row per expert);
  * the layer's routing readings: the k experts with the largest logits are
    selected (a piecewise-constant choice, so no gradient flows through it)
    and p_t = softmax over the k selected logits.
With dprob[t, j] the gradient of the loss with respect to p[t, j]:
  * dlogits[t, e_j] = sum_i dprob_i * d p_i / d l_j
                    = p_j * (dprob_j - sum_i p_i dprob_i),
    and 0 for the experts that token t did not select;
  * dwr = dlogits^T x   ([E, D]);
  * dx_router = dlogits wr   ([T, D]).
"""
import numpy as np


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """logits[t, e] = <x_t, wr_e> (float64)."""
    return np.asarray(x, np.float64) @ np.asarray(wr, np.float64).T


def router_probs(logits: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    """Softmax over the k selected logits of each token (max-subtracted)."""
    sel = np.take_along_axis(np.asarray(logits, np.float64), np.asarray(topk_idx, np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def router_dlogits(topk_idx: np.ndarray, topk_prob: np.ndarray, dprob: np.ndarray, num_experts: int) -> np.ndarray:
    """Dense [T, E] gradient of the loss with respect to the logits, given the
    gradient dprob [T, k] with respect to the selected probabilities."""
    idx = np.asarray(topk_idx, np.int64)
    p = np.asarray(topk_prob, np.float64)
    g = np.asarray(dprob, np.float64)
    T, k = idx.shape
    out = np.zeros((T, num_experts))
    for t in range(T):
        s = sum(p[t, i] * g[t, i] for i in range(k))
        for j in range(k):
            out[t, idx[t, j]] = p[t, j] * (g[t, j] - s)
    return out


def router_backward(topk_idx, topk_prob, dprob, x, wr) -> dict:
    """dlogits [T, E], dwr [E, D] and dx_router [T, D], all float64.  x and wr
    are given as float64 values (decode storage types first)."""
    x = np.asarray(x, np.float64)
    wr = np.asarray(wr, np.float64)
    dl = router_dlogits(topk_idx, topk_prob, dprob, wr.shape[0])
    return {"dlogits": dl, "dwr": dl.T @ x, "dx": dl @ wr}


def router_loss(logits: np.ndarray, topk_idx: np.ndarray, dprob: np.ndarray) -> float:
    """L = sum_t sum_j p[t, j] * dprob[t, j] with p recomputed from the logits
    over the given (fixed) selection.  dprob acts as a constant, so dL/dp is
    dprob and dL/dlogits is the router backward's dlogits."""
    p = router_probs(logits, topk_idx)
    return float(np.sum(p * np.asarray(dprob, np.float64)))
