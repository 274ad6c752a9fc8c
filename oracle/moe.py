"""Plain fp64 CPU definition of the MoE expert layer and its backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Written for a reader
to check by eye; no blocking, fusion or reordering.

Sources (the pages):
  * "Trillion-Parameter Pretraining Goes Bitwise-Deterministic" (English
    digest), section "Interpretation": the grouped-GEMM epilogue produces
    dprob per token, one contribution per N-tile; the deterministic fix sums
    the per-tile contributions in a fixed order.  Mathematically dprob is the
    plain gradient of the loss with respect to each routing probability, and
    that plain value is what this module computes.
  * Nemotron 3 Ultra interview notes, "concepts" list (LatentMoE): experts
    work in a 2048-wide latent, 512 experts per layer, 22 selected.
The pages do not state the router's tie-break, where the probability is
applied, the expert activation or width; the readings used are:
  * experts ordered by descending fp32 logit, ties to the lower expert index,
    -0.0 equal to +0.0;
  * softmax over the k selected logits;
  * expert MLP y = relu(x W1)^2 W2, no bias, W1 [D,F], W2 [F,D];
  * the probability weights the expert output in the combine:
    y_t = sum_j p_tj * o_(t,j), so dprob_tj = <dy_t, o_(t,j)>.
"""
import numpy as np


# ---------------------------------------------------------------- decoding
def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage values -> float64, exactly.  ``dtype``: "f32" (float32 array)
    or "bf16" (uint16 bit patterns of bfloat16)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------- routing
def route(logits: np.ndarray, top_k: int):
    """Top-k expert selection and softmax over the selected logits.

    ``logits``: float32 [T, E].  Returns ``topk_idx`` int32 [T, k] (slot j is
    the j-th largest logit; equal values go to the lower expert index) and
    ``topk_prob`` float64 [T, k].
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not (1 <= top_k <= E):
        raise ValueError("top_k out of range")
    neg = -logits.astype(np.float64)           # exact; -(+0.0) == -(-0.0) as values
    eidx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((eidx, neg), axis=-1)   # primary key: -logit, secondary: expert index
    topk_idx = order[:, :top_k].astype(np.int32)
    sel = np.take_along_axis(logits, topk_idx, axis=1).astype(np.float64)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    topk_prob = z / z.sum(axis=1, keepdims=True)
    return topk_idx, topk_prob


def permute(topk_idx: np.ndarray, expert_begin: int, num_local: int) -> dict:
    """Stable grouping of the (token, slot) pairs by local expert.

    Flat slot index i = t*k + j.  Rows are the local pairs sorted by
    (expert, i).  Returns counts[El], offsets[El+1], row_src[R] (row -> i),
    slot_row[T*k] (i -> row, -1 when the expert is not local) and
    row_tok[R] (row -> token).
    """
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1).astype(np.int64)
    local = (flat >= expert_begin) & (flat < expert_begin + num_local)
    i_local = np.nonzero(local)[0]
    e_local = flat[i_local] - expert_begin
    order = np.argsort(e_local, kind="stable")
    row_src = i_local[order]
    counts = np.bincount(e_local, minlength=num_local)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    slot_row = np.full(T * k, -1, dtype=np.int64)
    slot_row[row_src] = np.arange(len(row_src))
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                row_src=row_src.astype(np.int32), slot_row=slot_row.astype(np.int32),
                row_tok=(row_src // k).astype(np.int32))


# -------------------------------------------------------------- expert MLP
def _act(h):
    return np.maximum(h, 0.0) ** 2


def _act_grad(h):
    return 2.0 * np.maximum(h, 0.0)


def expert_forward(xr, w1e, w2e):
    """Rows of one expert: h = x W1, o = relu(h)^2 W2.  All float64."""
    h = xr @ w1e
    return h, _act(h) @ w2e


def expert_backward(xr, dyr, pr, hr, w1e, w2e) -> dict:
    """Backward of one expert's rows given the saved pre-activation ``hr``.

    xr [n,D], dyr [n,D] (upstream gradient of the token each row came from),
    pr [n] (routing probability of each row), hr [n,F].
    With L = sum_t <dy_t, y_t> and y_t = sum_j p_tj o_(t,j):
      dprob_r = <dy_r, o_r>
      dh_r    = p_r * (dy_r W2^T) * 2 relu(h_r)
      dx_r    = dh_r W1^T
      dW1     = x^T dh
      dW2     = relu(h)^2^T (p * dy)
    and act_p = p * relu(h)^2, the activation weighted by the probability
    (dW2 = act_p^T dy).
    """
    a = _act(hr)
    o = a @ w2e
    dprob = np.sum(dyr * o, axis=1)
    g = dyr @ w2e.T
    dh = pr[:, None] * g * _act_grad(hr)
    return dict(dprob=dprob, dh=dh, dx_rows=dh @ w1e.T, act_p=pr[:, None] * a,
                dw1=xr.T @ dh, dw2=a.T @ (pr[:, None] * dyr))


# ------------------------------------------------------------ whole layer
def combine_rows(rows: np.ndarray, slot_row: np.ndarray, weights: np.ndarray, T: int, k: int):
    """Token layout from row layout: out_t = sum over slots j (ascending) of
    weights[t,j] * rows[slot_row[t*k+j]], skipping non-local slots."""
    out = np.zeros((T, rows.shape[1]), dtype=np.float64)
    sr = slot_row.reshape(T, k)
    for j in range(k):
        r = sr[:, j]
        ok = r >= 0
        out[ok] += weights[ok, j][:, None] * rows[r[ok]]
    return out


def forward(x, w1, w2, topk_prob, perm, top_k, combine=True) -> dict:
    """Layer forward over the local experts.  x [T,D], w1 [El,D,F],
    w2 [El,F,D] float64.  Returns h [R,F], o_rows [R,D] and, with
    ``combine``, y [T,D]."""
    T = x.shape[0]
    off, row_tok = perm["offsets"], perm["row_tok"]
    R = int(off[-1])
    h = np.zeros((R, w1.shape[2]))
    o = np.zeros((R, w1.shape[1]))
    for e in range(w1.shape[0]):
        s, t = int(off[e]), int(off[e + 1])
        if t > s:
            h[s:t], o[s:t] = expert_forward(x[row_tok[s:t]], w1[e], w2[e])
    out = dict(h=h, o_rows=o)
    if combine:
        out["y"] = combine_rows(o, perm["slot_row"], topk_prob, T, top_k)
    return out


def backward(x, w1, w2, h, dy, topk_prob, perm, top_k, combine=True) -> dict:
    """Layer backward over the local experts, given the saved h [R,F].

    Returns dprob [T,k] (0 for non-local slots), dh [R,F], act_p [R,F], dx_rows [R,D],
    dW1 [El,D,F], dW2 [El,F,D] (exact zeros for empty experts) and, with
    ``combine``, dx [T,D] = sum over slots of dx_rows."""
    T = x.shape[0]
    off, row_tok, row_src = perm["offsets"], perm["row_tok"], perm["row_src"]
    R = int(off[-1])
    El, D, F = w1.shape
    p_rows = topk_prob.reshape(-1)[row_src]
    dprob_rows = np.zeros(R)
    dh = np.zeros((R, F))
    act_p = np.zeros((R, F))
    dx_rows = np.zeros((R, D))
    dw1 = np.zeros((El, D, F))
    dw2 = np.zeros((El, F, D))
    for e in range(El):
        s, t = int(off[e]), int(off[e + 1])
        if t == s:
            continue
        rows = row_tok[s:t]
        g = expert_backward(x[rows], dy[rows], p_rows[s:t], h[s:t], w1[e], w2[e])
        dprob_rows[s:t], dh[s:t], dx_rows[s:t] = g["dprob"], g["dh"], g["dx_rows"]
        act_p[s:t] = g["act_p"]
        dw1[e], dw2[e] = g["dw1"], g["dw2"]
    dprob = np.zeros(T * top_k)
    dprob[row_src] = dprob_rows
    out = dict(dprob=dprob.reshape(T, top_k), dh=dh, act_p=act_p, dx_rows=dx_rows, dw1=dw1, dw2=dw2)
    if combine:
        out["dx"] = combine_rows(dx_rows, perm["slot_row"], np.ones((T, top_k)), T, top_k)
    return out


def layer_loss(x, w1, w2, topk_prob, perm, top_k, dy) -> float:
    """L = sum_t <dy_t, y_t> for the full-layer (token layout) forward."""
    y = forward(x, w1, w2, topk_prob, perm, top_k, combine=True)["y"]
    return float(np.sum(dy * y))
