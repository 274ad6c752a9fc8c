"""Seeded synthetic inputs for the MoE expert layer.

Recipe (the same for every consumer):
  * numpy ``default_rng`` (PCG64) with one independent stream per tensor
    (and per expert for the weights), keyed ``[seed, tensor_code, expert]``,
    so any expert's weights can be drawn alone;
  * ``standard_normal(float32)`` times the tensor's standard deviation, in
    float32: logits N(0,1), x N(0, x_std), W1/W2 N(0, w_std), dy N(0,1);
  * for bf16 workloads the float32 value is rounded to bf16 (round to
    nearest, ties to even) and kept as raw uint16 bit patterns;
  * the skewed workload adds a per-expert Zipf(s=1.1) log-rank offset to the
    float32 logits (see ``zipf_bias``).

Nothing here implements the method (routing, expert MLP, combine, hashing).
"""
import json
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Config

_TENSOR_CODE = {"logits": 0, "x": 1, "w1": 2, "w2": 3, "dy": 4, "zipf_rank": 5, "wr": 6, "dprob": 7}
_HERE = os.path.dirname(os.path.abspath(__file__))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction (no NaN handling)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tensor: str, expert: int = -1) -> np.random.Generator:
    key = [seed, _TENSOR_CODE[tensor]] + ([expert] if expert >= 0 else [])
    return np.random.default_rng(key)


def _draw(rng, shape, std, dtype):
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def zipf_beta(cfg: Config) -> float:
    """Calibrated strength of the Zipf offset for ``cfg`` (stored by calibrate_zipf.py)."""
    with open(os.path.join(_HERE, "zipf_beta.json")) as f:
        table = json.load(f)
    key = f"{cfg.tokens}x{cfg.num_experts}k{cfg.top_k}s{cfg.seed}"
    return float(table[key]["beta"])


def zipf_bias(cfg: Config, beta: float) -> np.ndarray:
    """Per-expert logit offset b_e = -beta * 1.1 * ln(rank_e), rank a seeded
    permutation of 1..E; the ``cfg.zipf_empty`` lowest-ranked experts get -30
    so that they receive no tokens.  Computed in float64, returned as float32."""
    E = cfg.num_experts
    rank = _rng(cfg.seed, "zipf_rank").permutation(E).astype(np.float64) + 1.0
    b = -beta * 1.1 * np.log(rank)
    b[rank > E - cfg.zipf_empty] = -30.0
    return b.astype(np.float32)


def make_logits(cfg: Config, beta: float = None) -> np.ndarray:
    logits = _rng(cfg.seed, "logits").standard_normal((cfg.tokens, cfg.num_experts), dtype=np.float32)
    if cfg.skew == "zipf":
        if beta is None:
            beta = cfg.zipf_beta if cfg.zipf_beta is not None else zipf_beta(cfg)
        logits += zipf_bias(cfg, beta)[None, :]
    return logits


def make_expert_weights(cfg: Config, which: str, experts) -> np.ndarray:
    """Weights of the given global expert indices: w1 [n, D, F] or w2 [n, F, D].

    Same values as ``_draw`` on each expert's own stream; the draw and the
    rounding run in per-thread scratch buffers so that large expert counts
    do not spend their time allocating."""
    D, F = cfg.d_model, cfg.d_ffn
    shape = (D, F) if which == "w1" else (F, D)
    experts = list(experts)
    out = np.empty((len(experts),) + shape, dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)
    local = threading.local()

    def one(i):
        if not hasattr(local, "f"):
            local.f = np.empty(shape, dtype=np.float32)
            local.u = np.empty(shape, dtype=np.uint32)
        f, u = local.f, local.u
        _rng(cfg.seed, which, experts[i]).standard_normal(dtype=np.float32, out=f)
        if cfg.w_std != 1.0:
            f *= np.float32(cfg.w_std)
        if cfg.dtype != "bf16":
            out[i] = f
            return
        # round to nearest even, as f32_to_bf16_bits
        b = f.view(np.uint32)
        np.right_shift(b, np.uint32(16), out=u)
        u &= np.uint32(1)
        u += np.uint32(0x7FFF)
        u += b
        u >>= np.uint32(16)
        out[i] = u

    if len(experts) > 4:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(one, range(len(experts))))
    else:
        for i in range(len(experts)):
            one(i)
    return out


def make_inputs(cfg: Config, parts=("logits", "x", "w1", "w2", "dy"), experts=None) -> dict:
    """Draw the requested input tensors.

    ``experts`` selects which global experts' weights to draw (default: the
    local experts ``expert_begin .. expert_begin+num_local-1``)."""
    if experts is None:
        experts = range(cfg.expert_begin, cfg.expert_begin + cfg.num_local)
    out = {}
    if "logits" in parts:
        out["logits"] = make_logits(cfg)
    if "x" in parts:
        out["x"] = _draw(_rng(cfg.seed, "x"), (cfg.tokens, cfg.d_model), cfg.x_std, cfg.dtype)
    if "w1" in parts:
        out["w1"] = make_expert_weights(cfg, "w1", experts)
    if "w2" in parts:
        out["w2"] = make_expert_weights(cfg, "w2", experts)
    if "dy" in parts:
        out["dy"] = _draw(_rng(cfg.seed, "dy"), (cfg.tokens, cfg.d_model), 1.0, cfg.dtype)
    return out


def make_router_inputs(cfg: Config) -> dict:
    """Router weights wr [E, D] (storage dtype, N(0, w_std)) and an upstream
    gradient dprob [T, k] (float32, N(0, 1)) for exercising the router backward
    on its own.  Drawn from streams of their own, so the layer's other inputs
    are unchanged."""
    return {
        "wr": _draw(_rng(cfg.seed, "wr"), (cfg.num_experts, cfg.d_model), cfg.w_std, cfg.dtype),
        "dprob": _draw(_rng(cfg.seed, "dprob"), (cfg.tokens, cfg.top_k), 1.0, "f32"),
    }


def make_batch(cfg: Config, step: int) -> dict:
    """The batch of train step ``step``: x [T, D] (storage dtype, N(0, x_std))
    and the upstream gradient dy [T, D] (storage dtype, N(0, 1)) of the loss
    L = sum_t <dy_t, y_t>.  Streams keyed by the step, distinct from the
    layer's fixed x and dy."""
    key = 1_000_000 + int(step)
    return {
        "x": _draw(_rng(cfg.seed, "x", key), (cfg.tokens, cfg.d_model), cfg.x_std, cfg.dtype),
        "dy": _draw(_rng(cfg.seed, "dy", key), (cfg.tokens, cfg.d_model), 1.0, cfg.dtype),
    }
