"""Progressive fingerprint tracing of a deterministic train step of the MoE
layer, bit-exact checkpoint resume, and the first-divergence localiser.

What the pages describe (French article, section "Méthodologie de débogage du
non-déterminisme"; English digest, section "Interpretation"):
  * two guarantees: runs started from the same state stay bit-identical at
    every step, and a run resumed from a checkpoint is identical to the
    continuous run;
  * ordered tensor fingerprints, computed on the GPU with shape, dtype and
    element count recorded, chunk-wise for order-sensitive data (routing
    maps);
  * progressive narrowing: first the step where an end-to-end metric
    diverges; then broad tracing to find the earliest divergent step and
    phase (the first divergent bit can precede the visible loss gap); then
    op-level tracing on that step only;
  * a full-precision source of truth, with the runtime representation
    rebuilt through the training's own conversion path.

One train step on the layer (all device work through the library's C ABI):
    logits = moe_router_fwd(x, wr)              router (linear, no bias)
    routing, h, y = moe_fwd(logits, x, W1, W2)
    loss = sum_t <dy_t, y_t>                    (dy: the step's batch)
    dx, dprob, dh = moe_bwd_dgrad_dprob(dy)
    dW1, dW2 = moe_bwd_wgrad(x, dy, h, dh)
    dlogits, dwr, dx_router = moe_router_bwd(dprob)
    SGD on the float32 masters of W1, W2, wr; bf16 (or f32) runtime copies
    rebuilt by the same kernel (moe_sgd_step).
With mx=True (bf16 layers) every expert GEMM runs on MXFP8 operands: the
routing stage alone (moe_route), then moe_mx_fwd_fc1 / moe_mx_fwd_fc2 on x,
act and the transposed weights (moe_mx_quantize, moe_mx_quantize_t), the
data gradients moe_mx_dgrad_fc2 / moe_mx_dgrad_fc1 on dy, dh and the
weights, and the weight gradients moe_mx_wgrad on x, dh, p relu(h)^2 and dy
quantised along the routed rows (moe_mx_quantize_wgrad).  The op-level
trace fingerprints every encoded tensor and its scale buffer, as the pages
do for low-precision runs; it also records dh's NVFP4 encoding (codes,
block scales, tensor scale).
Metrics (loss, gradient norms) are summed on the host in float64 in a fixed
order, so they are deterministic too.
"""
import json
import math
from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np
import torch

from . import (MXW_ACT_P, MXW_ROW, MXW_TOKEN, MoeError, Problem, TORCH_DTYPE, moe_bwd_dgrad_dprob,
               moe_bwd_wgrad, moe_fingerprint, moe_fwd, moe_mx_dgrad_fc1, moe_mx_dgrad_fc2, moe_mx_fwd_fc1,
               moe_mx_fwd_fc2, moe_mx_quantize, moe_mx_quantize_t, moe_mx_quantize_wgrad, moe_mx_wgrad,
               moe_nvfp4_quantize, moe_route, moe_router_bwd, moe_router_fwd, moe_sgd_step)

LEVELS = {"metrics": 0, "phases": 1, "ops": 2}


@dataclass
class Record:
    step: int
    phase: str      # "metrics", "forward", "backward", "router", "optimizer"
    op: str         # the call that produced the tensor
    name: str
    dtype: str
    shape: list
    numel: int
    fp: str         # 64-bit fingerprint (hex), or the float64 bits of a metric

    def key(self):
        return (self.step, self.phase, self.op, self.name, self.dtype, tuple(self.shape), self.numel)


_DT = {torch.float32: "f32", torch.bfloat16: "bf16", torch.int32: "i32", torch.uint8: "u8", torch.int64: "i64",
       torch.float64: "f64"}


class Tracer:
    """Ordered log of fingerprints.  ``level``: "metrics" (loss and gradient
    norms per step), "phases" (also every call's outputs at phase level: the
    tensors that leave forward, backward, router and optimizer) or "ops"
    (also the intermediate tensors of each call: routing maps, h, dh,
    dlogits ...).  ``window``: steps traced above metric level (None = all)."""

    def __init__(self, level: str = "phases", window: Optional[range] = None):
        if level not in LEVELS:
            raise ValueError(level)
        self.level = LEVELS[level]
        self.window = window
        self.records: List[Record] = []

    def _on(self, step, level):
        if level > self.level:
            return False
        return level == 0 or self.window is None or step in self.window

    def metric(self, step: int, name: str, value: float):
        bits = np.array([value], dtype=np.float64).view(np.uint64)[0]
        self.records.append(Record(step, "metrics", "host", name, "f64", [], 1, f"{int(bits):016x}"))

    def tensor(self, step: int, phase: str, op: str, name: str, t: torch.Tensor, level: int):
        if not self._on(step, level):
            return
        fp = moe_fingerprint(t.contiguous())[1]
        self.records.append(Record(step, phase, op, name, _DT[t.dtype], list(t.shape), t.numel(), f"{fp:016x}"))

    def save(self, path: str):
        with open(path, "w") as f:
            for r in self.records:
                f.write(json.dumps(r.__dict__) + "\n")

    @staticmethod
    def load(path: str) -> List[Record]:
        with open(path) as f:
            return [Record(**json.loads(line)) for line in f if line.strip()]


def first_divergence(a: List[Record], b: List[Record]):
    """First position where the two ordered logs differ: returns (index, ra,
    rb) with ra / rb None where one log has ended, or None if they are equal."""
    for i in range(max(len(a), len(b))):
        ra = a[i] if i < len(a) else None
        rb = b[i] if i < len(b) else None
        if ra is None or rb is None or ra.key() != rb.key() or ra.fp != rb.fp:
            return i, ra, rb
    return None


@dataclass
class TrainState:
    """Float32 masters (the source of truth) and the runtime copies the
    layer computes with."""
    prob: Problem
    lr: float
    step: int
    master: dict                  # name -> float32 device tensor
    runtime: dict = field(default_factory=dict)

    def rebuild_runtime(self):
        """Runtime copies from the masters through the SGD kernel's
        conversion (a step with a zero gradient leaves the master unchanged)."""
        dt = TORCH_DTYPE[self.prob.dtype]
        for n, m in self.master.items():
            rt = torch.empty(m.shape, dtype=dt, device=m.device)
            moe_sgd_step(m, torch.zeros_like(m), 0.0, rt)
            self.runtime[n] = rt

    def save(self, path: str):
        """Checkpoint: the float32 masters and the step (npz, no pickles)."""
        arrays = {n: m.cpu().numpy() for n, m in self.master.items()}
        np.savez(path, step=np.int64(self.step), lr=np.float64(self.lr), **arrays)

    @staticmethod
    def load(path: str, prob: Problem) -> "TrainState":
        with np.load(path, allow_pickle=False) as z:
            master = {n: torch.from_numpy(z[n].copy()).cuda() for n in ("w1", "w2", "wr")}
            st = TrainState(prob, float(z["lr"]), int(z["step"]), master)
        st.rebuild_runtime()
        return st


def initial_state(cfg, lr: float = 0.05) -> TrainState:
    """Masters from the seeded weights (exact widening of the storage values)."""
    from synth import make_inputs, make_router_inputs
    from synth.inputs import bf16_bits_to_f32
    host = make_inputs(cfg, parts=("w1", "w2"))
    host["wr"] = make_router_inputs(cfg)["wr"]
    widen = (lambda a: bf16_bits_to_f32(a)) if cfg.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    master = {n: torch.from_numpy(np.ascontiguousarray(widen(host[n]))).cuda() for n in ("w1", "w2", "wr")}
    st = TrainState(Problem.from_config(cfg), lr, 0, master)
    st.rebuild_runtime()
    return st


def _device_batch(cfg, step: int):
    from synth import make_batch
    b = make_batch(cfg, step)
    if cfg.dtype == "bf16":
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)  # noqa
    else:
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()  # noqa
    return up(b["x"]), up(b["dy"])


def _host_sum_sq(t: torch.Tensor) -> float:
    a = t.double().cpu().numpy().ravel()
    return float(math.fsum((a * a).tolist())) if a.size < 1 << 20 else float(np.sum(a * a))


def _mx(t, rows: int, cols: int):
    """MXFP8 codes and scales of t viewed as [rows, cols]."""
    return moe_mx_quantize(t.reshape(rows, cols))


def train_step(cfg, st: TrainState, tracer: Tracer, hook: Optional[Callable] = None, mx: bool = False):
    """One step at st.step; advances st.step.  ``hook(step, where, st)`` may
    change the state at "before_forward" (a fault injector for tests).  With
    ``mx`` every expert GEMM runs on MXFP8 operands."""
    if cfg.combine != 1 or cfg.num_local != cfg.num_experts:
        raise MoeError("the train step covers the full layer (token layout, all experts local)")
    if mx and (cfg.dtype != "bf16" or cfg.d_model > 2048 or cfg.d_ffn > 2048):
        raise MoeError("the MXFP8 train step needs a bf16 layer with d_model and d_ffn at most 2048")
    s, prob = st.step, st.prob
    x, dy = _device_batch(cfg, s)
    if hook:
        hook(s, "before_forward", st)
    R = st.runtime
    logits = moe_router_fwd(prob, x, R["wr"])
    enc, fwd_enc, wg_enc = {}, {}, {}
    if mx:
        el, D, F = cfg.num_local, cfg.d_model, cfg.d_ffn
        routing = moe_route(prob, logits)
        fwd_enc["x"], fwd_enc["w1t"] = moe_mx_quantize(x), moe_mx_quantize_t(R["w1"].reshape(el, D, F))
        h, act = moe_mx_fwd_fc1(prob, routing, fwd_enc["x"], fwd_enc["w1t"])
        fwd_enc["act"], fwd_enc["w2t"] = moe_mx_quantize(act), moe_mx_quantize_t(R["w2"].reshape(el, F, D))
        y = moe_mx_fwd_fc2(prob, routing, fwd_enc["act"], fwd_enc["w2t"])
    else:
        routing, h, y = moe_fwd(prob, logits, x, R["w1"], R["w2"])
    if mx:
        el, D, F = cfg.num_local, cfg.d_model, cfg.d_ffn
        enc["dy"], enc["w2"] = _mx(dy, cfg.tokens, D), _mx(R["w2"], el * F, D)
        w2mx = (enc["w2"][0].reshape(el, F, D), enc["w2"][1].reshape(el, F, D // 32))
        dprob, dh = moe_mx_dgrad_fc2(prob, routing, enc["dy"], w2mx, h)
        enc["dh"], enc["w1"] = _mx(dh, prob.rows_cap, F), _mx(R["w1"], el * D, F)
        w1mx = (enc["w1"][0].reshape(el, D, F), enc["w1"][1].reshape(el, D, F // 32))
        dx = moe_mx_dgrad_fc1(prob, routing, enc["dh"], w1mx)     # per routed row
        for n, src, kind in (("x", x, MXW_TOKEN), ("dh", dh, MXW_ROW), ("act", h, MXW_ACT_P), ("dy", dy, MXW_TOKEN)):
            wg_enc[n] = moe_mx_quantize_wgrad(prob, routing, src, kind)
        dw1, dw2 = moe_mx_wgrad(prob, routing, wg_enc["x"], wg_enc["dh"], wg_enc["act"], wg_enc["dy"])
    else:
        dx, dprob, dh = moe_bwd_dgrad_dprob(prob, routing, dy, R["w1"], R["w2"], h)
        dw1, dw2 = moe_bwd_wgrad(prob, routing, x, dy, h, dh)
    dlogits, dwr, dxr = moe_router_bwd(prob, routing, dprob, x, R["wr"])
    torch.cuda.synchronize()

    T = tracer
    # forward
    T.tensor(s, "forward", "moe_router_fwd", "logits", logits, 1)
    for n in ("topk_idx", "topk_prob", "counts", "offsets", "row_src", "slot_row"):
        T.tensor(s, "forward", "moe_fwd", n, getattr(routing, n), 2)
    if mx:
        for n, op in (("x", "moe_mx_quantize"), ("w1t", "moe_mx_quantize_t")):
            T.tensor(s, "forward", op, f"{n}_codes", fwd_enc[n][0], 2)
            T.tensor(s, "forward", op, f"{n}_scales", fwd_enc[n][1], 2)
        T.tensor(s, "forward", "moe_mx_fwd_fc1", "h", h, 2)
        for n, op in (("act", "moe_mx_quantize"), ("w2t", "moe_mx_quantize_t")):
            T.tensor(s, "forward", op, f"{n}_codes", fwd_enc[n][0], 2)
            T.tensor(s, "forward", op, f"{n}_scales", fwd_enc[n][1], 2)
        T.tensor(s, "forward", "moe_mx_fwd_fc2", "y", y, 1)
    else:
        T.tensor(s, "forward", "moe_fwd", "h", h, 2)
        T.tensor(s, "forward", "moe_fwd", "y", y, 1)
    # backward
    if mx:
        for n in ("dy", "w2"):
            T.tensor(s, "backward", "moe_mx_quantize", f"{n}_codes", enc[n][0], 2)
            T.tensor(s, "backward", "moe_mx_quantize", f"{n}_scales", enc[n][1], 2)
        T.tensor(s, "backward", "moe_mx_dgrad_fc2", "dprob", dprob, 1)
        T.tensor(s, "backward", "moe_mx_dgrad_fc2", "dh", dh, 2)
        for n in ("dh", "w1"):
            T.tensor(s, "backward", "moe_mx_quantize", f"{n}_codes", enc[n][0], 2)
            T.tensor(s, "backward", "moe_mx_quantize", f"{n}_scales", enc[n][1], 2)
        T.tensor(s, "backward", "moe_mx_dgrad_fc1", "dx_rows", dx[: routing.rows], 1)
        nv = moe_nvfp4_quantize(dh)
        for n, t in zip(("dh_codes", "dh_scales", "dh_tensor_scale"), nv):
            T.tensor(s, "backward", "moe_nvfp4_quantize", n, t, 2)
        # the written part of the weight-gradient encodings: each expert's
        # rows padded to 64
        P = int(((routing.counts.long() + 63) // 64 * 64).sum().item())
        for n in ("x", "dh", "act", "dy"):
            codes, scales = wg_enc[n]
            T.tensor(s, "backward", "moe_mx_quantize_wgrad", f"{n}_codes", codes[: P // 64].contiguous(), 2)
            T.tensor(s, "backward", "moe_mx_quantize_wgrad", f"{n}_scales", scales[: P // 64].contiguous(), 2)
        T.tensor(s, "backward", "moe_mx_wgrad", "dw1", dw1, 1)
        T.tensor(s, "backward", "moe_mx_wgrad", "dw2", dw2, 1)
    else:
        T.tensor(s, "backward", "moe_bwd_dgrad_dprob", "dprob", dprob, 1)
        T.tensor(s, "backward", "moe_bwd_dgrad_dprob", "dh", dh, 2)
        T.tensor(s, "backward", "moe_bwd_dgrad_dprob", "dx", dx, 1)
        T.tensor(s, "backward", "moe_bwd_wgrad", "dw1", dw1, 1)
        T.tensor(s, "backward", "moe_bwd_wgrad", "dw2", dw2, 1)
    T.tensor(s, "router", "moe_router_bwd", "dlogits", dlogits, 2)
    T.tensor(s, "router", "moe_router_bwd", "dwr", dwr, 1)
    T.tensor(s, "router", "moe_router_bwd", "dx_router", dxr, 1)
    # end-to-end metrics of the step (host float64 in a fixed order)
    yd = (y.double() * dy.double()).cpu().numpy().ravel()
    T.metric(s, "loss", float(math.fsum(yd.tolist())) if yd.size < 1 << 21 else float(np.sum(yd)))
    T.metric(s, "grad_norm", math.sqrt(_host_sum_sq(dw1) + _host_sum_sq(dw2) + _host_sum_sq(dwr)))
    # optimizer: SGD on the masters, runtime copies rebuilt by the same kernel
    for n, g in (("w1", dw1), ("w2", dw2), ("wr", dwr)):
        moe_sgd_step(st.master[n], g.reshape(st.master[n].shape), st.lr, R[n])
    torch.cuda.synchronize()
    for n in ("w1", "w2", "wr"):
        T.tensor(s, "optimizer", "moe_sgd_step", f"master_{n}", st.master[n], 1)
        T.tensor(s, "optimizer", "moe_sgd_step", f"runtime_{n}", R[n], 2)
    st.step += 1


def run(cfg, steps: int, level: str = "phases", window: Optional[range] = None, st: Optional[TrainState] = None,
        hook: Optional[Callable] = None, lr: float = 0.05, mx: bool = False):
    """Train from st (or the initial state) until st.step == steps."""
    st = st or initial_state(cfg, lr)
    tr = Tracer(level, window)
    while st.step < steps:
        train_step(cfg, st, tr, hook, mx)
    return st, tr


def localise(cfg, steps: int, hook_a: Optional[Callable] = None, hook_b: Optional[Callable] = None) -> dict:
    """Progressive search for the first divergence between two runs (e.g. a
    reference and a run with a changed component):
      1. metrics over all steps: the first step whose loss or gradient norm
         differs (the visible symptom), if any;
      2. phase-level fingerprints over all steps up to it (all steps if the
         metrics agree): the earliest step and phase with a differing tensor
         (it can precede step 1's);
      3. op-level fingerprints on that step only: the first differing tensor.
    Returns the three findings (None where the runs agree)."""
    out = {"metric": None, "phase": None, "op": None}
    _, ta = run(cfg, steps, "metrics", hook=hook_a)
    _, tb = run(cfg, steps, "metrics", hook=hook_b)
    d = first_divergence(ta.records, tb.records)
    last = steps
    if d is not None:
        out["metric"] = (d[1] or d[2]).__dict__
        last = (d[1] or d[2]).step + 1
    # broad tracing up to the visible divergence (over every step when the
    # metrics agree: a divergent bit need not reach them)
    _, ta = run(cfg, last, "phases", hook=hook_a)
    _, tb = run(cfg, last, "phases", hook=hook_b)
    d = first_divergence([r for r in ta.records if r.phase != "metrics"],
                         [r for r in tb.records if r.phase != "metrics"])
    if d is None:
        return out
    out["phase"] = (d[1] or d[2]).__dict__
    s0 = (d[1] or d[2]).step
    _, ta = run(cfg, s0 + 1, "ops", window=range(s0, s0 + 1), hook=hook_a)
    _, tb = run(cfg, s0 + 1, "ops", window=range(s0, s0 + 1), hook=hook_b)
    d = first_divergence([r for r in ta.records if r.phase != "metrics" and r.step == s0],
                         [r for r in tb.records if r.phase != "metrics" and r.step == s0])
    out["op"] = (d[1] or d[2]).__dict__ if d else None
    return out


def main(argv=None):
    import argparse
    ap = argparse.ArgumentParser(description="Fingerprint-traced deterministic train steps of the MoE layer")
    ap.add_argument("--config", default="tiny_fp32")
    ap.add_argument("--steps", type=int, default=4)
    ap.add_argument("--level", default="phases", choices=list(LEVELS))
    ap.add_argument("--out", help="write the trace (JSON lines)")
    ap.add_argument("--compare", nargs=2, metavar=("A", "B"), help="report the first divergence of two traces")
    ap.add_argument("--mx", action="store_true", help="every expert GEMM on MXFP8 operands (bf16 layers)")
    a = ap.parse_args(argv)
    if a.compare:
        d = first_divergence(Tracer.load(a.compare[0]), Tracer.load(a.compare[1]))
        print(json.dumps(None if d is None else {"index": d[0], "a": d[1] and d[1].__dict__,
                                                 "b": d[2] and d[2].__dict__}))
        return
    from synth import CONFIGS
    _, tr = run(CONFIGS[a.config], a.steps, a.level, mx=a.mx)
    if a.out:
        tr.save(a.out)
    print(json.dumps({"records": len(tr.records), "steps": a.steps, "level": a.level}))


if __name__ == "__main__":
    main()
