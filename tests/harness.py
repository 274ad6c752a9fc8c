"""Helpers shared by the GPU tests: move seeded inputs to the device, run
the HIP path through the C ABI, run the CPU oracle on the same inputs, and
compare.  The oracle never sees a value produced by the HIP path."""
import numpy as np
import torch

import bitwise_deterministic_moe_amd as moe
import oracle
from compare import compare_full, tol_for  # noqa: F401  (tol_for re-exported for the tests)
from synth import make_inputs

DEV = "cuda"


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Seeded host array -> device tensor (bf16 given as uint16 bits)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 / int host array (exact widening)."""
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    if t.dtype in (torch.float32, torch.float64):
        return t.cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)


class DeviceInputs:
    def __init__(self, cfg, host: dict):
        self.cfg = cfg
        self.host = host
        self.logits = torch.from_numpy(host["logits"]).to(DEV)
        self.x = to_dev(host["x"], cfg.dtype)
        self.w1 = to_dev(host["w1"], cfg.dtype)
        self.w2 = to_dev(host["w2"], cfg.dtype)
        self.dy = to_dev(host["dy"], cfg.dtype)


def device_inputs(cfg) -> DeviceInputs:
    return DeviceInputs(cfg, make_inputs(cfg))


def run_layer(prob: moe.Problem, di: DeviceInputs, mode=moe.DETERMINISTIC, poison=None):
    """moe_fwd + moe_bwd_dgrad_dprob + moe_bwd_wgrad; returns a dict of device tensors.
    ``poison``: optional float fill value for every output and workspace."""
    def mk(shape, dt):
        t = torch.empty(shape, dtype=dt, device=DEV)
        if poison is not None:
            if dt in (torch.int32, torch.int64, torch.uint8):
                t.fill_(-123456 if dt != torch.uint8 else 171)
            else:
                t.fill_(poison)
        return t
    dt = moe.TORCH_DTYPE[prob.dtype]
    T, k, el, rc, D, F = prob.tokens, prob.top_k, prob.local, prob.rows_cap, prob.d_model, prob.d_ffn
    ws = [mk((max(n, 1),), torch.uint8) for n in moe.moe_workspace_size(prob, mode)]
    r = moe.Routing(mk((T, k), torch.int32), mk((T, k), torch.float32), mk((el,), torch.int32),
                    mk((el + 1,), torch.int32), mk((rc,), torch.int32), mk((rc,), torch.int32),
                    mk((rc,), torch.float32), mk((T * k,), torch.int32), mk((moe.moe_sched_elems(prob),), torch.int32))
    out_rows = T if prob.combine else rc
    routing, h, y = moe.moe_fwd(prob, di.logits, di.x, di.w1, di.w2, mode, routing=r,
                                h=mk((rc, F), dt), y=mk((out_rows, D), dt), ws=ws[0])
    dx, dprob, dh = moe.moe_bwd_dgrad_dprob(prob, routing, di.dy, di.w1, di.w2, h, mode,
                                            dx=mk((out_rows, D), dt), dprob=mk((T, k), torch.float32),
                                            dh=mk((rc, F), dt), ws=ws[1])
    dw1, dw2 = moe.moe_bwd_wgrad(prob, routing, di.x, di.dy, h, dh, mode, dw1=mk((el, D, F), torch.float32),
                                 dw2=mk((el, F, D), torch.float32), ws=ws[2])
    torch.cuda.synchronize()
    return dict(routing=routing, h=h, y=y, dx=dx, dprob=dprob, dh=dh, dw1=dw1, dw2=dw2)


def oracle_layer(cfg, host: dict) -> dict:
    """Full oracle forward + backward in float64 on the seeded inputs."""
    idx, prob = oracle.route(host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, cfg.num_local)
    x, w1, w2, dy = (oracle.decode(host[n], cfg.dtype) for n in ("x", "w1", "w2", "dy"))
    f = oracle.forward(x, w1, w2, prob, perm, cfg.top_k, combine=bool(cfg.combine))
    b = oracle.backward(x, w1, w2, f["h"], dy, prob, perm, cfg.top_k, combine=bool(cfg.combine))
    return dict(topk_idx=idx, topk_prob=prob, perm=perm, **f, **b)


def routing_host(r: moe.Routing, R: int) -> dict:
    return dict(topk_idx=to_host(r.topk_idx), topk_prob=to_host(r.topk_prob), counts=to_host(r.counts),
                offsets=to_host(r.offsets), row_src=to_host(r.row_src)[:R], row_tok=to_host(r.row_tok)[:R],
                row_prob=to_host(r.row_prob)[:R], slot_row=to_host(r.slot_row))


def compare_routing(gpu: moe.Routing, ref: dict):
    """Integer routing state exactly, probabilities to 1e-5."""
    R = int(ref["perm"]["offsets"][-1])
    g = routing_host(gpu, R)
    np.testing.assert_array_equal(g["topk_idx"], ref["topk_idx"])
    for n in ("counts", "offsets", "row_src", "row_tok", "slot_row"):
        np.testing.assert_array_equal(g[n], ref["perm"][n], err_msg=n)
    assert rel_l2(g["topk_prob"], ref["topk_prob"]) <= 1e-5
    assert rel_l2(g["row_prob"], ref["topk_prob"].reshape(-1)[ref["perm"]["row_src"]]) <= 1e-5
    return R


def compare_layer(cfg, out: dict, ref: dict, tol=None):
    """Element-by-element comparison of every output: integer routing state
    exactly; every float output by whole-tensor rel-L2, worst-row rel-L2 and
    (dprob) per-slot bounds (tests/compare.py); empty experts exact zero dW."""
    R = compare_routing(out["routing"], ref)
    got = {n: to_host(out[n]) for n in ("h", "dh", "y", "dx", "dprob", "dw1", "dw2")}
    errs = compare_full(cfg.dtype, got, ref, bool(cfg.combine), cfg.top_k)
    if tol is not None:
        bad = {k: v for k, v in errs.items() if not k.endswith(("worst_row", "worst_z")) and not v <= tol}
        assert not bad, f"rel-L2 above {tol}: {bad}"
    empty = np.nonzero(ref["perm"]["counts"] == 0)[0]
    if len(empty):
        assert torch.all(out["dw1"][torch.as_tensor(empty, device=DEV)] == 0)
        assert torch.all(out["dw2"][torch.as_tensor(empty, device=DEV)] == 0)
    assert R == ref["perm"]["offsets"][-1]
    return errs


FP_OUTPUTS = ("h", "y", "dx", "dprob", "dh", "dw1", "dw2")
FP_ROUTING = ("topk_idx", "topk_prob", "counts", "offsets", "row_src", "row_tok", "row_prob", "slot_row")


def fingerprints(out: dict, combine: int) -> dict:
    """Fingerprint totals of every output and routing array (device hash).
    Row-layout tensors are hashed over their R written rows only."""
    r = out["routing"]
    R = r.rows
    rowwise = {"h", "dh"} | (set() if combine else {"y", "dx"})
    fp = {}
    for n in FP_OUTPUTS:
        t = out[n][:R] if n in rowwise else out[n]
        fp[n] = moe.moe_fingerprint(t.contiguous())[1]
    for n in FP_ROUTING:
        t = getattr(r, n)
        if n in ("row_src", "row_tok", "row_prob"):
            t = t[:R]
        fp[n] = moe.moe_fingerprint(t.contiguous(), chunk_elems=4096)[1]
    return fp


def compare_layer_unordered(cfg, out: dict, ref: dict, tol=None):
    """Comparison for runs whose row order inside an expert is not fixed
    (atomic-mode permutation): rows are matched through their flat slot."""
    tol = tol or tol_for(cfg.dtype)
    r = out["routing"]
    np.testing.assert_array_equal(to_host(r.topk_idx), ref["topk_idx"])
    np.testing.assert_array_equal(to_host(r.counts), ref["perm"]["counts"])
    np.testing.assert_array_equal(to_host(r.offsets), ref["perm"]["offsets"])
    R = int(ref["perm"]["offsets"][-1])
    src = to_host(r.row_src)[:R]
    np.testing.assert_array_equal(np.sort(src), np.sort(ref["perm"]["row_src"]))
    ref_row = ref["perm"]["slot_row"][src]           # oracle row of each GPU row
    np.testing.assert_array_equal(to_host(r.slot_row)[src], np.arange(R))
    errs = dict(h=rel_l2(to_host(out["h"])[:R], ref["h"][ref_row]),
                dh=rel_l2(to_host(out["dh"])[:R], ref["dh"][ref_row]),
                dprob=rel_l2(to_host(out["dprob"]), ref["dprob"]),
                dw1=rel_l2(to_host(out["dw1"]), ref["dw1"]), dw2=rel_l2(to_host(out["dw2"]), ref["dw2"]))
    if cfg.combine:
        errs["y"] = rel_l2(to_host(out["y"]), ref["y"])
        errs["dx"] = rel_l2(to_host(out["dx"]), ref["dx"])
    else:
        errs["y"] = rel_l2(to_host(out["y"])[:R], ref["o_rows"][ref_row])
        errs["dx"] = rel_l2(to_host(out["dx"])[:R], ref["dx_rows"][ref_row])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"rel-L2 above {tol}: {bad} (all: {errs})"
    return errs


class LayerRunner:
    """Runs the layer (moe_fwd, moe_bwd_dgrad_dprob, moe_bwd_wgrad) again and
    again into the same output and workspace buffers, so that repeated runs at
    full size do not allocate."""

    def __init__(self, prob: moe.Problem, di: DeviceInputs, mode=moe.DETERMINISTIC):
        self.prob, self.di, self.mode = prob, di, mode
        dt = moe.TORCH_DTYPE[prob.dtype]
        T, k, el, rc, D, F = prob.tokens, prob.top_k, prob.local, prob.rows_cap, prob.d_model, prob.d_ffn
        out_rows = T if prob.combine else rc
        self.ws = [torch.empty(max(n, 1), dtype=torch.uint8, device=DEV) for n in moe.moe_workspace_size(prob, mode)]
        self.routing = moe.Routing.empty(prob, DEV)
        self.h = torch.empty((rc, F), dtype=dt, device=DEV)
        self.y = torch.empty((out_rows, D), dtype=dt, device=DEV)
        self.dx = torch.empty((out_rows, D), dtype=dt, device=DEV)
        self.dprob = torch.empty((T, k), dtype=torch.float32, device=DEV)
        self.dh = torch.empty((rc, F), dtype=dt, device=DEV)
        self.dw1 = torch.empty((el, D, F), dtype=torch.float32, device=DEV)
        self.dw2 = torch.empty((el, F, D), dtype=torch.float32, device=DEV)

    def run(self, seed: int = 0) -> dict:
        prob, di, mode = self.prob.with_seed(seed), self.di, self.mode
        moe.moe_fwd(prob, di.logits, di.x, di.w1, di.w2, mode, routing=self.routing, h=self.h, y=self.y,
                    ws=self.ws[0])
        moe.moe_bwd_dgrad_dprob(prob, self.routing, di.dy, di.w1, di.w2, self.h, mode, dx=self.dx, dprob=self.dprob,
                                dh=self.dh, ws=self.ws[1])
        moe.moe_bwd_wgrad(prob, self.routing, di.x, di.dy, self.h, self.dh, mode, dw1=self.dw1, dw2=self.dw2,
                          ws=self.ws[2])
        torch.cuda.synchronize()
        return dict(routing=self.routing, h=self.h, y=self.y, dx=self.dx, dprob=self.dprob, dh=self.dh,
                    dw1=self.dw1, dw2=self.dw2)


REPEATS = 20
SHUFFLE_SEEDS = (1, 0x5EED, 0xDEADBEEF, 0x9E3779B97F4A7C15)


def determinism_runs(runner: LayerRunner, combine: int, repeats: int = REPEATS, seeds=SHUFFLE_SEEDS,
                     per_seed: int = 2, label: str = "") -> int:
    """Fingerprints of every output and routing array: ``repeats`` runs with
    the natural launch order, then ``per_seed`` runs under each shuffled
    workgroup order (with seeded delays), all against the first run.
    Returns the number of runs compared."""
    ref = fingerprints(runner.run(0), combine)
    n = 0
    plan = [0] * repeats + [s for s in seeds for _ in range(per_seed)]
    for i, seed in enumerate(plan):
        fp = fingerprints(runner.run(seed), combine)
        diff = [k for k in ref if fp[k] != ref[k]]
        assert not diff, f"{label} run {i} (shuffle seed {seed:#x}): outputs differ from the first run: {diff}"
        n += 1
    return n
