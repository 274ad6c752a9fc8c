#!/usr/bin/env python3
"""Benchmark of the bitwise-deterministic MoE grouped-GEMM backward on one
MI355X.

A step is one backward of the expert layer: moe_bwd_dgrad_dprob followed by
moe_bwd_wgrad (fc2 dgrad with the dprob partial epilogue, the fixed-order
dprob combine, fc1 dgrad, the fixed-order dx combine, act_p rebuilt from h,
both weight gradients with their ordered split-K reduction).  The headline
workload is the largest single-GPU one, the LatentMoE-shaped layer: 4096
tokens, latent 2048, 512 experts top-22 (90,112 routed rows), expert MLP
2048 -> 2048 -> 2048 ReLU^2, bf16 storage, float32 accumulation and float32
dprob / dW.  The inputs are seeded synthetic tensors already resident in HBM;
routing and the saved h come from one untimed moe_fwd.

Prints one JSON line.  ``value`` is 8*R*D*F / (time of one deterministic
step), in TFLOP/s, from K steps back to back between synchronisations.  The
line also carries, per workload: cold-cache (512 MB written between steps)
and warm per-step medians, the determinism tax (deterministic and atomic
steps interleaved A B B A, medians and IQR, and the tax of the GEMM launches
alone), the forward time, per-kernel times, and each kernel's roofline
(algorithmic FLOPs and bytes against the bf16 MFMA and HBM peaks; the bound is
whichever takes longer).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config NAME] [--sub-configs A,B|none]
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6    # MI355X dense bf16 MFMA, vendor figure
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
HEADLINE = "latent_e512k22"
SUBS = "bf16_e8k2,skewed_e512k22,shard_e512k22_l4"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--sub-configs", default=SUBS, help="comma-separated workloads reported beside the headline, "
                                                         "or 'none'")
    ap.add_argument("--stage-reps", type=int, default=10)
    ap.add_argument("--flush-mb", type=int, default=512, help="bytes written between cold-cache steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the router / MXFP8 / NVFP4 legs")
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + timed steps of the headline workload only (for rocprofv3 runs)")
    ap.add_argument("--profile-mx-wgrad", action="store_true",
                    help="with --profile-only: time the MXFP8 weight gradients (the four row quantisations "
                         "and the GEMM) instead of the bf16 backward step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    return ap.parse_args()


# ------------------------------------------------------------ algorithmic cost
def stage_cost(stage: str, cfg, R: int) -> dict:
    """Algorithmic FLOPs and compulsory HBM bytes of one launch of a stage:
    every operand read once, every output written once (gathered rows count
    once per distinct row of the source).  R: routed rows held here."""
    T, D, F, El, k = cfg.tokens, cfg.d_model, cfg.d_ffn, cfg.num_local, cfg.top_k
    es = 2 if cfg.dtype == "bf16" else 4
    nT = F // 256 if cfg.dtype == "bf16" else F // 64
    tok = min(T, R) * D * es              # x or dy: the distinct token rows read (at most R)
    rowsF, rowsD = R * F * es, R * D * es
    w = El * D * F * es                   # W1 or W2
    if stage.startswith("fc2_dgrad"):     # dy rows, W2, h -> dh, per-N-tile partials
        return dict(flops=2.0 * R * D * F, bytes=tok + w + rowsF + rowsF + R * nT * 4 + R * 4)
    if stage.startswith("fc1_dgrad"):     # dh, W1 -> dx rows; the dprob combine (partials -> dprob)
        return dict(flops=2.0 * R * D * F, bytes=rowsF + w + rowsD + R * nT * 4 + T * k * 4)
    if stage.startswith("dx_combine"):    # dx rows -> dx
        return dict(flops=0.0, bytes=rowsD + tok + T * k * 4)
    if stage.startswith("wgrad_prep"):    # h, p -> act_p
        return dict(flops=0.0, bytes=2 * rowsF + R * 4)
    if stage.startswith("wgrad_fc1_fc2"):  # x, dy, dh, act_p -> dW1, dW2 (float32)
        return dict(flops=4.0 * R * D * F, bytes=2 * tok + 2 * rowsF + 2 * El * D * F * 4)
    if stage in ("wgrad_fc1", "wgrad_fc2"):
        return dict(flops=2.0 * R * D * F, bytes=tok + rowsF + El * D * F * 4)
    if stage in ("fc1_fwd", "fc2_fwd"):
        return dict(flops=2.0 * R * D * F, bytes=tok + w + 2 * rowsF)
    if stage.startswith("combine_gather"):
        return dict(flops=0.0, bytes=rowsD + tok + T * k * 8)
    # routing: chunk histograms of 16 tokens per local expert
    hist = (T + 15) // 16 * El * 4
    if stage == "route":                  # logits -> top-k indices and probabilities, chunk histograms
        return dict(flops=0.0, bytes=T * cfg.num_experts * 4 + T * k * 8 + hist)
    if stage == "permute_scan":           # histograms read twice, chunk bases written
        return dict(flops=0.0, bytes=3 * hist)
    if stage.startswith("permute_scatter"):  # top-k and bases -> slot_row, row_src, row_tok, row_prob
        return dict(flops=0.0, bytes=T * k * 8 + hist + T * k * 4 + R * 12)
    return dict(flops=0.0, bytes=0.0)


def roofline(stage: str, ms: float, cfg, R: int) -> dict:
    """Roofline of one launch: the bound is whichever of the FLOP time at the
    bf16 MFMA peak and the byte time at the HBM peak is longer; ``achieved``
    and ``peak`` are in that bound's unit and ``frac`` = achieved / peak
    (= bound time / measured time)."""
    c = stage_cost(stage, cfg, R)
    t_f = c["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    t_b = c["bytes"] / (HBM_PEAK_GBS * 1e9)
    sec = ms * 1e-3
    if t_f >= t_b:
        ach = c["flops"] / sec / 1e12
        return {"kernel": stage, "bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "flops_per_launch": c["flops"],
                "bytes_per_launch": c["bytes"], "ms_per_launch": round(ms, 5),
                "hbm_frac": round(c["bytes"] / sec / 1e9 / HBM_PEAK_GBS, 4)}
    ach = c["bytes"] / sec / 1e9
    return {"kernel": stage, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "flops_per_launch": c["flops"], "bytes_per_launch": c["bytes"],
            "ms_per_launch": round(ms, 5), "mfma_frac": round(c["flops"] / sec / 1e12 / BF16_PEAK_TFLOPS, 4)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ one workload
class Workload:
    """Device inputs, routing, saved h and output buffers of one workload."""

    def __init__(self, cfg):
        import numpy as np
        import torch
        import bitwise_deterministic_moe_amd as moe
        from synth import make_inputs
        self.cfg, self.moe, self.torch = cfg, moe, torch
        self.prob = moe.Problem.from_config(cfg)
        self.host = make_inputs(cfg)
        dev = "cuda"

        def up(a, dt):
            if dt == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        self.logits = torch.from_numpy(self.host["logits"]).to(dev)
        self.x, self.w1, self.w2, self.dy = (up(self.host[n], cfg.dtype) for n in ("x", "w1", "w2", "dy"))
        self.fwd_ws = torch.empty(max(moe.moe_workspace_size(self.prob)[0], 1), dtype=torch.uint8, device=dev)
        self.routing, self.h, self.y = moe.moe_fwd(self.prob, self.logits, self.x, self.w1, self.w2,
                                                   moe.DETERMINISTIC, ws=self.fwd_ws)
        torch.cuda.synchronize()
        self.R = self.routing.rows
        D, F, el = cfg.d_model, cfg.d_ffn, cfg.num_local
        dt = moe.TORCH_DTYPE[cfg.dtype]
        out_rows = cfg.tokens if cfg.combine else self.prob.rows_cap
        self.bufs = {}
        for mode in (moe.DETERMINISTIC, moe.ATOMIC):
            sz = moe.moe_workspace_size(self.prob, mode)
            self.bufs[mode] = dict(
                dx=torch.empty((out_rows, D), dtype=dt, device=dev),
                dprob=torch.empty((cfg.tokens, cfg.top_k), dtype=torch.float32, device=dev),
                dh=torch.empty((self.prob.rows_cap, F), dtype=dt, device=dev),
                dw1=torch.empty((el, D, F), dtype=torch.float32, device=dev),
                dw2=torch.empty((el, F, D), dtype=torch.float32, device=dev),
                ws1=torch.empty(max(sz[1], 1), dtype=torch.uint8, device=dev),
                ws2=torch.empty(max(sz[2], 1), dtype=torch.uint8, device=dev))

    def step(self, mode, ev1=None, ev2=None):
        moe, b = self.moe, self.bufs[mode]
        moe.moe_bwd_dgrad_dprob(self.prob, self.routing, self.dy, self.w1, self.w2, self.h, mode, dx=b["dx"],
                                dprob=b["dprob"], dh=b["dh"], ws=b["ws1"], events=ev1)
        moe.moe_bwd_wgrad(self.prob, self.routing, self.x, self.dy, self.h, b["dh"], mode, dw1=b["dw1"],
                          dw2=b["dw2"], ws=b["ws2"], events=ev2)

    def fwd(self, ev=None):
        self.moe.moe_fwd(self.prob, self.logits, self.x, self.w1, self.w2, self.moe.DETERMINISTIC,
                         routing=self.routing, h=self.h, y=self.y, ws=self.fwd_ws, events=ev)


def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def _iqr(v):
    if len(v) < 2:
        return 0.0
    q = statistics.quantiles(v, n=4)
    return q[2] - q[0]


def _busy():
    """A short spin kernel, so that the host has enqueued the next work before
    the GPU reaches it (no host-enqueue gap inside a timed step)."""
    import torch
    torch.cuda._sleep(100_000)


def measure(wl: "Workload", args, flush) -> dict:
    """Every timing of one workload (deterministic step back to back, cold and
    warm per-step medians, ABBA determinism tax, per-kernel stage times in
    both modes, forward)."""
    torch, moe, cfg = wl.torch, wl.moe, wl.cfg
    DET, ATOM = moe.DETERMINISTIC, moe.ATOMIC
    R, D, F = wl.R, cfg.d_model, cfg.d_ffn
    flops = 8.0 * R * D * F
    for _ in range(args.warmup):
        wl.step(DET)
        wl.step(ATOM)
    torch.cuda.synchronize()

    # K deterministic steps back to back (the headline number)
    t0, t1 = _ev(), _ev()
    torch.cuda.synchronize()
    _busy()
    t0.record()
    for _ in range(args.steps):
        wl.step(DET)
    t1.record()
    torch.cuda.synchronize()
    ms_det = t0.elapsed_time(t1) / args.steps

    # per-step medians, cold (flush written before every step) and warm
    def per_step(mode, cold):
        ts = []
        evs = []
        _busy()
        for _ in range(args.steps):
            if cold:
                flush.add_(1)
            e0, e1 = _ev(), _ev()
            e0.record()
            wl.step(mode)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) for a, b in evs]
        return statistics.median(ts), _iqr(ts)

    cold_med, cold_iqr = per_step(DET, True)
    warm_med, warm_iqr = per_step(DET, False)

    # determinism tax: deterministic (A) and atomic (B) steps interleaved A B B A,
    # one continuous stream of work (no synchronisation between steps), cold
    td, ta = [], []
    evs = []
    _busy()
    for i in range(args.steps):
        order = (DET, ATOM) if i % 2 == 0 else (ATOM, DET)
        for mode in order:
            flush.add_(1)
            e0, e1 = _ev(), _ev()
            e0.record()
            wl.step(mode)
            e1.record()
            evs.append((mode, e0, e1))
    torch.cuda.synchronize()
    for mode, a, b in evs:
        (td if mode == DET else ta).append(a.elapsed_time(b))
    med_d, med_a = statistics.median(td), statistics.median(ta)

    # per-kernel times (library stage events), cold, both modes
    def stage_times(mode):
        names1 = moe.moe_stage_names(wl.prob, mode, 1)
        names2 = moe.moe_stage_names(wl.prob, mode, 2)
        acc = {}
        for _ in range(args.stage_reps):
            ev1 = [_ev() for _ in range(len(names1) + 1)]
            ev2 = [_ev() for _ in range(len(names2) + 1)]
            for e in ev1 + ev2:   # materialise the events before handing them to the library
                e.record()
            flush.add_(1)
            _busy()
            wl.step(mode, ev1, ev2)
            torch.cuda.synchronize()
            for names, ev in ((names1, ev1), (names2, ev2)):
                for i, n in enumerate(names):
                    acc.setdefault(n, []).append(ev[i].elapsed_time(ev[i + 1]))
        return {n: statistics.median(v) for n, v in acc.items()}

    st_det = stage_times(DET)
    st_atom = stage_times(ATOM)
    gemm = ("fc2_dgrad", "fc1_dgrad", "wgrad_fc1")
    g_det = sum(v for n, v in st_det.items() if n.startswith(gemm))
    g_atom = sum(v for n, v in st_atom.items() if n.startswith(gemm))

    # forward (deterministic), warm, back to back
    for _ in range(2):
        wl.fwd()
    torch.cuda.synchronize()
    f0, f1 = _ev(), _ev()
    _busy()
    f0.record()
    for _ in range(args.steps):
        wl.fwd()
    f1.record()
    torch.cuda.synchronize()
    ms_fwd = f0.elapsed_time(f1) / args.steps
    names0 = moe.moe_stage_names(wl.prob, DET, 0)
    ev0 = [_ev() for _ in range(len(names0) + 1)]
    for e in ev0:
        e.record()
    _busy()
    wl.fwd(ev0)
    torch.cuda.synchronize()
    st_fwd = {n: ev0[i].elapsed_time(ev0[i + 1]) for i, n in enumerate(names0)}

    stage_roof = {n: roofline(n, v, cfg, R) for n, v in st_det.items()}
    dom = max((n for n in st_det if stage_cost(n, cfg, R)["flops"] > 0), key=lambda n: st_det[n])
    return {
        "routed_rows": R, "flops_per_step": flops,
        "ms_per_step": ms_det, "tflops": flops / (ms_det * 1e-3) / 1e12,
        "cold_ms_median": cold_med, "cold_ms_iqr": cold_iqr, "warm_ms_median": warm_med, "warm_ms_iqr": warm_iqr,
        "tax": {"tax": med_d / med_a - 1.0, "det_ms_median": med_d, "det_ms_iqr": _iqr(td),
                "atomic_ms_median": med_a, "atomic_ms_iqr": _iqr(ta), "pairs_abba": args.steps,
                "gemm_launches_tax": g_det / g_atom - 1.0, "gemm_launches_det_ms": g_det,
                "gemm_launches_atomic_ms": g_atom},
        "stages_ms_det": st_det, "stages_ms_atomic": st_atom, "stage_roofline": stage_roof,
        "dominant": dom,
        "fwd": {"ms": ms_fwd, "tflops": 4.0 * R * D * F / (ms_fwd * 1e-3) / 1e12, "stages_ms": st_fwd,
                "stage_roofline": {n: roofline(n, v, cfg, R) for n, v in st_fwd.items()}},
    }


def _r(v, n=5):
    if isinstance(v, float):
        return round(v, n)
    if isinstance(v, dict):
        return {k: _r(x, n) for k, x in v.items()}
    return v


def workload_desc(cfg, R) -> str:
    lay = "token layout" if cfg.combine else f"expert shard: experts {cfg.expert_begin}..{cfg.expert_begin + cfg.num_local - 1} of {cfg.num_experts}, row layout"
    skew = ", Zipf(1.1) routing skew" if cfg.skew else ""
    return (f"{cfg.name}: {cfg.tokens} tokens, d_model {cfg.d_model}, {cfg.num_experts} experts top-{cfg.top_k}{skew}, "
            f"{R} routed rows, expert MLP {cfg.d_model}->{cfg.d_ffn}->{cfg.d_model} ReLU^2, {cfg.dtype} storage, "
            f"fp32 dprob/dW, {lay}")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU's share of the layer; it takes --gpus 1 only "
                                   "(no multi-GPU path is built)"}))
        sys.exit(2)
    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4}))
        return

    import bitwise_deterministic_moe_amd as moe
    from synth import CONFIGS

    moe.load_library()
    cfg = CONFIGS[args.config]
    wl = Workload(cfg)
    if args.profile_only:
        run = mx_wgrad_runner(wl) if args.profile_mx_wgrad else (lambda: wl.step(moe.DETERMINISTIC))
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t0, t1 = _ev(), _ev()
        t0.record()
        for _ in range(args.steps):
            run()
        t1.record()
        torch.cuda.synchronize()
        print(json.dumps({"profile_only": True, "config": cfg.name, "ms_per_step": t0.elapsed_time(t1) / args.steps}))
        return
    flush = torch.empty(args.flush_mb * (1 << 20) // 4, dtype=torch.float32, device="cuda").zero_()
    m = measure(wl, args, flush)
    R = m["routed_rows"]
    dom = m["dominant"]
    roof = dict(m["stage_roofline"][dom])
    roof["traffic"] = measured_traffic(cfg.name, dom)
    value = m["tflops"]
    mfma_peak = measured_mfma_peak()
    result = {
        "metric": "MoE grouped-GEMM bwd TFLOP/s (det mode), % bf16 peak; determinism tax vs atomic",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "library_source_hash": moe.moe_source_hash(),
        "config": {"workload": workload_desc(cfg, R), "tokens": cfg.tokens, "d_model": cfg.d_model,
                   "d_ffn": cfg.d_ffn, "experts": cfg.num_experts, "top_k": cfg.top_k, "local_experts": cfg.num_local,
                   "routed_rows": R, "mode": "deterministic", "parallelism": "single GPU"},
        "pct_bf16_peak": round(100.0 * value / BF16_PEAK_TFLOPS, 2),
        "mfma_peak_measured": dict(mfma_peak, pct_of_measured=round(100.0 * value / mfma_peak["tflops"], 2)),
        "step_roofline": _r(step_roofline(m, cfg), 4),
        "cold_cache": _r({"flush_mb": args.flush_mb, "ms_median": m["cold_ms_median"], "ms_iqr": m["cold_ms_iqr"],
                          "tflops": m["flops_per_step"] / (m["cold_ms_median"] * 1e-3) / 1e12}),
        "warm_cache": _r({"ms_median": m["warm_ms_median"], "ms_iqr": m["warm_ms_iqr"],
                          "tflops": m["flops_per_step"] / (m["warm_ms_median"] * 1e-3) / 1e12}),
        "determinism_tax": _r(m["tax"], 5),
        "forward": _r(m["fwd"], 5),
        "stages_ms_det": _r(m["stages_ms_det"]),
        "stages_ms_atomic": _r(m["stages_ms_atomic"]),
        "stage_roofline": m["stage_roofline"],
        "roofline": roof,
    }
    if not args.no_extras:
        b = wl.bufs[moe.DETERMINISTIC]
        st = m["stages_ms_det"]
        if cfg.combine and cfg.num_local == cfg.num_experts:
            result["router_bwd"] = measured_router_bwd(cfg, wl.prob, wl.routing, wl.x, b["dprob"])
        result["mx_quantize"] = measured_mx_quantize(b["dh"][:R])
        result["nvfp4_quantize"] = measured_nvfp4_quantize(b["dh"][:R])
        result["mx_dgrad_fc1"] = measured_mx_dgrad_fc1(cfg, wl.prob, wl.routing, b["dh"], wl.w1,
                                                       st.get("fc1_dgrad_dprob_combine"))
        result["mx_dgrad_fc2"] = measured_mx_dgrad_fc2(cfg, wl.prob, wl.routing, wl.dy, wl.w2, wl.h, b["ws1"],
                                                       st.get("fc2_dgrad_dprob_partials"))
        result["mx_fwd"] = measured_mx_fwd(cfg, wl, m["fwd"]["stages_ms"])
        result["mx_wgrad"] = measured_mx_wgrad(cfg, wl, b["dh"], st.get("wgrad_prep_act_p", 0.0) +
                                               st.get("wgrad_fc1_fc2_ordered", float("nan")))
        result["fingerprint"] = measured_fingerprint(b["dw1"])
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, wl.host, R)
    del wl
    torch.cuda.empty_cache()
    subs = {}
    if args.sub_configs and args.sub_configs != "none":
        for name in args.sub_configs.split(","):
            if name == cfg.name:
                continue
            c = CONFIGS[name]
            w = Workload(c)
            s = measure(w, args, flush)
            d = s["dominant"]
            subs[name] = _r({"workload": workload_desc(c, s["routed_rows"]), "ms_per_step": s["ms_per_step"],
                             "tflops": s["tflops"], "pct_bf16_peak": 100.0 * s["tflops"] / BF16_PEAK_TFLOPS,
                             "step_roofline": step_roofline(s, c),
                             "cold_ms_median": s["cold_ms_median"], "warm_ms_median": s["warm_ms_median"],
                             "determinism_tax": s["tax"], "forward": s["fwd"], "stages_ms_det": s["stages_ms_det"],
                             "stages_ms_atomic": s["stages_ms_atomic"],
                             "roofline": dict(s["stage_roofline"][d], traffic=measured_traffic(name, d))}, 5)
            del w
            torch.cuda.empty_cache()
    result["other_workloads"] = subs
    print(json.dumps(result), flush=True)


def step_roofline(m, cfg) -> dict:
    """The whole step against its bound: the sum over its launches of
    max(FLOP time, byte time), divided by the measured step time."""
    R = m["routed_rows"]
    t_bound = 0.0
    for n in m["stages_ms_det"]:
        c = stage_cost(n, cfg, R)
        t_bound += max(c["flops"] / (BF16_PEAK_TFLOPS * 1e12), c["bytes"] / (HBM_PEAK_GBS * 1e9))
    return {"bound_ms": t_bound * 1e3, "frac": t_bound * 1e3 / m["ms_per_step"]}


def measured_fingerprint(t, reps=5):
    """moe_fingerprint of a float32 weight gradient (chunks of 65536): average
    of `reps` calls against HBM for one read of the tensor."""
    import torch
    import bitwise_deterministic_moe_amd as moe
    moe.moe_fingerprint(t, sync=False)
    torch.cuda.synchronize()
    e0, e1 = _ev(), _ev()
    e0.record()
    for _ in range(reps):
        moe.moe_fingerprint(t, sync=False)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nb = t.numel() * t.element_size()
    return {"tensor": f"dW1 {list(t.shape)} float32", "ms": round(ms, 5), "bytes": nb,
            "achieved_GBs": round(nb / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "elements_per_s": round(t.numel() / (ms * 1e-3), 1)}


def measured_mfma_peak(iters=20000, reps=5):
    """Attainable bf16 MFMA rate of this device: the library's register-only
    MFMA loop (moe_mfma_rate) on two workgroups per compute unit, best of
    `reps` timed launches.  The sink is checked against its closed form."""
    import torch
    import bitwise_deterministic_moe_amd as moe
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    v = 0.125
    sink = moe.moe_mfma_rate(blocks, 200, v)   # warm-up
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.moe_mfma_rate(blocks, iters, v, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, blocks * 4 * iters * 8 * 32768 / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    expect = 2048.0 * v * v * iters
    ok = bool(torch.all(sink == expect).item())
    return {"tflops": round(best, 1), "kernel": "v_mfma_f32_32x32x16_bf16 register loop", "blocks": blocks,
            "iters": iters, "sink_check": ok}


def measured_router_bwd(cfg, prob, routing, x, dprob, reps=20):
    """The router backward (outside the step) on the same routing and the
    step's dprob, with seeded router weights: average launch-sequence time over
    `reps` back-to-back calls, against HBM for its algorithmic bytes (x and
    the router weights read once, dlogits, dw_router and dx_router written once,
    the routing's per-slot arrays read once)."""
    import torch
    import bitwise_deterministic_moe_amd as moe
    from synth import make_router_inputs
    import numpy as np
    ri = make_router_inputs(cfg)
    wr = torch.from_numpy(np.ascontiguousarray(ri["wr"]).view(np.int16 if cfg.dtype == "bf16" else np.float32))
    wr = wr.cuda().view(torch.bfloat16) if cfg.dtype == "bf16" else wr.cuda()
    outs = moe.moe_router_bwd(prob, routing, dprob, x, wr)
    for mode in (moe.DETERMINISTIC, moe.ATOMIC):
        moe.moe_router_bwd(prob, routing, dprob, x, wr, mode, *outs)
    torch.cuda.synchronize()
    res = {}
    for name, mode in (("det", moe.DETERMINISTIC), ("atomic", moe.ATOMIC)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            moe.moe_router_bwd(prob, routing, dprob, x, wr, mode, *outs)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / reps
    T, E, D, k = cfg.tokens, cfg.num_experts, cfg.d_model, cfg.top_k
    es = 2 if cfg.dtype == "bf16" else 4
    hbm = T * D * es + E * D * es + T * E * 4 + E * D * 4 + T * D * es + T * k * 12 + T * k * 4
    # both reductions gather T*k rows of D elements (x rows for dw_router,
    # router rows for dx_router), which the L2 serves
    gather = 2 * T * k * D * es
    sec = res["det"] * 1e-3
    return {"ms_det": round(res["det"], 5), "ms_atomic": round(res["atomic"], 5),
            "tax": round(res["det"] / res["atomic"] - 1.0, 4), "hbm_bytes": hbm,
            "achieved_GBs": round(hbm / sec / 1e9, 1), "frac_hbm": round(hbm / sec / 1e9 / HBM_PEAK_GBS, 4),
            "gather_bytes": gather, "gather_GBs": round(gather / sec / 1e9, 1)}


def measured_nvfp4_quantize(t, reps=20):
    """NVFP4 quantisation (tensor amax pass, then E2M1 codes + E4M3 block
    scales) of the step's dh, average over `reps` calls (three launches each),
    against HBM for its bytes (read the tensor twice, write half a byte per
    element and one scale byte per 16 elements)."""
    import torch
    import bitwise_deterministic_moe_amd as moe
    moe.moe_nvfp4_quantize(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        moe.moe_nvfp4_quantize(t)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n = t.numel()
    hbm = 2 * n * t.element_size() + n // 2 + n // 16
    return {"tensor": f"dh {list(t.shape)} {str(t.dtype).replace('torch.', '')}", "ms": round(ms, 5),
            "hbm_bytes": hbm, "achieved_GBs": round(hbm / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def measured_mx_quantize(t, reps=20):
    """MXFP8 quantisation (E4M3 codes + E8M0 block scales) of the step's dh,
    average over `reps` back-to-back launches, against HBM for its bytes
    (read the tensor, write one code byte per element and one scale byte per
    32 elements)."""
    import torch
    import bitwise_deterministic_moe_amd as moe
    codes, scales = moe.moe_mx_quantize(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        moe.moe_mx_quantize(t, codes, scales)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n = t.numel()
    hbm = n * t.element_size() + n + n // 32
    return {"tensor": f"dh {list(t.shape)} {str(t.dtype).replace('torch.', '')}", "ms": round(ms, 5),
            "hbm_bytes": hbm, "achieved_GBs": round(hbm / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


FP8_PEAK_TFLOPS = 5033.2   # MI355X dense fp8 MFMA, vendor figure


def measured_mx_dgrad_fc1(cfg, prob, routing, dh, w1, bf16_ms, reps=20):
    """The MXFP8 variant of the fc1 data gradient (dx_rows = dh W1^T on E4M3
    codes with E8M0 block scales) on the step's dh and W1, quantised once
    outside the timed region; average of `reps` launches, against the dense
    fp8 peak, beside the bf16 fc1 dgrad stage of the same step."""
    import torch
    import bitwise_deterministic_moe_amd as moe
    if cfg.dtype != "bf16" or cfg.d_ffn > 2048:
        return None
    D, F, el = cfg.d_model, cfg.d_ffn, cfg.num_local
    dmx = moe.moe_mx_quantize(dh)
    wq = moe.moe_mx_quantize(w1.reshape(el * D, F))
    wmx = (wq[0].reshape(el, D, F), wq[1].reshape(el, D, F // 32))
    out = moe.moe_mx_dgrad_fc1(prob, routing, dmx, wmx)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        moe.moe_mx_dgrad_fc1(prob, routing, dmx, wmx, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * routing.rows * D * F
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 5), "tflops": round(tf, 1), "peak_fp8": FP8_PEAK_TFLOPS,
            "frac": round(tf / FP8_PEAK_TFLOPS, 4), "bf16_stage_ms": None if bf16_ms is None else round(bf16_ms, 5)}


def measured_mx_dgrad_fc2(cfg, prob, routing, dy, w2, h, ws, bf16_ms, reps=20):
    """The MXFP8 variant of the fc2 data gradient with its fused epilogue
    (dprob partials and their fixed-order combine, dh) on the step's
    dy, W2 and h, quantised once outside the timed region; deterministic
    mode, average of `reps` calls (GEMM launch + combine launch), against the
    dense fp8 peak, beside the bf16 fc2 dgrad stage (whose combine rides in
    the next launch)."""
    import torch
    import bitwise_deterministic_moe_amd as moe
    if cfg.dtype != "bf16" or cfg.d_model > 2048:
        return None
    D, F, el = cfg.d_model, cfg.d_ffn, cfg.num_local
    dymx = moe.moe_mx_quantize(dy)
    wq = moe.moe_mx_quantize(w2.reshape(el * F, D))
    wmx = (wq[0].reshape(el, F, D), wq[1].reshape(el, F, D // 32))
    dprob, dh = moe.moe_mx_dgrad_fc2(prob, routing, dymx, wmx, h, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        moe.moe_mx_dgrad_fc2(prob, routing, dymx, wmx, h, dprob=dprob, dh=dh, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * routing.rows * D * F
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 5), "tflops": round(tf, 1), "peak_fp8": FP8_PEAK_TFLOPS,
            "frac": round(tf / FP8_PEAK_TFLOPS, 4), "bf16_stage_ms": None if bf16_ms is None else round(bf16_ms, 5)}


def measured_mx_fwd(cfg, wl, bf16_stages, reps=20):
    """The MXFP8 forward GEMMs on the workload's x, W1 and W2 (quantised once
    outside the timed region, the weights along their contraction axis):
    fc1 (h and relu(h)^2) and fc2 with the fixed-order combine, average of
    `reps` calls each, against the dense fp8 peak, beside the bf16 forward
    stages."""
    import torch
    import bitwise_deterministic_moe_amd as moe
    if cfg.dtype != "bf16" or cfg.d_model > 2048 or cfg.d_ffn > 2048:
        return None
    xmx, w1t, w2t = moe.moe_mx_quantize(wl.x), moe.moe_mx_quantize_t(wl.w1), moe.moe_mx_quantize_t(wl.w2)
    h, act = moe.moe_mx_fwd_fc1(wl.prob, wl.routing, xmx, w1t)
    amx = moe.moe_mx_quantize(act)
    y = moe.moe_mx_fwd_fc2(wl.prob, wl.routing, amx, w2t, ws=wl.fwd_ws)
    torch.cuda.synchronize()
    res = {}
    flops = 2.0 * wl.R * cfg.d_model * cfg.d_ffn
    for name, fn in (("fc1", lambda: moe.moe_mx_fwd_fc1(wl.prob, wl.routing, xmx, w1t, h=h, act=act)),
                     ("fc2_combine", lambda: moe.moe_mx_fwd_fc2(wl.prob, wl.routing, amx, w2t, y=y, ws=wl.fwd_ws))):
        e0, e1 = _ev(), _ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 5), "tflops": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)}
    res["fc1"]["bf16_stage_ms"] = round(bf16_stages.get("fc1_fwd", float("nan")), 5)
    res["fc2_combine"]["bf16_stage_ms"] = round(bf16_stages.get("fc2_fwd", float("nan")) +
                                                bf16_stages.get("combine_gather", 0.0), 5)
    return res


def mx_wgrad_runner(wl):
    """A closure running the MXFP8 weight gradients once on the workload:
    dh from one deterministic bf16 data-gradient call, then the four row
    quantisations and the GEMM into preallocated buffers."""
    import bitwise_deterministic_moe_amd as moe
    b = wl.bufs[moe.DETERMINISTIC]
    moe.moe_bwd_dgrad_dprob(wl.prob, wl.routing, wl.dy, wl.w1, wl.w2, wl.h, moe.DETERMINISTIC, dx=b["dx"],
                            dprob=b["dprob"], dh=b["dh"], ws=b["ws1"])
    srcs = (("x", wl.x, moe.MXW_TOKEN), ("dh", b["dh"], moe.MXW_ROW), ("act", wl.h, moe.MXW_ACT_P),
            ("dy", wl.dy, moe.MXW_TOKEN))
    enc = {n: moe.moe_mx_quantize_wgrad(wl.prob, wl.routing, t, k) for n, t, k in srcs}

    def run():
        for n, t, k in srcs:
            moe.moe_mx_quantize_wgrad(wl.prob, wl.routing, t, k, *enc[n])
        moe.moe_mx_wgrad(wl.prob, wl.routing, enc["x"], enc["dh"], enc["act"], enc["dy"], dw1=b["dw1"],
                         dw2=b["dw2"])
    return run


def measured_mx_wgrad(cfg, wl, dh, bf16_ms, reps=10):
    """The MXFP8 weight gradients on the workload's x, dY, saved h and the
    backward's dh: the four row-quantised encodings (moe_mx_quantize_wgrad)
    and the GEMM of both dW (moe_mx_wgrad), average of `reps` calls each,
    beside the bf16 weight-gradient stages.  The GEMM stores 2 El D F float32
    and reads each operand about once from HBM; its bound is
    max(FLOP time at the fp8 peak, those bytes at HBM peak)."""
    import torch
    import bitwise_deterministic_moe_amd as moe
    if cfg.dtype != "bf16":
        return None
    D, F, el = cfg.d_model, cfg.d_ffn, cfg.num_local
    srcs = (("x", wl.x, moe.MXW_TOKEN), ("dh", dh, moe.MXW_ROW), ("act", wl.h, moe.MXW_ACT_P),
            ("dy", wl.dy, moe.MXW_TOKEN))
    enc = {n: moe.moe_mx_quantize_wgrad(wl.prob, wl.routing, t, k) for n, t, k in srcs}
    dw1, dw2 = moe.moe_mx_wgrad(wl.prob, wl.routing, enc["x"], enc["dh"], enc["act"], enc["dy"])
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = _ev(), _ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def quantise_all():
        for n, t, k in srcs:
            moe.moe_mx_quantize_wgrad(wl.prob, wl.routing, t, k, *enc[n])

    q_ms = timed(quantise_all)
    g_ms = timed(lambda: moe.moe_mx_wgrad(wl.prob, wl.routing, enc["x"], enc["dh"], enc["act"], enc["dy"],
                                          dw1=dw1, dw2=dw2))
    rp = moe.moe_mx_wgrad_rows(wl.prob)
    counts = wl.routing.counts.long()
    P = int(((counts + 63) // 64 * 64).sum().item())
    flops = 4.0 * wl.R * D * F
    out_bytes = 2.0 * el * D * F * 4
    in_bytes = 2.0 * (D + F) * P * (1 + 1 / 32)
    bound_ms = max(flops / (FP8_PEAK_TFLOPS * 1e12), (out_bytes + in_bytes) / (HBM_PEAK_GBS * 1e9)) * 1e3
    return {"gemm_ms": round(g_ms, 5), "gemm_tflops": round(flops / (g_ms * 1e-3) / 1e12, 1),
            "gemm_GBs": round((out_bytes + in_bytes) / (g_ms * 1e-3) / 1e9, 1),
            "gemm_traffic": measured_traffic(cfg.name, "mx_wgrad"),
            "gemm_bound_ms": round(bound_ms, 5), "gemm_frac_of_bound": round(bound_ms / g_ms, 4),
            "quantise_ms": round(q_ms, 5), "padded_rows": P, "rows": wl.R, "rpad_cap": rp,
            "bf16_wgrad_ms": round(bf16_ms, 5), "total_ms": round(q_ms + g_ms, 5)}


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` from profiles/<workload>_hbm_traffic.txt
    (rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a plain-copy calibration), or
    None when the running library was built from other sources than the
    profiled one."""
    import bitwise_deterministic_moe_amd as moe
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        parts = line.split()
        if not parts or parts[0].startswith("#"):
            continue
        if parts[0] == "stage" and len(parts) >= 8:
            fields[("stage", parts[1])] = float(parts[7])
        elif len(parts) == 2:
            fields[parts[0]] = parts[1]
    if fields.get("source_hash") != moe.moe_source_hash():
        return None
    return fields.get(("stage", stage))


def cpu_baseline(cfg, host, R):
    """The oracle's backward (numpy, as it stands) on the same inputs, on this
    host's cores: oracle.expert_backward over every local expert in order
    (what oracle.backward does, one expert's float64 weights at a time, so
    that the 512-expert layer needs no 34 GB of float64 weights).  The saved
    h comes from oracle.expert_forward outside the timed calls.  Also the
    same code on float32 arrays over the first experts (a bounded sample)."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    import oracle
    idx, p = oracle.route(host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, cfg.num_local)
    off, row_tok, row_src = perm["offsets"], perm["row_tok"], perm["row_src"]
    p_rows = p.reshape(-1)[row_src]
    x = oracle.decode(host["x"], cfg.dtype)
    dy = oracle.decode(host["dy"], cfg.dtype)

    def run(dtype, experts):
        sec, rows = 0.0, 0
        for e in experts:
            s, t = int(off[e]), int(off[e + 1])
            if t == s:
                continue
            w1 = oracle.decode(host["w1"][e], cfg.dtype).astype(dtype)
            w2 = oracle.decode(host["w2"][e], cfg.dtype).astype(dtype)
            xr, dyr, pr = x[row_tok[s:t]].astype(dtype), dy[row_tok[s:t]].astype(dtype), p_rows[s:t].astype(dtype)
            h, _ = oracle.expert_forward(xr, w1, w2)
            t0 = time.perf_counter()
            oracle.expert_backward(xr, dyr, pr, h, w1, w2)
            sec += time.perf_counter() - t0
            rows += t - s
        return sec, rows

    el = cfg.num_local
    sec64, rows64 = run(np.float64, range(el))
    n32 = min(el, 64)
    sec32, rows32 = run(np.float32, range(n32))
    fl = lambda rows: 8.0 * rows * cfg.d_model * cfg.d_ffn  # noqa: E731
    return {"value": round(fl(rows64) / sec64 / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
            "sample": f"float64 oracle backward (oracle.expert_backward) over all {el} local experts of "
                      f"{cfg.name}, {rows64} routed rows, {sec64:.2f} s of timed calls",
            "seconds_per_step": round(sec64, 3),
            "fp32_variant": {"value": round(fl(rows32) / sec32 / 1e12, 5), "unit": "TFLOP/s",
                             "sample": f"the same calls on float32 arrays, first {n32} experts ({rows32} rows), "
                                       f"{sec32:.2f} s"}}


if __name__ == "__main__":
    main()
