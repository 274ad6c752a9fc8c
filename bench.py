#!/usr/bin/env python3
"""Benchmark of the bitwise-deterministic MoE grouped-GEMM backward on one
MI355X.

A step is one backward of the expert layer: moe_bwd_dgrad_dprob followed by
moe_bwd_wgrad (fc2 dgrad with the dprob partial epilogue, the fixed-order
dprob combine, fc1 dgrad, the fixed-order dx combine, both split-K weight
gradients and their ordered reduction) on the default workload: 4096 tokens,
d_model 1024, 8 experts, top-2, expert MLP 1024 -> 2048 -> 1024 with ReLU^2,
bf16 storage, float32 accumulation and float32 dprob / dW.  The inputs are
seeded synthetic tensors already resident in HBM, and routing and the saved h
come from one untimed moe_fwd.

Prints one JSON line.  ``value`` is 8*R*D*F / (time of one deterministic
step), in TFLOP/s.  The determinism tax compares deterministic with atomic
steps, which are interleaved step by step.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
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
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="bf16_e8k2")
    ap.add_argument("--stage-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + timed steps only (for rocprofv3 runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs the layer on one GPU; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
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
    from synth import CONFIGS, make_inputs

    moe.load_library()
    cfg = CONFIGS[args.config]
    prob = moe.Problem.from_config(cfg)
    host = make_inputs(cfg)
    dev = "cuda"

    def up(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    logits = torch.from_numpy(host["logits"]).to(dev)
    x, w1, w2, dy = (up(host[n], cfg.dtype) for n in ("x", "w1", "w2", "dy"))
    routing, h, _ = moe.moe_fwd(prob, logits, x, w1, w2, moe.DETERMINISTIC)
    torch.cuda.synchronize()
    R = routing.rows
    D, F, el = cfg.d_model, cfg.d_ffn, cfg.num_local
    flops = 8.0 * R * D * F
    gemm_flops = 2.0 * R * D * F
    dt = moe.TORCH_DTYPE[cfg.dtype]
    out_rows = cfg.tokens if cfg.combine else prob.rows_cap

    class Bufs:
        def __init__(self, mode):
            self.mode = mode
            self.dx = torch.empty((out_rows, D), dtype=dt, device=dev)
            self.dprob = torch.empty((cfg.tokens, cfg.top_k), dtype=torch.float32, device=dev)
            self.dh = torch.empty((prob.rows_cap, F), dtype=dt, device=dev)
            self.act_p = torch.empty((prob.rows_cap, F), dtype=dt, device=dev)
            self.dw1 = torch.empty((el, D, F), dtype=torch.float32, device=dev)
            self.dw2 = torch.empty((el, F, D), dtype=torch.float32, device=dev)
            sz = moe.moe_workspace_size(prob, mode)
            self.ws1 = torch.empty(max(sz[1], 1), dtype=torch.uint8, device=dev)
            self.ws2 = torch.empty(max(sz[2], 1), dtype=torch.uint8, device=dev)

    def step(b, ev1=None, ev2=None):
        moe.moe_bwd_dgrad_dprob(prob, routing, dy, w1, w2, h, b.mode, dx=b.dx, dprob=b.dprob, dh=b.dh,
                                act_p=b.act_p, ws=b.ws1, events=ev1)
        moe.moe_bwd_wgrad(prob, routing, x, dy, b.dh, b.act_p, b.mode, dw1=b.dw1, dw2=b.dw2, ws=b.ws2, events=ev2)

    det, atom = Bufs(moe.DETERMINISTIC), Bufs(moe.ATOMIC)
    for _ in range(args.warmup):
        step(det)
        step(atom)
    torch.cuda.synchronize()

    # ---- timed region: K deterministic steps back to back
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    t0, t1 = E(), E()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step(det)
    t1.record()
    torch.cuda.synchronize()
    ms_det = t0.elapsed_time(t1) / args.steps
    if args.profile_only:
        print(json.dumps({"profile_only": True, "ms_per_step": ms_det}))
        return

    # ---- determinism tax: det and atomic steps interleaved, per-step events
    td, ta = [], []
    for _ in range(args.steps):
        e = [E() for _ in range(3)]
        e[0].record()
        step(det)
        e[1].record()
        step(atom)
        e[2].record()
        torch.cuda.synchronize()
        td.append(e[0].elapsed_time(e[1]))
        ta.append(e[1].elapsed_time(e[2]))
    med_d, med_a = statistics.median(td), statistics.median(ta)

    def iqr(v):
        q = statistics.quantiles(v, n=4)
        return q[2] - q[0]

    # ---- per-kernel times through the library's stage-event hook
    def stage_times(mode, b):
        names1 = moe.moe_stage_names(prob, mode, 1)
        names2 = moe.moe_stage_names(prob, mode, 2)
        acc = {}
        for _ in range(args.stage_reps):
            ev1 = [E() for _ in range(len(names1) + 1)]
            ev2 = [E() for _ in range(len(names2) + 1)]
            for e in ev1 + ev2:   # materialise the events before handing them to the library
                e.record()
            step(b, ev1, ev2)
            torch.cuda.synchronize()
            for names, ev in ((names1, ev1), (names2, ev2)):
                for i, n in enumerate(names):
                    acc.setdefault(n, []).append(ev[i].elapsed_time(ev[i + 1]))
        return {n: statistics.mean(v) for n, v in acc.items()}

    st_det = stage_times(moe.DETERMINISTIC, det)
    st_atom = stage_times(moe.ATOMIC, atom)
    # grouped GEMMs per launch of each GEMM stage (both weight gradients share one launch for bf16)
    gemms_in = {"fc2_dgrad_dprob_partials": 1, "fc1_dgrad_dprob_combine": 1, "wgrad_fc1": 1, "wgrad_fc2": 1,
                "wgrad_fc1_fc2": 2}
    gemm_stages = [n for n in gemms_in if n in st_det]
    dom = max(gemm_stages, key=lambda n: st_det[n])
    dom_ms = st_det[dom]
    dom_flops = gemms_in[dom] * gemm_flops
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12

    value = flops / (ms_det * 1e-3) / 1e12
    mfma_peak = measured_mfma_peak()
    router = measured_router_bwd(cfg, prob, routing, x, det.dprob) if cfg.combine and el == cfg.num_experts else None
    mxq = measured_mx_quantize(det.dh[: R])
    nvq = measured_nvfp4_quantize(det.dh[: R])
    mxg = measured_mx_dgrad_fc1(cfg, prob, routing, det.dh, w1, st_det.get("fc1_dgrad_dprob_combine"))
    mxg2 = measured_mx_dgrad_fc2(cfg, prob, routing, dy, w2, h, det.ws1, st_det.get("fc2_dgrad_dprob_partials"))
    result = {
        "metric": "MoE grouped-GEMM bwd TFLOP/s (det mode), % bf16 peak; determinism tax vs atomic",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_det, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.tokens} tokens, d_model {D}, {cfg.num_experts} experts top-{cfg.top_k}, "
                               f"expert MLP {D}->{F}->{D} ReLU^2, {cfg.dtype} storage, fp32 dprob/dW",
                   "tokens": cfg.tokens, "d_model": D, "d_ffn": F, "experts": cfg.num_experts,
                   "top_k": cfg.top_k, "routed_rows": R, "mode": "deterministic", "parallelism": "single GPU"},
        "pct_bf16_peak": round(100.0 * value / BF16_PEAK_TFLOPS, 2),
        "mfma_peak_measured": dict(mfma_peak, pct_of_measured=round(100.0 * value / mfma_peak["tflops"], 2)),
        "determinism_tax": {
            "tax": round(med_d / med_a - 1.0, 4),
            "det_ms_median": round(med_d, 5), "det_ms_iqr": round(iqr(td), 5),
            "atomic_ms_median": round(med_a, 5), "atomic_ms_iqr": round(iqr(ta), 5),
            "interleaved_pairs": args.steps,
        },
        "router_bwd": router,
        "mx_quantize": mxq,
        "nvfp4_quantize": nvq,
        "mx_dgrad_fc1": mxg,
        "mx_dgrad_fc2": mxg2,
        "stages_ms_det": {k: round(v, 5) for k, v in st_det.items()},
        "stages_ms_atomic": {k: round(v, 5) for k, v in st_atom.items()},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(dom) if args.config == "bf16_e8k2" else None,
                     "flops_per_launch": dom_flops, "ms_per_launch": round(dom_ms, 5)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, host, flops)
    print(json.dumps(result), flush=True)


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
    (dprob partials and their fixed-order combine, dh, act_p) on the step's
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
    dprob, dh, act_p = moe.moe_mx_dgrad_fc2(prob, routing, dymx, wmx, h, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        moe.moe_mx_dgrad_fc2(prob, routing, dymx, wmx, h, dprob=dprob, dh=dh, act_p=act_p, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * routing.rows * D * F
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 5), "tflops": round(tf, 1), "peak_fp8": FP8_PEAK_TFLOPS,
            "frac": round(tf / FP8_PEAK_TFLOPS, 4), "bf16_stage_ms": None if bf16_ms is None else round(bf16_ms, 5)}


def measured_traffic(stage):
    """HBM bytes per launch of `stage` from profiles/bench_bf16_e8k2_hbm_traffic.txt
    (rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a plain-copy calibration), or
    None when the library source changed since those counters were taken."""
    import glob
    import hashlib
    path = os.path.join(ROOT, "profiles", "bench_bf16_e8k2_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    m = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "bitwise_deterministic_moe_amd", "csrc", "*"))):
        m.update(os.path.basename(f).encode())
        m.update(open(f, "rb").read())
    fields = {}
    for line in open(path):
        parts = line.split()
        if not parts or parts[0].startswith("#"):
            continue
        if parts[0] == "stage" and len(parts) >= 8:
            fields[("stage", parts[1])] = float(parts[7])
        elif len(parts) == 2:
            fields[parts[0]] = parts[1]
    if fields.get("csrc_sha256") != m.hexdigest()[:16]:
        return None
    return fields.get(("stage", stage))


def cpu_baseline(cfg, host, gpu_flops):
    """The oracle's backward (float64 numpy, as it stands) on the same inputs."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    import oracle
    idx, p = oracle.route(host["logits"], cfg.top_k)
    perm = oracle.permute(idx, cfg.expert_begin, cfg.num_local)
    x, w1, w2, dy = (oracle.decode(host[n], cfg.dtype) for n in ("x", "w1", "w2", "dy"))
    h = oracle.forward(x, w1, w2, p, perm, cfg.top_k, combine=bool(cfg.combine))["h"]
    times = []
    t_end = time.perf_counter() + 10.0
    while len(times) < 3 and (not times or time.perf_counter() < t_end):
        t = time.perf_counter()
        oracle.backward(x, w1, w2, h, dy, p, perm, cfg.top_k, combine=bool(cfg.combine))
        times.append(time.perf_counter() - t)
    sec = statistics.median(times)
    R = int(perm["offsets"][-1])
    fl = 8.0 * R * cfg.d_model * cfg.d_ffn
    return {"value": round(fl / sec / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full float64 oracle backward of {cfg.name} (all {cfg.num_local} experts, {R} rows), "
                      f"median of {len(times)} runs, {sec:.2f} s each",
            "seconds_per_step": round(sec, 3)}


if __name__ == "__main__":
    main()
