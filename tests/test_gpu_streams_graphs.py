"""The C ABI enqueues everything on the stream it is given and allocates,
copies and synchronises nothing, so the whole layer runs on a side stream
and can be captured in a HIP graph.  Checked here against an eager run on
the default stream, bit for bit (fingerprints of every output and routing
array):
  * forward + both backward calls enqueued on a side stream;
  * the same three calls captured once in a graph and replayed several
    times, with eager work and synchronisations between the replays and the
    outputs poisoned before each replay;
  * moe_bwd_dgrad_dprob_noalloc (workspace in the library's static array)
    captured in a graph, against the eager workspace entry point."""
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
from harness import LayerRunner, device_inputs, fingerprints
from synth import CONFIGS
from test_gpu_parity import EDGE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()


def _enqueue(runner: LayerRunner):
    """The layer's three calls into the runner's buffers, no synchronisation."""
    prob, di = runner.prob, runner.di
    moe.moe_fwd(prob, di.logits, di.x, di.w1, di.w2, runner.mode, routing=runner.routing, h=runner.h, y=runner.y,
                ws=runner.ws[0])
    moe.moe_bwd_dgrad_dprob(prob, runner.routing, di.dy, di.w1, di.w2, runner.h, runner.mode, dx=runner.dx,
                            dprob=runner.dprob, dh=runner.dh, ws=runner.ws[1])
    moe.moe_bwd_wgrad(prob, runner.routing, di.x, di.dy, runner.h, runner.dh, runner.mode, dw1=runner.dw1,
                      dw2=runner.dw2, ws=runner.ws[2])


def _outputs(runner: LayerRunner) -> dict:
    return dict(routing=runner.routing, h=runner.h, y=runner.y, dx=runner.dx, dprob=runner.dprob, dh=runner.dh,
                dw1=runner.dw1, dw2=runner.dw2)


def _poison(runner: LayerRunner):
    for t in (runner.h, runner.y, runner.dx, runner.dprob, runner.dh, runner.dw1, runner.dw2):
        t.fill_(float("nan"))
    for w in runner.ws:
        w.fill_(171)


@pytest.mark.parametrize("name", ["bf16_e8k2", "tiny_fp32", "ragged_bf16", "shard_bf16"])
def test_side_stream_and_graph_replays_match_eager(name):
    cfg = CONFIGS.get(name) or EDGE[name]
    print(f"streams/graphs {name}", flush=True)
    di = device_inputs(cfg)
    prob = moe.Problem.from_config(cfg)
    runner = LayerRunner(prob, di)
    ref = fingerprints(runner.run(0), cfg.combine)

    # side stream
    _poison(runner)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _enqueue(runner)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    fp = fingerprints(_outputs(runner), cfg.combine)
    assert fp == ref, [k for k in ref if fp[k] != ref[k]]

    # one graph of the whole layer, replayed with eager work in between
    graph = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        _enqueue(runner)
    torch.cuda.synchronize()
    for i in range(3):
        _poison(runner)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        fp = fingerprints(_outputs(runner), cfg.combine)
        assert fp == ref, (i, [k for k in ref if fp[k] != ref[k]])
        # eager work on the same buffers between replays (a shuffled run)
        fp_eager = fingerprints(runner.run(0x5EED), cfg.combine)
        assert fp_eager == ref, (i, [k for k in ref if fp_eager[k] != ref[k]])


def test_noalloc_entry_point_in_a_graph():
    cfg = CONFIGS["bf16_e8k2"]
    di = device_inputs(cfg)
    prob = moe.Problem.from_config(cfg)
    routing, h, _ = moe.moe_fwd(prob, di.logits, di.x, di.w1, di.w2)
    ref = moe.moe_bwd_dgrad_dprob(prob, routing, di.dy, di.w1, di.w2, h)
    torch.cuda.synchronize()
    ref_fp = [moe.moe_fingerprint(t.contiguous())[1] for t in ref]
    dt = moe.TORCH_DTYPE[cfg.dtype]
    dx = torch.empty((cfg.tokens, cfg.d_model), dtype=dt, device="cuda")
    dprob = torch.empty((cfg.tokens, cfg.top_k), dtype=torch.float32, device="cuda")
    dh = torch.empty((prob.rows_cap, cfg.d_ffn), dtype=dt, device="cuda")
    # the first call on a device looks up the static array's address
    moe.moe_bwd_dgrad_dprob_noalloc(prob, routing, di.dy, di.w1, di.w2, h, dx, dprob, dh)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        moe.moe_bwd_dgrad_dprob_noalloc(prob, routing, di.dy, di.w1, di.w2, h, dx, dprob, dh)
    torch.cuda.synchronize()
    for i in range(3):
        for t in (dx, dprob, dh):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        fp = [moe.moe_fingerprint(t.contiguous())[1] for t in (dx, dprob, dh)]
        assert fp == ref_fp, i
        # eager calls of both entry points between replays
        moe.moe_bwd_dgrad_dprob(prob, routing, di.dy, di.w1, di.w2, h)
        moe.moe_bwd_dgrad_dprob_noalloc(prob, routing, di.dy, di.w1, di.w2, h, dx, dprob, dh)
        torch.cuda.synchronize()
