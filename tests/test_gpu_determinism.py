"""Bit-identity of every output across repeated runs and across shuffled
workgroup launch orders (fingerprints, never tolerances), the atomic-mode
negative control, and poisoned outputs/workspaces."""
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
from synth import CONFIGS
from harness import REPEATS, SHUFFLE_SEEDS, LayerRunner, determinism_runs, device_inputs, fingerprints, run_layer
from test_gpu_parity import EDGE

pytestmark = pytest.mark.gpu

SEEDS = [0, 1, 0x5EED, 0xDEADBEEF]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    moe.load_library()


def _fps(cfg, di, seed, mode=moe.DETERMINISTIC, poison=None):
    out = run_layer(moe.Problem.from_config(cfg, shuffle_seed=seed), di, mode, poison=poison)
    return fingerprints(out, cfg.combine)


@pytest.mark.parametrize("name", ["tiny_fp32", "bf16_e8k2"])
def test_det_bits_identical_20_repeats_and_4_shuffles(name):
    """Every output and routing array bit-identical over 20 repeated runs and
    under four shuffled workgroup orders (twice each).  The three full-size
    workloads get the same runs in test_gpu_large.py."""
    cfg = CONFIGS[name]
    n = determinism_runs(LayerRunner(moe.Problem.from_config(cfg), device_inputs(cfg)), cfg.combine, label=name)
    assert n == REPEATS + 2 * len(SHUFFLE_SEEDS)


@pytest.mark.parametrize("name", ["split_k_bf16", "split_k_fp32", "shard_bf16", "empty_experts_bf16",
                                  "max_experts_bf16", "max_chunk_split_bf16"])
def test_det_bits_identical_across_repeats_and_shuffles(name):
    cfg = CONFIGS.get(name) or EDGE[name]
    determinism_runs(LayerRunner(moe.Problem.from_config(cfg), device_inputs(cfg)), cfg.combine, repeats=4,
                     label=name)


def test_poisoned_outputs_and_workspace_give_same_bits():
    for name in ("bf16_e8k2", "split_k_bf16", "split_k_fp32", "shard_bf16"):
        cfg = CONFIGS.get(name) or EDGE[name]
        di = device_inputs(cfg)
        ref = _fps(cfg, di, 0)
        for poison in (float("nan"), -7.5e30):
            assert _fps(cfg, di, 0, poison=poison) == ref, (name, poison)


@pytest.mark.parametrize("name,keys", [("bf16_e8k2", ("dprob",)), ("split_k_bf16", ("dw1", "dw2")),
                                       ("split_k_fp32", ("dw1", "dw2"))])
def test_atomic_mode_is_order_dependent(name, keys):
    """Negative control: with shuffled launch orders the atomic reduction
    sites (dprob over 8 N-tiles; split-K wgrad over 3 chunks) must produce
    differing bits, which shows the harness can see nondeterminism."""
    cfg = CONFIGS.get(name) or EDGE[name]
    di = device_inputs(cfg)
    seen = {k: set() for k in keys}
    for seed in range(1, 9):
        fp = _fps(cfg, di, seed, mode=moe.ATOMIC)
        for k in keys:
            seen[k].add(fp[k])
    for k in keys:
        assert len(seen[k]) >= 2, f"atomic {k} never changed over 8 shuffled runs"
