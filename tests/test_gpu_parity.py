"""HIP path vs the CPU oracle, element by element, on seeded inputs:
integers exact, floating point within rel-L2 2e-2 (bf16 storage) or 1e-5
(fp32 storage), topk_prob within 1e-5."""
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
from synth import CONFIGS, Config
from harness import (compare_layer, compare_layer_unordered, device_inputs, oracle_layer, run_layer)

pytestmark = pytest.mark.gpu

# Small shapes that still span several tiles and a ragged tail, plus the
# degenerate cases of the method.
EDGE = {
    "ragged_bf16": Config("ragged_bf16", 700, 256, 512, 5, 2, 0, 5, "bf16", 1, 11),
    "many_experts_bf16": Config("many_experts_bf16", 200, 256, 256, 64, 8, 0, 64, "bf16", 1, 12),
    "single_token_bf16": Config("single_token_bf16", 1, 256, 256, 6, 3, 0, 6, "bf16", 1, 13),
    "dense_e1k1_bf16": Config("dense_e1k1_bf16", 130, 256, 512, 1, 1, 0, 1, "bf16", 1, 14),
    "k_equals_e_bf16": Config("k_equals_e_bf16", 70, 256, 256, 4, 4, 0, 4, "bf16", 1, 15),
    "shard_bf16": Config("shard_bf16", 500, 256, 512, 16, 4, 5, 3, "bf16", 0, 16),
    "empty_experts_bf16": Config("empty_experts_bf16", 260, 256, 256, 16, 2, 0, 16, "bf16", 1, 17,
                                 skew="zipf", zipf_beta=0.3),
    "split_k_bf16": Config("split_k_bf16", 2048, 256, 256, 16, 1, 0, 16, "bf16", 1, 18, skew="zipf",
                           zipf_beta=2.0, zipf_empty=2),
    "no_tokens_bf16": Config("no_tokens_bf16", 0, 256, 256, 4, 2, 0, 4, "bf16", 1, 19),
    # mean 750 rows per expert: the fc1 dgrad runs the 192-row tile list
    # (three full tiles and a ragged one per expert), the fc2 dgrad 256-row tiles
    "rows192_bf16": Config("rows192_bf16", 1500, 256, 512, 4, 2, 0, 4, "bf16", 1, 22),
    # the widest router the library takes: 1024 experts, all local (the
    # routing scan's block holds exactly one thread per expert)
    "max_experts_bf16": Config("max_experts_bf16", 300, 256, 256, 1024, 8, 0, 1024, "bf16", 1, 24),
    "ragged_fp32": Config("ragged_fp32", 37, 64, 192, 3, 2, 0, 3, "f32", 1, 20),
    # float32 storage with experts above the chunk (4 x 128 mean rows = 512):
    # the float32 weight-gradient kernels' partial slots and ordered reduction
    "split_k_fp32": Config("split_k_fp32", 2048, 64, 128, 16, 1, 0, 16, "f32", 1, 23, skew="zipf",
                           zipf_beta=2.0, zipf_empty=2),
    "shard_fp32": Config("shard_fp32", 90, 128, 64, 8, 3, 2, 4, "f32", 0, 21),
    # one expert holding the largest weight-gradient chunk (4096 rows) whole,
    # and one holding two such chunks (8192 rows: split, ordered reduction):
    # the gathered-row table is filled to its last padded entry
    "max_chunk_bf16": Config("max_chunk_bf16", 4096, 256, 256, 1, 1, 0, 1, "bf16", 1, 25),
    "max_chunk_split_bf16": Config("max_chunk_split_bf16", 8192, 256, 256, 1, 1, 0, 1, "bf16", 1, 26),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()


def _run(cfg, mode=moe.DETERMINISTIC):
    di = device_inputs(cfg)
    out = run_layer(moe.Problem.from_config(cfg), di, mode)
    ref = oracle_layer(cfg, di.host)
    return out, ref


@pytest.mark.parametrize("name", ["tiny_fp32", "bf16_e8k2"])
def test_config_parity_det(name):
    cfg = CONFIGS[name]
    out, ref = _run(cfg)
    errs = compare_layer(cfg, out, ref)
    print(name, errs)


@pytest.mark.parametrize("name", ["tiny_fp32", "bf16_e8k2"])
def test_config_parity_atomic(name):
    cfg = CONFIGS[name]
    out, ref = _run(cfg, moe.ATOMIC)
    print(name, compare_layer_unordered(cfg, out, ref))


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_parity(name):
    cfg = EDGE[name]
    out, ref = _run(cfg)
    print(name, compare_layer(cfg, out, ref))


@pytest.mark.parametrize("name", ["ragged_bf16", "split_k_bf16", "split_k_fp32", "shard_bf16"])
def test_edge_parity_atomic(name):
    cfg = EDGE[name]
    out, ref = _run(cfg, moe.ATOMIC)
    print(name, compare_layer_unordered(cfg, out, ref))


@pytest.mark.parametrize("name", ["split_k_bf16", "split_k_fp32"])
def test_split_config_really_splits(name):
    """The split-K path is exercised: some expert holds more than twice the
    chunk (4 x mean rows = 512), so it is reduced over at least three chunks."""
    import numpy as np
    from oracle import route
    from synth import make_inputs
    cfg = EDGE[name]
    idx, _ = route(make_inputs(cfg, parts=("logits",))["logits"], cfg.top_k)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.num_experts)
    kc = 512
    assert counts.max() > 2 * kc, counts
