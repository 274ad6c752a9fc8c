"""Routing (moe_route: top-k, softmax, stable permutation, work list) against
the oracle on logits built to tie: small integers (many equal logits per
token), +0.0 mixed with -0.0 (equal as values), every logit of a token
equal, and random normal logits for reference.  Equal logits go to the lower
expert index and -0.0 equals +0.0 (oracle.route); the integer state must be
bit-exact, the probabilities within 1e-5 (harness.compare_routing), and the
bits identical under shuffled launch orders."""
import numpy as np
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
import oracle
from harness import compare_routing

pytestmark = pytest.mark.gpu

# (tokens, experts, top_k, expert_begin, num_local, combine)
SHAPES = [(2048, 512, 22, 0, 512, 1), (1000, 1024, 8, 0, 1024, 1), (300, 8, 2, 0, 8, 1), (257, 64, 64, 0, 64, 1),
          (700, 512, 22, 128, 4, 0), (64, 3, 3, 0, 3, 1)]
KINDS = ["integers", "signed_zeros", "constant", "normal"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()


def _logits(kind, T, E, seed):
    rng = np.random.default_rng([seed, T, E])
    if kind == "integers":
        return rng.integers(-2, 3, (T, E)).astype(np.float32)
    if kind == "signed_zeros":
        # zeros of both signs, a few ones and minus ones
        z = np.where(rng.random((T, E)) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        r = rng.random((T, E))
        z[r < 0.05] = 1.0
        z[r > 0.95] = -1.0
        return z
    if kind == "constant":
        return np.full((T, E), 0.75, dtype=np.float32)
    return rng.standard_normal((T, E)).astype(np.float32)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"T{s[0]}_E{s[1]}_k{s[2]}_l{s[4]}")
def test_route_ties_exact(shape, kind):
    T, E, k, eb, el, combine = shape
    print(f"route {kind} {shape}", flush=True)
    logits = _logits(kind, T, E, 7)
    prob = moe.Problem(T, 256, 256, E, k, eb, el, "bf16", combine)
    r = moe.moe_route(prob, torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    idx, p = oracle.route(logits, k)
    compare_routing(r, dict(topk_idx=idx, topk_prob=p, perm=oracle.permute(idx, eb, el)))


def test_route_bits_identical_under_shuffles():
    T, E, k = 2048, 512, 22
    logits = torch.from_numpy(_logits("integers", T, E, 9)).cuda()
    prob = moe.Problem(T, 256, 256, E, k)
    # every element written (the full layer routes all T * k slots)
    names = ("topk_idx", "topk_prob", "counts", "offsets", "row_src", "row_tok", "row_prob", "slot_row")
    ref = None
    for seed in (0, 3, 0xBEEF, 0x9E3779B97F4A7C15):
        r = moe.moe_route(prob.with_seed(seed), logits)
        fps = [moe.moe_fingerprint(getattr(r, n).contiguous(), chunk_elems=4096)[1] for n in names]
        ref = fps if ref is None else ref
        assert fps == ref, seed
