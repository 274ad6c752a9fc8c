"""GPU fingerprint == CPU fingerprint definition, bit for bit."""
import numpy as np
import pytest
import torch

import bitwise_deterministic_moe_amd as moe
from oracle import fingerprint

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "i32": torch.int32, "u8": torch.uint8, "i64": torch.int64, "f64": torch.float64}


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32", "u8", "i64", "f64"])
@pytest.mark.parametrize("shape,chunk", [((1000,), 64), ((37, 129), 1000), ((4, 65536 + 3), 65536), ((0, 3), 7),
                                         ((), 5), ((200, 1001), 1000), ((130, 64), 64)])
def test_matches_cpu(dtype, shape, chunk):
    rng = np.random.default_rng(hash((dtype, shape, chunk)) & 0xFFFF)
    n = int(np.prod(shape)) if shape else 1
    raw = rng.integers(0, 2**63 - 1, size=n, dtype=np.int64).view(np.uint8)
    width = {"f32": 4, "bf16": 2, "i32": 4, "u8": 1, "i64": 8, "f64": 8}[dtype]
    host = raw[: n * width].copy()
    np_view = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32, "u8": np.uint8, "i64": np.int64,
               "f64": np.float64}[dtype]
    a = host.view(np_view).reshape(shape)
    ref_h, ref_t = fingerprint(a, dtype, chunk)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16).copy()).cuda().view(torch.bfloat16)
    else:
        t = torch.from_numpy(a.copy()).cuda()
    h, tot = moe.moe_fingerprint(t, dtype=dtype, chunk_elems=chunk, shape=shape)
    assert tot == ref_t
    assert [x & 0xFFFFFFFFFFFFFFFF for x in h.cpu().tolist()] == [int(v) for v in ref_h]


@pytest.mark.parametrize("dtype", ["bf16", "f32", "u8"])
def test_matches_cpu_from_an_unaligned_start(dtype):
    """A contiguous view that starts one element into its allocation (not on
    a 16-byte boundary) takes the element-wise path and gives the same bits."""
    rng = np.random.default_rng(7)
    np_view = {"f32": np.float32, "bf16": np.uint16, "u8": np.uint8}[dtype]
    width = {"f32": 4, "bf16": 2, "u8": 1}[dtype]
    raw = rng.integers(0, 256, size=5001 * width, dtype=np.uint8)
    a = raw.view(np_view)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16).copy()).cuda().view(torch.bfloat16)[1:]
    else:
        t = torch.from_numpy(a.copy()).cuda()[1:]
    assert t.data_ptr() % 16 != 0
    ref_h, ref_t = fingerprint(a[1:], dtype, 256)
    h, tot = moe.moe_fingerprint(t, dtype=dtype, chunk_elems=256)
    assert tot == ref_t
    assert [x & 0xFFFFFFFFFFFFFFFF for x in h.cpu().tolist()] == [int(v) for v in ref_h]
