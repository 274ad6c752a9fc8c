"""Pins of the CPU fingerprint definition: the published SplitMix64 vectors
fix the finalizer, and properties fix what the chunked hash must notice."""
import os

import numpy as np
import pytest

from oracle import fingerprint, mix64
from oracle.fingerprint import GAMMA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_vectors.txt")
M64 = (1 << 64) - 1


def _splitmix_scalar(state, n):
    out = []
    for _ in range(n):
        state = (state + GAMMA) & M64
        out.append(int(mix64(np.uint64(state))))
    return out


def test_splitmix64_published_vectors():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert rows
    for r in rows:
        seed, expect = int(r[0]), [int(v) for v in r[1:]]
        assert _splitmix_scalar(seed, len(expect)) == expect


def _py_fingerprint(values_bits, dtype_code, shape, chunk):
    """Pure-Python loop version on tiny inputs (brute force)."""
    def mix(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
        return z ^ (z >> 31)
    n = len(values_bits)
    hs = []
    for c in range((n + chunk - 1) // chunk):
        s = 0
        for i in range(c * chunk, min(n, (c + 1) * chunk)):
            s = (s + mix(values_bits[i] ^ ((i * GAMMA) & M64))) & M64
        hs.append(mix(s ^ c))
    h = GAMMA
    for w in [dtype_code, len(shape), *shape, n, chunk] + hs:
        h = mix(h ^ w)
    return hs, h


def test_matches_python_loop():
    a = np.array([[1.5, -0.0, 3.0], [0.0, 7.25, -2.0]], np.float32)
    hs, tot = fingerprint(a, "f32", chunk_elems=4)
    bits = [int(b) for b in a.reshape(-1).view(np.uint32)]
    phs, ptot = _py_fingerprint(bits, 0, (2, 3), 4)
    assert [int(x) for x in hs] == phs and tot == ptot


def test_bit_flip_changes_total_and_one_chunk():
    rng = np.random.default_rng(0)
    a = rng.standard_normal(1000).astype(np.float32)
    hs, t = fingerprint(a, "f32", 100)
    b = a.copy()
    b.view(np.uint32)[537] ^= 1
    hs2, t2 = fingerprint(b, "f32", 100)
    assert t != t2
    assert np.sum(hs != hs2) == 1 and hs[5] != hs2[5]


def test_permutation_is_seen():
    a = np.arange(64, dtype=np.int32)
    b = a.copy()
    b[[3, 9]] = b[[9, 3]]                                  # swap inside one chunk
    assert fingerprint(a, "i32", 16)[1] != fingerprint(b, "i32", 16)[1]
    c = np.concatenate([a[16:32], a[:16], a[32:]])         # swap two chunks
    ha, hc = fingerprint(a, "i32", 16)[0], fingerprint(c, "i32", 16)[0]
    assert ha[0] != hc[0] and ha[1] != hc[1] and np.all(ha[2:] == hc[2:])


def test_shape_dtype_and_zero_sign_matter():
    a = np.zeros(12, np.float32)
    assert fingerprint(a, "f32")[1] != fingerprint(a.reshape(3, 4), "f32")[1]
    assert fingerprint(a, "f32")[1] != fingerprint(a.view(np.int32), "i32")[1]
    b = a.copy()
    b[4] = -0.0
    assert fingerprint(a, "f32")[1] != fingerprint(b, "f32")[1]
    assert fingerprint(a, "f32", 4)[1] != fingerprint(a, "f32", 6)[1]


def test_empty_and_bf16():
    hs, t = fingerprint(np.zeros((0, 5), np.uint16), "bf16")
    assert hs.size == 0 and isinstance(t, int)
    assert t != fingerprint(np.zeros((5, 0), np.uint16), "bf16")[1]
    x = np.array([0x3F80, 0x3F81], np.uint16)
    assert fingerprint(x, "bf16")[1] != fingerprint(x[::-1].copy(), "bf16")[1]


def test_bad_chunk():
    with pytest.raises(ValueError):
        fingerprint(np.zeros(3, np.float32), "f32", 0)
