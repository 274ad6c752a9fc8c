"""Chunk-wise tensor fingerprint, CPU definition (TEST INFRASTRUCTURE ONLY).

The French article's section "Méthodologie de débogage du non-déterminisme"
describes GPU fingerprints that record shape, dtype and element count, and
chunk-wise fingerprints for order-sensitive data such as routing maps and
MoE dispatch outputs.  It names no hash.  The definition used here (the same
one the GPU kernel implements from its own source) is:

  mix64(z)  = SplitMix64 output finalizer (Steele, Lea, Flood, OOPSLA 2014):
              z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
              z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31   (mod 2^64)
  GAMMA     = 0x9E3779B97F4A7C15
  bits_i    = raw bits of element i (row-major), zero-extended to 64 bits
  v_i       = mix64(bits_i XOR (i * GAMMA mod 2^64))
  H_c       = mix64((sum of v_i over chunk c, mod 2^64) XOR c),  chunks of C
              consecutive elements (the last one may be short)
  total     = h folded over the words [dtype code, ndim, shape..., numel, C,
              H_0, ..., H_{m-1}] with h0 = GAMMA and h <- mix64(h XOR word)

The wrapping sum makes the chunk hash independent of the order the GPU adds
the v_i in, while the index mixed into v_i keeps it sensitive to position.
dtype codes: f32 0, bf16 1, i32 2, u8 3, i64 4, f64 5.
"""
import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
DTYPE_CODE = {"f32": 0, "bf16": 1, "i32": 2, "u8": 3, "i64": 4, "f64": 5}
_WIDTH_VIEW = {"f32": np.uint32, "bf16": np.uint16, "i32": np.uint32, "u8": np.uint8,
               "i64": np.uint64, "f64": np.uint64}


def mix64(z):
    """SplitMix64 finalizer on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def element_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Raw element bits zero-extended to uint64 (bf16 given as uint16 bits)."""
    a = np.ascontiguousarray(a)
    return a.reshape(-1).view(_WIDTH_VIEW[dtype]).astype(np.uint64)


def fingerprint(a: np.ndarray, dtype: str, chunk_elems: int = 65536, shape=None):
    """Return (chunk_hashes uint64[m], total python int) for array ``a``.

    ``shape`` defaults to ``a.shape``; ``dtype`` names the element type
    (bf16 arrays are passed as their uint16 bit patterns)."""
    if chunk_elems <= 0:
        raise ValueError("chunk_elems must be positive")
    shape = tuple(a.shape) if shape is None else tuple(shape)
    bits = element_bits(a, dtype)
    n = bits.size
    idx = np.arange(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        v = mix64(bits ^ (idx * np.uint64(GAMMA)))
    m = (n + chunk_elems - 1) // chunk_elems
    hashes = np.zeros(m, dtype=np.uint64)
    for c in range(m):
        s = np.sum(v[c * chunk_elems:(c + 1) * chunk_elems], dtype=np.uint64)  # wraps mod 2^64
        hashes[c] = mix64(np.uint64(s) ^ np.uint64(c))
    words = [DTYPE_CODE[dtype], len(shape), *shape, n, chunk_elems] + [int(x) for x in hashes]
    h = np.uint64(GAMMA)
    for w in words:
        h = mix64(h ^ np.uint64(w & 0xFFFFFFFFFFFFFFFF))
    return hashes, int(h)
