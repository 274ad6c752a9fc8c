"""Comparison of HIP-path outputs with the oracle, element by element.

Three kinds of bound, all in float64 on the host:

* whole-tensor rel-L2 ``||got - ref|| / ||ref||`` (2e-2 for bf16 storage,
  1e-5 for float32), accumulated over pieces when a tensor is compared one
  expert at a time;
* per-row rel-L2 over the last axis, worst row, against the same bound: a
  single wrong row of a [T, D] tensor shifts the whole-tensor figure by only
  about 1/sqrt(T), so the rows are bounded one by one.  A row is measured
  against max(its own norm, 1e-3 x the RMS row norm of the tensor): an
  element's rounding error scales with the sum of its terms' magnitudes, so
  a row a thousand times smaller than the typical row (its terms cancel, or
  it comes from a pre-activation that barely clears the ReLU) is held to the
  tensor's scale instead of its own.  A wrong row is off by about a typical
  row norm and still fails by orders of magnitude;
* per-slot bound for dprob.  dprob_r = sum_f G[r,f] a[r,f] with G = dy W2^T
  and a = relu(h)^2.  The path rounds h to the storage type before squaring
  it, so each term carries a relative error 2 eps with |eps| <= u (u = 2^-8
  for bf16); for independent eps the error of the sum has standard deviation
  about 2u/sqrt(3) * sqrt(sum_f (G a)^2).  The slot is held to ``z`` such
  standard deviations of its own terms, with the term scale rebuilt from the
  oracle's outputs alone: |G a| = |dh| relu(h) / (2 p).  A slot routed to a
  non-local expert must be exactly zero.

Nothing here computes the method: the oracle's values come in as ``ref``.
"""
import numpy as np

BF16_U = 2.0 ** -8


def tol_for(dtype: str) -> float:
    return 2e-2 if dtype == "bf16" else 1e-5


ROW_FLOOR = 1e-3


class Piecewise:
    """rel-L2 of a tensor compared in pieces, and the worst per-row rel-L2
    (rows measured against max(own norm, ROW_FLOOR x RMS row norm))."""

    def __init__(self, name: str, tol: float, row_tol: float = None):
        self.name = name
        self.tol = tol
        self.row_tol = tol if row_tol is None else row_tol
        self.num = 0.0
        self.den = 0.0
        self._dn, self._rn, self._lab = [], [], []
        self.pieces = 0
        self._worst = None

    def add(self, got, ref, label=None, rows=True):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if got.shape != ref.shape:
            raise AssertionError(f"{self.name}: shape {got.shape} != oracle {ref.shape}")
        d = got - ref
        self.num += float(np.sum(d * d))
        self.den += float(np.sum(ref * ref))
        self.pieces += 1
        if rows and got.ndim >= 1 and got.size:
            g2 = d.reshape(-1, got.shape[-1]) if got.ndim >= 2 else d.reshape(1, -1)
            r2 = ref.reshape(g2.shape)
            self._dn.append(np.sqrt(np.sum(g2 * g2, axis=1)))
            self._rn.append(np.sqrt(np.sum(r2 * r2, axis=1)))
            self._lab.append(label)
            self._worst = None
        return self

    def rel(self) -> float:
        if self.den == 0:
            return 0.0 if self.num == 0 else float("inf")
        return float(np.sqrt(self.num / self.den))

    def _worst_row(self):
        if self._worst is None:
            if not self._dn:
                self._worst = (0.0, None)
            else:
                dn, rn = np.concatenate(self._dn), np.concatenate(self._rn)
                floor = ROW_FLOOR * float(np.sqrt(np.mean(rn * rn)))
                den = np.maximum(rn, floor)
                with np.errstate(divide="ignore", invalid="ignore"):
                    ratio = np.where(den > 0, dn / np.where(den > 0, den, 1.0), np.where(dn > 0, np.inf, 0.0))
                i = int(np.argmax(ratio))
                sizes = np.cumsum([len(a) for a in self._dn])
                piece = int(np.searchsorted(sizes, i, side="right"))
                row = i - (int(sizes[piece - 1]) if piece else 0)
                self._worst = (float(ratio[i]), (self._lab[piece], row))
        return self._worst

    @property
    def worst(self) -> float:
        return self._worst_row()[0]

    @property
    def worst_at(self):
        return self._worst_row()[1]

    def failures(self) -> list:
        out = []
        if not self.rel() <= self.tol:
            out.append(f"{self.name}: rel-L2 {self.rel():.3e} > {self.tol}")
        if not self.worst <= self.row_tol:
            out.append(f"{self.name}: worst row rel-L2 {self.worst:.3e} > {self.row_tol} at {self.worst_at}")
        return out


def dprob_term_scale(dh_ref, h_ref, p_rows):
    """sqrt(sum_f (G a)^2) per row from the oracle's dh and h: |G a| = |dh| relu(h) / (2p)."""
    dh_ref = np.asarray(dh_ref, dtype=np.float64)
    rh = np.maximum(np.asarray(h_ref, dtype=np.float64), 0.0)
    p = np.asarray(p_rows, dtype=np.float64)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0, np.abs(dh_ref) * rh / (2.0 * p), 0.0)
    return np.sqrt(np.sum(t * t, axis=1))


def dprob_slot_z(dtype: str) -> float:
    """Standard deviations allowed per dprob slot, for either storage type
    (see the module docstring and dprob_slot_sigma)."""
    return 10.0


def dprob_slot_sigma(dtype: str, scale, k_len: int):
    """Standard deviation of a slot's error for the rounding model of ``dtype``.
    bf16: 2u/sqrt(3) of the term scale.  float32: the accumulations of h and G
    (k_len terms each) in float32, sqrt(k_len) * 2^-24 of the term scale."""
    scale = np.asarray(scale, dtype=np.float64)
    if dtype == "bf16":
        return 2.0 * BF16_U / np.sqrt(3.0) * scale
    return np.sqrt(float(k_len)) * 2.0 ** -24 * 4.0 * scale


class SlotBound:
    """Per-slot check of dprob against ``z`` standard deviations of its terms."""

    def __init__(self, dtype: str, k_len: int):
        self.dtype = dtype
        self.k_len = k_len
        self.z = dprob_slot_z(dtype)
        self.worst = 0.0
        self.worst_at = None
        self.bad_zero = 0

    def add(self, got, ref, scale, label=None):
        got = np.asarray(got, dtype=np.float64).ravel()
        ref = np.asarray(ref, dtype=np.float64).ravel()
        sig = dprob_slot_sigma(self.dtype, scale, self.k_len).ravel()
        err = np.abs(got - ref)
        # tiny absolute floor: a slot whose terms are all zero must be exact
        with np.errstate(divide="ignore", invalid="ignore"):
            zs = np.where(sig > 0, err / np.where(sig > 0, sig, 1.0), np.where(err > 0, np.inf, 0.0))
        if zs.size:
            i = int(np.argmax(zs))
            if zs[i] > self.worst or self.worst_at is None:
                self.worst = float(zs[i])
                self.worst_at = (label, i)
        return self

    def add_zero(self, got):
        got = np.asarray(got, dtype=np.float64).ravel()
        self.bad_zero += int(np.count_nonzero(got))
        return self

    def failures(self) -> list:
        out = []
        if not self.worst <= self.z:
            out.append(f"dprob: worst slot {self.worst:.2f} standard deviations > {self.z} at {self.worst_at}")
        if self.bad_zero:
            out.append(f"dprob: {self.bad_zero} non-local slots are not exactly 0")
        return out


def compare_full(dtype: str, got: dict, ref: dict, combine: bool, k: int, rows=None) -> dict:
    """Whole-layer comparison of host arrays.

    ``got`` / ``ref``: h, dh [R, F], dw1 [El, D, F], dw2 [El, F, D],
    dprob [T, k]; with ``combine`` y, dx [T, D], else o_rows, dx_rows [R, D].
    ``ref`` also holds topk_prob [T, k] and perm (the oracle's permutation).
    Returns {name: rel-L2}; raises AssertionError listing every failed bound."""
    tol = tol_for(dtype)
    perm = ref["perm"]
    R = int(perm["offsets"][-1])
    checks = {}
    for n in ("h", "dh"):
        checks[n] = Piecewise(n, tol).add(got[n][:R], ref[n], "row")
    pairs = (("y", "y"), ("dx", "dx")) if combine else (("y", "o_rows"), ("dx", "dx_rows"))
    for gn, rn in pairs:
        g = got[gn] if combine else got[gn][:R]
        checks[gn] = Piecewise(gn, tol).add(g, ref[rn], "row")
    for n in ("dw1", "dw2"):
        pw = Piecewise(n, tol)
        for e in range(ref[n].shape[0]):
            pw.add(got[n][e], ref[n][e], ("expert", e))
        checks[n] = pw
    sb = SlotBound(dtype, max(ref["dw1"].shape[1], ref["dw1"].shape[2]))
    p_rows = ref["topk_prob"].reshape(-1)[perm["row_src"]]
    scale = dprob_term_scale(ref["dh"], ref["h"], p_rows)
    gd = np.asarray(got["dprob"], dtype=np.float64).reshape(-1)
    rd = np.asarray(ref["dprob"], dtype=np.float64).reshape(-1)
    sb.add(gd[perm["row_src"]], rd[perm["row_src"]], scale, "row")
    nonlocal_ = perm["slot_row"] < 0
    sb.add_zero(gd[nonlocal_])
    checks["dprob"] = Piecewise("dprob", tol).add(gd, rd, rows=False)
    fails = [f for c in checks.values() for f in c.failures()] + sb.failures()
    errs = {n: c.rel() for n, c in checks.items()}
    errs.update({f"{n}_worst_row": c.worst for n, c in checks.items() if n != "dprob"})
    errs["dprob_worst_z"] = sb.worst
    assert not fails, f"{fails} (all: {errs})"
    return errs


def fp32_sum_bound(abs_terms, k: int):
    """Largest error of a float32 accumulation of k exactly representable
    products whose magnitudes sum to ``abs_terms`` (per element): each of
    the k - 1 additions errs by at most one float32 ulp (2^-23 relative) of
    a partial sum, whatever the rounding rule of the adder (so truncating
    matrix units are covered too), and each partial sum is at most
    abs_terms; plus half an ulp for the final value."""
    return (max(k - 1, 0) * 2.0 ** -23 + 2.0 ** -24) * np.asarray(abs_terms, dtype=np.float64)


class ElementBound:
    """Per-element check |got - ref| <= bound; tracks the worst ratio."""

    def __init__(self, name: str):
        self.name = name
        self.worst = 0.0
        self.worst_at = None

    def add(self, got, ref, bound, label=None):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        bound = np.asarray(bound, dtype=np.float64)
        err = np.abs(got - ref)
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
        if ratio.size:
            i = int(np.argmax(ratio))
            if ratio.flat[i] > self.worst or self.worst_at is None:
                self.worst = float(ratio.flat[i])
                self.worst_at = (label, np.unravel_index(i, ratio.shape))
        return self

    def failures(self) -> list:
        if self.worst <= 1.0:
            return []
        return [f"{self.name}: error {self.worst:.3g} x the bound at {self.worst_at}"]


# The scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) does not return the
# exactly rounded float32 sum of its 64 products.  On a single-wave probe
# (1024 outputs, E4M3 codes over the whole range, block scales over
# 2^-7 .. 2^2) its result differed from the exact sum by a median 1.6e-5 and
# at most 1.6e-4 of the sum of |products|, where a float32-exact sum stays
# within 64 * 2^-24 = 3.8e-6; no model of float32 adds (sequential, per
# instruction, truncating to 16..26 bits) reproduces its bits.  So the
# float32 outputs of the MXFP8 path are held to MX_TERM_BOUND of their sum
# of |terms| element by element, and to MX_REL_TOL in rel-L2, instead of
# the float32 bounds above.
MX_TERM_BOUND = 2e-4
MX_REL_TOL = 1e-4
# Where a block's products are much smaller than its scale allows (sparse
# blocks such as p relu(h)^2, or few routed rows), the error is better
# described against the scale: measured on the weight gradients, it stays
# below 2^-12.5 of the block's largest representable product
# 448^2 * 2^(sa + sb) (the instruction accumulates each block in fixed point
# relative to its scale).  mx_block_bound allows 2^-10 of that per block.
MX_BLOCK_TAU = 2.0 ** -10


def mx_block_bound(a_scales, b_scales):
    """Per-element error bound of a scaled-MFMA product from the E8M0 scale
    bytes of its operands (a_scales [M, nb], b_scales [N, nb], block b of
    row i and column j meeting in element (i, j)):
    MX_BLOCK_TAU * 448^2 * sum_b 2^(sa_ib + sb_jb)."""
    ea = np.exp2(np.asarray(a_scales, dtype=np.float64) - 127.0)
    eb = np.exp2(np.asarray(b_scales, dtype=np.float64) - 127.0)
    return MX_BLOCK_TAU * 448.0 ** 2 * (ea @ eb.T)
