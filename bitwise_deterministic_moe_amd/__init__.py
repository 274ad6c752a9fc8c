"""Python binding of libmoedet: the bitwise-deterministic MoE expert layer
for MI355X (gfx950).

Argument marshalling only.  Every step of the layer runs in the HIP kernels
of ``libmoedet.so``; PyTorch supplies device memory and the current stream.
The functions carry the names of the C ABI (include/moedet.h).  There is no
fallback: a missing library raises ``MoeLibraryMissing``.
"""
import ctypes
import os
from dataclasses import dataclass, replace
from typing import Optional

import torch

__all__ = [
    "DETERMINISTIC", "ATOMIC", "Problem", "Routing", "MoeError", "MoeLibraryMissing",
    "load_library", "library_path", "moe_workspace_size", "moe_rows_cap", "moe_stage_names",
    "moe_fwd", "moe_bwd_dgrad_dprob", "moe_bwd_wgrad", "moe_fingerprint", "moe_sched_elems", "moe_mfma_rate",
    "moe_router_bwd", "moe_router_fwd", "moe_sgd_step", "moe_mx_quantize", "moe_mx_dgrad_fc1",
    "moe_bwd_dgrad_dprob_noalloc", "moe_mx_quantize_t", "moe_mx_fwd_fc1", "moe_mx_fwd_fc2", "EXPORTED_SYMBOLS",
    "moe_mx_wgrad_rows", "moe_mx_quantize_wgrad", "moe_mx_wgrad", "MXW_TOKEN", "MXW_ROW", "MXW_ACT_P",
    "moe_route",
]

DETERMINISTIC = 0
ATOMIC = 1
DTYPE_CODE = {"f32": 0, "bf16": 1, "i32": 2, "u8": 3, "i64": 4, "f64": 5}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_TORCH_TO_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.int32: 2, torch.uint8: 3,
                  torch.int64: 4, torch.float64: 5}
EXPORTED_SYMBOLS = ("moe_abi_version", "moe_status_string", "moe_rows_cap", "moe_sched_elems",
                    "moe_workspace_size", "moe_stage_names", "moe_fwd", "moe_bwd_dgrad_dprob", "moe_bwd_wgrad",
                    "moe_fingerprint", "moe_mfma_rate", "moe_router_bwd", "moe_router_fwd", "moe_sgd_step",
                    "moe_mx_quantize", "moe_mx_dgrad_fc1", "moe_mx_dgrad_fc2",
                    "moe_nvfp4_quantize", "moe_bwd_dgrad_dprob_noalloc", "moe_mx_quantize_t", "moe_mx_fwd_fc1",
                    "moe_mx_fwd_fc2", "moe_mx_wgrad_rows", "moe_mx_quantize_wgrad", "moe_mx_wgrad", "moe_route",
                    "moe_source_hash")
# rows read by moe_mx_quantize_wgrad (moe_mxw_src)
MXW_TOKEN, MXW_ROW, MXW_ACT_P = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class MoeError(RuntimeError):
    pass


class MoeLibraryMissing(MoeError):
    pass


class MoeLibraryStale(MoeError):
    """The in-tree libmoedet.so was built from other sources than the tree's."""


class _CProblem(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("expert_begin", ctypes.c_int32), ("num_local", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("combine", ctypes.c_int32),
                ("debug_shuffle_seed", ctypes.c_uint64), ("stage_events", ctypes.c_void_p),
                ("n_stage_events", ctypes.c_int32)]


class _CRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_idx", "topk_prob", "counts", "offsets",
                                                "row_src", "row_tok", "row_prob", "slot_row", "sched")]


def library_path() -> str:
    return os.environ.get("MOEDET_LIB", os.path.join(_HERE, "libmoedet.so"))


def load_library() -> ctypes.CDLL:
    """Load libmoedet.so (build it with ``python -m bitwise_deterministic_moe_amd.build``)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise MoeLibraryMissing(f"{path} not found; build it with python -m bitwise_deterministic_moe_amd.build")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(_CProblem)
    R = ctypes.POINTER(_CRouting)
    lib.moe_abi_version.restype = ctypes.c_int
    lib.moe_source_hash.restype = ctypes.c_char_p
    lib.moe_source_hash.argtypes = []
    if "MOEDET_LIB" not in os.environ and os.path.isdir(os.path.join(_HERE, "csrc")):
        # the in-tree library must have been built from the tree's sources
        from .build import source_hash
        built, tree = lib.moe_source_hash().decode(), source_hash()
        if built != tree:
            raise MoeLibraryStale(f"{path} was built from sources {built}, the tree holds {tree}; rebuild it with "
                                  "python -m bitwise_deterministic_moe_amd.build")
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_rows_cap.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    lib.moe_sched_elems.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    lib.moe_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.moe_stage_names.restype = ctypes.c_char_p
    lib.moe_stage_names.argtypes = [P, ctypes.c_int, ctypes.c_int]
    lib.moe_fwd.argtypes = [P, vp, vp, vp, vp, R, vp, vp, vp, sz, ctypes.c_int, vp]
    lib.moe_bwd_dgrad_dprob.argtypes = [P, R, vp, vp, vp, vp, vp, vp, vp, vp, sz, ctypes.c_int, vp]
    lib.moe_bwd_wgrad.argtypes = [P, R, vp, vp, vp, vp, vp, vp, vp, sz, ctypes.c_int, vp]
    lib.moe_bwd_dgrad_dprob_noalloc.argtypes = [P, R, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    lib.moe_fingerprint.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                    vp, vp, vp]
    lib.moe_mfma_rate.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_float, vp, vp]
    lib.moe_router_bwd.argtypes = [P, R, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    lib.moe_router_fwd.argtypes = [P, vp, vp, vp, vp]
    lib.moe_sgd_step.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_float, vp, ctypes.c_int, vp]
    lib.moe_mx_quantize.argtypes = [vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, vp, vp, ctypes.c_uint64, vp]
    lib.moe_mx_dgrad_fc1.argtypes = [P, R, vp, vp, vp, vp, vp, vp]
    lib.moe_nvfp4_quantize.argtypes = [vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, vp, vp, vp, ctypes.c_uint64,
                                       vp]
    lib.moe_mx_dgrad_fc2.argtypes = [P, R, vp, vp, vp, vp, vp, vp, vp, vp, sz, ctypes.c_int, vp]
    lib.moe_mx_quantize_t.argtypes = [vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp, vp,
                                      ctypes.c_uint64, vp]
    lib.moe_mx_fwd_fc1.argtypes = [P, R, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_mx_fwd_fc2.argtypes = [P, R, vp, vp, vp, vp, vp, vp, sz, ctypes.c_int, vp]
    lib.moe_mx_wgrad_rows.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    lib.moe_route.argtypes = [P, vp, R, vp, sz, ctypes.c_int, vp]
    lib.moe_mx_quantize_wgrad.argtypes = [P, R, vp, ctypes.c_int, vp, vp, vp]
    lib.moe_mx_wgrad.argtypes = [P, R, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    for f in ("moe_route", "moe_mx_wgrad_rows", "moe_mx_quantize_wgrad", "moe_mx_wgrad", "moe_rows_cap",
              "moe_sched_elems", "moe_workspace_size", "moe_fwd", "moe_bwd_dgrad_dprob",
              "moe_bwd_dgrad_dprob_noalloc", "moe_mx_quantize_t", "moe_mx_fwd_fc1", "moe_mx_fwd_fc2",
              "moe_bwd_wgrad", "moe_fingerprint", "moe_mfma_rate", "moe_router_bwd", "moe_router_fwd",
              "moe_sgd_step", "moe_mx_quantize", "moe_mx_dgrad_fc1", "moe_mx_dgrad_fc2", "moe_nvfp4_quantize"):
        getattr(lib, f).restype = ctypes.c_int
    _LIB = lib
    return lib


def moe_source_hash() -> str:
    """Hash of the sources the loaded library was built from."""
    return load_library().moe_source_hash().decode()


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().moe_status_string(status).decode()
        raise MoeError(f"{what}: status {status} ({msg})")


@dataclass(frozen=True)
class Problem:
    """Mirror of ``moe_problem``."""
    tokens: int
    d_model: int
    d_ffn: int
    num_experts: int
    top_k: int
    expert_begin: int = 0
    num_local: Optional[int] = None
    dtype: str = "bf16"
    combine: int = 1
    shuffle_seed: int = 0

    @property
    def local(self) -> int:
        return self.num_experts if self.num_local is None else self.num_local

    @property
    def rows_cap(self) -> int:
        return self.tokens * min(self.top_k, self.local)

    def with_seed(self, seed: int) -> "Problem":
        return replace(self, shuffle_seed=seed)

    def c(self, events=None) -> _CProblem:
        p = _CProblem(self.tokens, self.d_model, self.d_ffn, self.num_experts, self.top_k,
                      self.expert_begin, self.local, DTYPE_CODE[self.dtype], self.combine,
                      self.shuffle_seed & 0xFFFFFFFFFFFFFFFF, None, 0)
        if events:
            arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
            p.stage_events = ctypes.cast(arr, ctypes.c_void_p)
            p.n_stage_events = len(events)
            p._keep = arr
        return p

    @classmethod
    def from_config(cls, cfg, shuffle_seed: int = 0) -> "Problem":
        return cls(cfg.tokens, cfg.d_model, cfg.d_ffn, cfg.num_experts, cfg.top_k, cfg.expert_begin,
                   cfg.num_local, cfg.dtype, cfg.combine, shuffle_seed)


@dataclass
class Routing:
    """Device routing state (mirror of ``moe_routing``)."""
    topk_idx: torch.Tensor
    topk_prob: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    row_src: torch.Tensor
    row_tok: torch.Tensor
    row_prob: torch.Tensor
    slot_row: torch.Tensor
    sched: torch.Tensor

    @classmethod
    def empty(cls, prob: Problem, device="cuda") -> "Routing":
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        T, k, el, rc = prob.tokens, prob.top_k, prob.local, prob.rows_cap
        return cls(torch.empty((T, k), **i32), torch.empty((T, k), **f32), torch.empty(el, **i32),
                   torch.empty(el + 1, **i32), torch.empty(rc, **i32), torch.empty(rc, **i32),
                   torch.empty(rc, **f32), torch.empty(T * k, **i32), torch.empty(moe_sched_elems(prob), **i32))

    def c(self) -> _CRouting:
        return _CRouting(*[_ptr(getattr(self, n)) for n, _ in _CRouting._fields_])

    @property
    def rows(self) -> int:
        """R (synchronises: reads offsets[-1] to the host)."""
        return int(self.offsets[-1].item())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return t.data_ptr() or None


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ws(nbytes: int, ws: Optional[torch.Tensor], device) -> torch.Tensor:
    if ws is not None:
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def moe_rows_cap(prob: Problem) -> int:
    v = ctypes.c_int64()
    _check(load_library().moe_rows_cap(ctypes.byref(prob.c()), ctypes.byref(v)), "moe_rows_cap")
    return v.value


def moe_sched_elems(prob: Problem) -> int:
    """int32 elements of Routing.sched."""
    v = ctypes.c_int64()
    _check(load_library().moe_sched_elems(ctypes.byref(prob.c()), ctypes.byref(v)), "moe_sched_elems")
    return v.value


def moe_workspace_size(prob: Problem, mode: int = DETERMINISTIC):
    """Bytes of workspace for (moe_fwd, moe_bwd_dgrad_dprob, moe_bwd_wgrad)."""
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().moe_workspace_size(ctypes.byref(prob.c()), mode, ctypes.byref(a), ctypes.byref(b),
                                             ctypes.byref(c)), "moe_workspace_size")
    return a.value, b.value, c.value


def moe_stage_names(prob: Problem, mode: int, call: int):
    s = load_library().moe_stage_names(ctypes.byref(prob.c()), mode, call)
    return s.decode().split(",") if s else None


def moe_fwd(prob: Problem, logits, x, w1, w2, mode: int = DETERMINISTIC, routing: Routing = None,
            h=None, y=None, ws=None, events=None):
    """Routing + expert MLP + combine.  Returns (routing, h, y_or_rows)."""
    lib = load_library()
    dev = x.device
    dt = TORCH_DTYPE[prob.dtype]
    routing = routing or Routing.empty(prob, dev)
    if h is None:
        h = torch.empty((prob.rows_cap, prob.d_ffn), dtype=dt, device=dev)
    if y is None:
        y = torch.empty((prob.tokens if prob.combine else prob.rows_cap, prob.d_model), dtype=dt, device=dev)
    need = moe_workspace_size(prob, mode)[0]
    ws = _ws(need, ws, dev)
    T, E, D, F, el, rc = prob.tokens, prob.num_experts, prob.d_model, prob.d_ffn, prob.local, prob.rows_cap
    _need(logits, T * E, torch.float32, "moe_fwd logits")
    _need(x, T * D, dt, "moe_fwd x")
    _need(w1, el * D * F, dt, "moe_fwd w1")
    _need(w2, el * F * D, dt, "moe_fwd w2")
    _need(h, rc * F, dt, "moe_fwd h")
    _need(y, (T if prob.combine else rc) * D, dt, "moe_fwd y")
    cp, cr = prob.c(events), routing.c()
    _check(lib.moe_fwd(ctypes.byref(cp), _ptr(logits), _ptr(x), _ptr(w1), _ptr(w2), ctypes.byref(cr), _ptr(h),
                       _ptr(y), _ptr(ws), ws.numel(), mode, _stream()), "moe_fwd")
    return routing, h, y


def moe_route(prob: Problem, logits, mode: int = DETERMINISTIC, routing: Routing = None, ws=None, events=None):
    """The routing stage of moe_fwd alone (top-k, permutation, work list).
    Returns the routing."""
    lib = load_library()
    dev = logits.device
    routing = routing or Routing.empty(prob, dev)
    ws = _ws(moe_workspace_size(prob, mode)[0], ws, dev)
    _need(logits, prob.tokens * prob.num_experts, torch.float32, "moe_route logits")
    cp, cr = prob.c(events), routing.c()
    _check(lib.moe_route(ctypes.byref(cp), _ptr(logits), ctypes.byref(cr), _ptr(ws), ws.numel(), mode, _stream()),
           "moe_route")
    return routing


def moe_bwd_dgrad_dprob(prob: Problem, routing: Routing, dy, w1, w2, h, mode: int = DETERMINISTIC,
                        dx=None, dprob=None, dh=None, ws=None, events=None):
    """fc2 dgrad with dprob + fc1 dgrad + dx combine.
    Returns (dx_or_rows, dprob, dh)."""
    lib = load_library()
    dev = h.device
    dt = TORCH_DTYPE[prob.dtype]
    if dx is None:
        dx = torch.empty((prob.tokens if prob.combine else prob.rows_cap, prob.d_model), dtype=dt, device=dev)
    if dprob is None:
        dprob = torch.empty((prob.tokens, prob.top_k), dtype=torch.float32, device=dev)
    if dh is None:
        dh = torch.empty((prob.rows_cap, prob.d_ffn), dtype=dt, device=dev)
    need = moe_workspace_size(prob, mode)[1]
    ws = _ws(need, ws, dev)
    T, k, D, F, el, rc = prob.tokens, prob.top_k, prob.d_model, prob.d_ffn, prob.local, prob.rows_cap
    _need(dy, T * D, dt, "moe_bwd_dgrad_dprob dy")
    _need(w1, el * D * F, dt, "moe_bwd_dgrad_dprob w1")
    _need(w2, el * F * D, dt, "moe_bwd_dgrad_dprob w2")
    _need(h, rc * F, dt, "moe_bwd_dgrad_dprob h")
    _need(dx, (T if prob.combine else rc) * D, dt, "moe_bwd_dgrad_dprob dx")
    _need(dprob, T * k, torch.float32, "moe_bwd_dgrad_dprob dprob")
    _need(dh, rc * F, dt, "moe_bwd_dgrad_dprob dh")
    cp, cr = prob.c(events), routing.c()
    _check(lib.moe_bwd_dgrad_dprob(ctypes.byref(cp), ctypes.byref(cr), _ptr(dy), _ptr(w1), _ptr(w2), _ptr(h),
                                   _ptr(dx), _ptr(dprob), _ptr(dh), _ptr(ws), ws.numel(), mode, _stream()),
           "moe_bwd_dgrad_dprob")
    return dx, dprob, dh


NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES of moedet.h


def moe_bwd_dgrad_dprob_noalloc(prob: Problem, routing: Routing, dy, w1, w2, h, dx, dprob, dh,
                                mode: int = DETERMINISTIC, events=None):
    """moe_bwd_dgrad_dprob with the library's static per-GPU workspace: the
    caller passes inputs and preallocated outputs, nothing is allocated.
    Returns (dx_or_rows, dprob, dh)."""
    lib = load_library()
    dt = TORCH_DTYPE[prob.dtype]
    T, k, D, F, el, rc = prob.tokens, prob.top_k, prob.d_model, prob.d_ffn, prob.local, prob.rows_cap
    _need(dy, T * D, dt, "moe_bwd_dgrad_dprob_noalloc dy")
    _need(w1, el * D * F, dt, "moe_bwd_dgrad_dprob_noalloc w1")
    _need(w2, el * F * D, dt, "moe_bwd_dgrad_dprob_noalloc w2")
    _need(h, rc * F, dt, "moe_bwd_dgrad_dprob_noalloc h")
    _need(dx, (T if prob.combine else rc) * D, dt, "moe_bwd_dgrad_dprob_noalloc dx")
    _need(dprob, T * k, torch.float32, "moe_bwd_dgrad_dprob_noalloc dprob")
    _need(dh, rc * F, dt, "moe_bwd_dgrad_dprob_noalloc dh")
    cp, cr = prob.c(events), routing.c()
    _check(lib.moe_bwd_dgrad_dprob_noalloc(ctypes.byref(cp), ctypes.byref(cr), _ptr(dy), _ptr(w1), _ptr(w2), _ptr(h),
                                           _ptr(dx), _ptr(dprob), _ptr(dh), mode, _stream()),
           "moe_bwd_dgrad_dprob_noalloc")
    return dx, dprob, dh


def moe_bwd_wgrad(prob: Problem, routing: Routing, x, dy, h, dh, mode: int = DETERMINISTIC, dw1=None,
                  dw2=None, ws=None, events=None):
    """Expert weight gradients (float32) from the layer input x, the upstream
    gradient dy, the saved h and dh.  Returns (dw1, dw2)."""
    lib = load_library()
    dev = dh.device
    el, D, F = prob.local, prob.d_model, prob.d_ffn
    if dw1 is None:
        dw1 = torch.empty((el, D, F), dtype=torch.float32, device=dev)
    if dw2 is None:
        dw2 = torch.empty((el, F, D), dtype=torch.float32, device=dev)
    need = moe_workspace_size(prob, mode)[2]
    ws = _ws(need, ws, dev)
    dt = TORCH_DTYPE[prob.dtype]
    T, rc = prob.tokens, prob.rows_cap
    _need(x, T * D, dt, "moe_bwd_wgrad x")
    _need(dy, T * D, dt, "moe_bwd_wgrad dy")
    _need(h, rc * F, dt, "moe_bwd_wgrad h")
    _need(dh, rc * F, dt, "moe_bwd_wgrad dh")
    _need(dw1, el * D * F, torch.float32, "moe_bwd_wgrad dw1")
    _need(dw2, el * F * D, torch.float32, "moe_bwd_wgrad dw2")
    cp, cr = prob.c(events), routing.c()
    _check(lib.moe_bwd_wgrad(ctypes.byref(cp), ctypes.byref(cr), _ptr(x), _ptr(dy), _ptr(h), _ptr(dh), _ptr(dw1),
                             _ptr(dw2), _ptr(ws), ws.numel(), mode, _stream()), "moe_bwd_wgrad")
    return dw1, dw2


def moe_router_bwd(prob: Problem, routing: Routing, dprob, x, w_router, mode: int = DETERMINISTIC, dlogits=None,
                   dw_router=None, dx_router=None):
    """Router backward (full layer only).  Returns (dlogits float32 [T,E],
    dw_router float32 [E,D], dx_router [T,D] in the storage dtype)."""
    lib = load_library()
    dev = w_router.device
    T, E, D = prob.tokens, prob.num_experts, prob.d_model
    if dlogits is None:
        dlogits = torch.empty((T, E), dtype=torch.float32, device=dev)
    if dw_router is None:
        dw_router = torch.empty((E, D), dtype=torch.float32, device=dev)
    if dx_router is None:
        dx_router = torch.empty((T, D), dtype=TORCH_DTYPE[prob.dtype], device=dev)
    dt = TORCH_DTYPE[prob.dtype]
    _need(dprob, T * prob.top_k, torch.float32, "moe_router_bwd dprob")
    _need(x, T * D, dt, "moe_router_bwd x")
    _need(w_router, E * D, dt, "moe_router_bwd w_router")
    _need(dlogits, T * E, torch.float32, "moe_router_bwd dlogits")
    _need(dw_router, E * D, torch.float32, "moe_router_bwd dw_router")
    _need(dx_router, T * D, dt, "moe_router_bwd dx_router")
    cp, cr = prob.c(), routing.c()
    _check(lib.moe_router_bwd(ctypes.byref(cp), ctypes.byref(cr), _ptr(dprob), _ptr(x), _ptr(w_router), _ptr(dlogits),
                              _ptr(dw_router), _ptr(dx_router), mode, _stream()), "moe_router_bwd")
    return dlogits, dw_router, dx_router


def moe_router_fwd(prob: Problem, x, w_router, logits=None):
    """Router logits float32 [T,E] = x w_router^T (d ascending, fp32 FMA)."""
    lib = load_library()
    if logits is None:
        logits = torch.empty((prob.tokens, prob.num_experts), dtype=torch.float32, device=w_router.device)
    dt = TORCH_DTYPE[prob.dtype]
    _need(x, prob.tokens * prob.d_model, dt, "moe_router_fwd x")
    _need(w_router, prob.num_experts * prob.d_model, dt, "moe_router_fwd w_router")
    _need(logits, prob.tokens * prob.num_experts, torch.float32, "moe_router_fwd logits")
    cp = prob.c()
    _check(lib.moe_router_fwd(ctypes.byref(cp), _ptr(x), _ptr(w_router), _ptr(logits), _stream()), "moe_router_fwd")
    return logits


def moe_sgd_step(master: torch.Tensor, grad: torch.Tensor, lr: float, runtime: torch.Tensor):
    """master -= lr * grad (float32, in place); runtime = master rounded to
    runtime's dtype.  All three tensors contiguous with the same element count."""
    lib = load_library()
    if not (master.is_contiguous() and grad.is_contiguous() and runtime.is_contiguous()):
        raise MoeError("moe_sgd_step needs contiguous tensors")
    n = master.numel()
    if grad.numel() != n or runtime.numel() != n or master.dtype != torch.float32 or grad.dtype != torch.float32:
        raise MoeError("moe_sgd_step: master and grad float32 with runtime's element count")
    code = _TORCH_TO_CODE[runtime.dtype]
    _check(lib.moe_sgd_step(_ptr(master), _ptr(grad), n, lr, _ptr(runtime), code, _stream()), "moe_sgd_step")
    return master, runtime


def _need(t: torch.Tensor, numel: int, dtype, what: str):
    """Argument check before a raw pointer crosses the boundary: the kernels
    behind it take sizes from the problem, not from the tensor."""
    if t.dtype != dtype or not t.is_contiguous() or t.numel() != numel:
        raise MoeError(f"{what}: need a contiguous {dtype} tensor of {numel} elements, "
                       f"got {t.dtype} {tuple(t.shape)} (contiguous={t.is_contiguous()})")


def moe_mx_quantize(t: torch.Tensor, codes=None, scales=None, shuffle_seed: int = 0):
    """MXFP8 (E4M3 codes, E8M0 scales per 32 elements of the last dimension)
    of a contiguous float32 or bf16 tensor.  Returns (codes uint8 with t's
    shape, scales uint8 [..., cols/32])."""
    lib = load_library()
    if not t.is_contiguous() or t.dim() < 1:
        raise MoeError("moe_mx_quantize needs a contiguous tensor")
    cols = t.shape[-1]
    rows = t.numel() // cols if cols else 0
    if codes is None:
        codes = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
    if scales is None:
        scales = torch.empty(tuple(t.shape[:-1]) + (cols // 32,), dtype=torch.uint8, device=t.device)
    _need(codes, t.numel(), torch.uint8, "moe_mx_quantize codes")
    _need(scales, rows * (cols // 32), torch.uint8, "moe_mx_quantize scales")
    _check(lib.moe_mx_quantize(_ptr(t), _TORCH_TO_CODE[t.dtype], rows, cols, _ptr(codes), _ptr(scales),
                               shuffle_seed & 0xFFFFFFFFFFFFFFFF, _stream()), "moe_mx_quantize")
    return codes, scales


def moe_nvfp4_quantize(t: torch.Tensor, shuffle_seed: int = 0):
    """NVFP4 of a contiguous float32 or bf16 tensor (blocks of 16 along the
    last dimension).  Returns (packed codes uint8 [..., cols/2], block scales
    uint8 [..., cols/16], tensor scale float32 [1])."""
    lib = load_library()
    if not t.is_contiguous() or t.dim() < 1:
        raise MoeError("moe_nvfp4_quantize needs a contiguous tensor")
    cols = t.shape[-1]
    rows = t.numel() // cols if cols else 0
    codes = torch.empty(tuple(t.shape[:-1]) + (cols // 2,), dtype=torch.uint8, device=t.device)
    scales = torch.empty(tuple(t.shape[:-1]) + (cols // 16,), dtype=torch.uint8, device=t.device)
    g = torch.empty(1, dtype=torch.float32, device=t.device)
    _check(lib.moe_nvfp4_quantize(_ptr(t), _TORCH_TO_CODE[t.dtype], rows, cols, _ptr(codes), _ptr(scales), _ptr(g),
                                  shuffle_seed & 0xFFFFFFFFFFFFFFFF, _stream()), "moe_nvfp4_quantize")
    return codes, scales, g


def moe_mx_dgrad_fc1(prob: Problem, routing: Routing, dh_mx, w1_mx, dx_rows=None):
    """MXFP8 fc1 data gradient: dx_rows [rows_cap, D] bf16 from (codes, scales)
    of dh [rows_cap, F] and of W1 [num_local, D, F] (moe_mx_quantize outputs)."""
    lib = load_library()
    (dc, ds), (wc, wsc) = dh_mx, w1_mx
    if dx_rows is None:
        dx_rows = torch.empty((prob.rows_cap, prob.d_model), dtype=torch.bfloat16, device=dc.device)
    rc, D, F, el = prob.rows_cap, prob.d_model, prob.d_ffn, prob.local
    _need(dc, rc * F, torch.uint8, "moe_mx_dgrad_fc1 dh codes")
    _need(ds, rc * (F // 32), torch.uint8, "moe_mx_dgrad_fc1 dh scales")
    _need(wc, el * D * F, torch.uint8, "moe_mx_dgrad_fc1 W1 codes")
    _need(wsc, el * D * (F // 32), torch.uint8, "moe_mx_dgrad_fc1 W1 scales")
    _need(dx_rows, rc * D, torch.bfloat16, "moe_mx_dgrad_fc1 dx_rows")
    cp, cr = prob.c(), routing.c()
    _check(lib.moe_mx_dgrad_fc1(ctypes.byref(cp), ctypes.byref(cr), _ptr(dc), _ptr(ds), _ptr(wc), _ptr(wsc),
                                _ptr(dx_rows), _stream()), "moe_mx_dgrad_fc1")
    return dx_rows


def moe_mx_dgrad_fc2(prob: Problem, routing: Routing, dy_mx, w2_mx, h, mode: int = DETERMINISTIC, dprob=None,
                     dh=None, ws=None):
    """MXFP8 fc2 data gradient with the fused dprob / dh epilogue, from
    (codes, scales) of dy [T, D] and of W2 [num_local, F, D] (moe_mx_quantize
    outputs) and the saved h.  Returns (dprob float32 [T, k], dh bf16
    [rows_cap, F]).  The workspace is the dgrad one (moe_workspace_size)."""
    lib = load_library()
    (dc, ds), (wc, wsc) = dy_mx, w2_mx
    dev = h.device
    if dprob is None:
        dprob = torch.empty((prob.tokens, prob.top_k), dtype=torch.float32, device=dev)
    if dh is None:
        dh = torch.empty((prob.rows_cap, prob.d_ffn), dtype=torch.bfloat16, device=dev)
    ws = _ws(moe_workspace_size(prob, mode)[1], ws, dev)
    T, k, rc, D, F, el = prob.tokens, prob.top_k, prob.rows_cap, prob.d_model, prob.d_ffn, prob.local
    _need(dc, T * D, torch.uint8, "moe_mx_dgrad_fc2 dy codes")
    _need(ds, T * (D // 32), torch.uint8, "moe_mx_dgrad_fc2 dy scales")
    _need(wc, el * F * D, torch.uint8, "moe_mx_dgrad_fc2 W2 codes")
    _need(wsc, el * F * (D // 32), torch.uint8, "moe_mx_dgrad_fc2 W2 scales")
    _need(h, rc * F, torch.bfloat16, "moe_mx_dgrad_fc2 h")
    _need(dprob, T * k, torch.float32, "moe_mx_dgrad_fc2 dprob")
    _need(dh, rc * F, torch.bfloat16, "moe_mx_dgrad_fc2 dh")
    cp, cr = prob.c(), routing.c()
    _check(lib.moe_mx_dgrad_fc2(ctypes.byref(cp), ctypes.byref(cr), _ptr(dc), _ptr(ds), _ptr(wc), _ptr(wsc), _ptr(h),
                                _ptr(dprob), _ptr(dh), _ptr(ws), ws.numel(), mode, _stream()),
           "moe_mx_dgrad_fc2")
    return dprob, dh


def moe_mx_quantize_t(t: torch.Tensor, codes=None, scales=None, shuffle_seed: int = 0):
    """MXFP8 of the transpose of each [rows, cols] matrix of a contiguous
    [groups, rows, cols] (or [rows, cols]) float32 / bf16 tensor: blocks of 32
    consecutive rows of a column.  Returns (codes uint8 [groups, cols, rows],
    scales uint8 [groups, cols, rows/32]) (without the group axis for 2-D input)."""
    lib = load_library()
    if not t.is_contiguous() or t.dim() not in (2, 3):
        raise MoeError("moe_mx_quantize_t needs a contiguous [groups,] rows, cols tensor")
    g, rows, cols = (1,) + tuple(t.shape) if t.dim() == 2 else tuple(t.shape)
    shp = (cols, rows) if t.dim() == 2 else (g, cols, rows)
    if codes is None:
        codes = torch.empty(shp, dtype=torch.uint8, device=t.device)
    if scales is None:
        scales = torch.empty(shp[:-1] + (rows // 32,), dtype=torch.uint8, device=t.device)
    _need(codes, g * rows * cols, torch.uint8, "moe_mx_quantize_t codes")
    _need(scales, g * cols * (rows // 32), torch.uint8, "moe_mx_quantize_t scales")
    _check(lib.moe_mx_quantize_t(_ptr(t), _TORCH_TO_CODE[t.dtype], g, rows, cols, _ptr(codes), _ptr(scales),
                                 shuffle_seed & 0xFFFFFFFFFFFFFFFF, _stream()), "moe_mx_quantize_t")
    return codes, scales


def moe_mx_fwd_fc1(prob: Problem, routing: Routing, x_mx, w1t_mx, h=None, act=None):
    """MXFP8 forward fc1: h and act = relu(h)^2 (bf16 [rows_cap, F]) from the
    (codes, scales) of x [T, D] (moe_mx_quantize) and of W1 transposed
    [num_local, F, D] (moe_mx_quantize_t of W1).  Returns (h, act)."""
    lib = load_library()
    (xc, xs), (wc, wsc) = x_mx, w1t_mx
    rc, T, D, F, el = prob.rows_cap, prob.tokens, prob.d_model, prob.d_ffn, prob.local
    if h is None:
        h = torch.empty((rc, F), dtype=torch.bfloat16, device=xc.device)
    if act is None:
        act = torch.empty((rc, F), dtype=torch.bfloat16, device=xc.device)
    _need(xc, T * D, torch.uint8, "moe_mx_fwd_fc1 x codes")
    _need(xs, T * (D // 32), torch.uint8, "moe_mx_fwd_fc1 x scales")
    _need(wc, el * F * D, torch.uint8, "moe_mx_fwd_fc1 W1^T codes")
    _need(wsc, el * F * (D // 32), torch.uint8, "moe_mx_fwd_fc1 W1^T scales")
    _need(h, rc * F, torch.bfloat16, "moe_mx_fwd_fc1 h")
    _need(act, rc * F, torch.bfloat16, "moe_mx_fwd_fc1 act")
    cp, cr = prob.c(), routing.c()
    _check(lib.moe_mx_fwd_fc1(ctypes.byref(cp), ctypes.byref(cr), _ptr(xc), _ptr(xs), _ptr(wc), _ptr(wsc), _ptr(h),
                              _ptr(act), _stream()), "moe_mx_fwd_fc1")
    return h, act


def moe_mx_fwd_fc2(prob: Problem, routing: Routing, act_mx, w2t_mx, mode: int = DETERMINISTIC, y=None, ws=None):
    """MXFP8 forward fc2 and the combine: y [T, D] (combine=1) or the o rows
    [rows_cap, D] (bf16) from the (codes, scales) of act [rows_cap, F]
    (moe_mx_quantize) and of W2 transposed [num_local, D, F] (moe_mx_quantize_t
    of W2).  The workspace is the forward one (moe_workspace_size)."""
    lib = load_library()
    (ac, asc), (wc, wsc) = act_mx, w2t_mx
    rc, T, D, F, el = prob.rows_cap, prob.tokens, prob.d_model, prob.d_ffn, prob.local
    out_rows = T if prob.combine else rc
    if y is None:
        y = torch.empty((out_rows, D), dtype=torch.bfloat16, device=ac.device)
    ws = _ws(moe_workspace_size(prob, mode)[0], ws, ac.device)
    _need(ac, rc * F, torch.uint8, "moe_mx_fwd_fc2 act codes")
    _need(asc, rc * (F // 32), torch.uint8, "moe_mx_fwd_fc2 act scales")
    _need(wc, el * D * F, torch.uint8, "moe_mx_fwd_fc2 W2^T codes")
    _need(wsc, el * D * (F // 32), torch.uint8, "moe_mx_fwd_fc2 W2^T scales")
    _need(y, out_rows * D, torch.bfloat16, "moe_mx_fwd_fc2 y")
    cp, cr = prob.c(), routing.c()
    _check(lib.moe_mx_fwd_fc2(ctypes.byref(cp), ctypes.byref(cr), _ptr(ac), _ptr(asc), _ptr(wc), _ptr(wsc), _ptr(y),
                              _ptr(ws), ws.numel(), mode, _stream()), "moe_mx_fwd_fc2")
    return y


def moe_mx_wgrad_rows(prob: Problem) -> int:
    """rpad_cap: padded rows of the MXFP8 weight-gradient operands (each
    expert's routed rows padded to a multiple of 64)."""
    v = ctypes.c_int64()
    _check(load_library().moe_mx_wgrad_rows(ctypes.byref(prob.c()), ctypes.byref(v)), "moe_mx_wgrad_rows")
    return v.value


def moe_mx_quantize_wgrad(prob: Problem, routing: Routing, src: torch.Tensor, kind: int, codes=None, scales=None):
    """MXFP8 of a weight-gradient operand along each expert's routed rows.
    kind MXW_TOKEN: src [T, D] gathered by token (x, dY); MXW_ROW: src
    [rows_cap, F] (dH); MXW_ACT_P: src = h [rows_cap, F], encodes
    p relu(h)^2.  Returns (codes uint8 [rpad_cap / 64, cols, 64], scales
    uint8 [rpad_cap / 64, cols, 2]), slice-major; slices past the padded
    total are not written."""
    lib = load_library()
    rp = moe_mx_wgrad_rows(prob)
    cols = prob.d_model if kind == MXW_TOKEN else prob.d_ffn
    rows = prob.tokens if kind == MXW_TOKEN else prob.rows_cap
    _need(src, rows * cols, torch.bfloat16, "moe_mx_quantize_wgrad src")
    if codes is None:
        codes = torch.empty((rp // 64, cols, 64), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty((rp // 64, cols, 2), dtype=torch.uint8, device=src.device)
    _need(codes, cols * rp, torch.uint8, "moe_mx_quantize_wgrad codes")
    _need(scales, cols * (rp // 32), torch.uint8, "moe_mx_quantize_wgrad scales")
    cp, cr = prob.c(), routing.c()
    _check(lib.moe_mx_quantize_wgrad(ctypes.byref(cp), ctypes.byref(cr), _ptr(src), kind, _ptr(codes), _ptr(scales),
                                     _stream()), "moe_mx_quantize_wgrad")
    return codes, scales


def moe_mx_wgrad(prob: Problem, routing: Routing, x_mx, dh_mx, act_mx, dy_mx, dw1=None, dw2=None):
    """MXFP8 weight gradients dW1 [num_local, D, F] and dW2 [num_local, F, D]
    (float32) from the moe_mx_quantize_wgrad encodings of x (MXW_TOKEN), dH
    (MXW_ROW), h (MXW_ACT_P) and dY (MXW_TOKEN)."""
    lib = load_library()
    rp = moe_mx_wgrad_rows(prob)
    D, F, el = prob.d_model, prob.d_ffn, prob.local
    ops = []
    for (c, s), n, name in ((x_mx, D, "x"), (dh_mx, F, "dh"), (act_mx, F, "act"), (dy_mx, D, "dy")):
        _need(c, n * rp, torch.uint8, f"moe_mx_wgrad {name} codes")
        _need(s, n * (rp // 32), torch.uint8, f"moe_mx_wgrad {name} scales")
        ops += [_ptr(c), _ptr(s)]
    dev = x_mx[0].device
    if dw1 is None:
        dw1 = torch.empty((el, D, F), dtype=torch.float32, device=dev)
    if dw2 is None:
        dw2 = torch.empty((el, F, D), dtype=torch.float32, device=dev)
    _need(dw1, el * D * F, torch.float32, "moe_mx_wgrad dw1")
    _need(dw2, el * F * D, torch.float32, "moe_mx_wgrad dw2")
    cp, cr = prob.c(), routing.c()
    _check(lib.moe_mx_wgrad(ctypes.byref(cp), ctypes.byref(cr), *ops, _ptr(dw1), _ptr(dw2), _stream()),
           "moe_mx_wgrad")
    return dw1, dw2


def moe_fingerprint(t: torch.Tensor, dtype: Optional[str] = None, chunk_elems: int = 65536,
                    shape=None, sync: bool = True):
    """Chunk hashes (device uint64 as int64 tensor) and the total.

    ``dtype`` names the element type ("f32", "bf16", "i32", ...); by default
    it follows the tensor.  With ``sync`` the 8-byte total is copied to the
    host and returned as a Python int; otherwise the device tensor."""
    lib = load_library()
    if not t.is_contiguous():
        raise MoeError("fingerprint needs a contiguous tensor")
    code = DTYPE_CODE[dtype] if dtype else _TORCH_TO_CODE[t.dtype]
    shape = tuple(t.shape) if shape is None else tuple(shape)
    n = 1
    for s in shape:
        n *= s
    m = (n + chunk_elems - 1) // chunk_elems
    hashes = torch.empty(max(m, 1), dtype=torch.int64, device=t.device)
    total = torch.empty(1, dtype=torch.int64, device=t.device)
    arr = (ctypes.c_int64 * max(len(shape), 1))(*shape)
    _check(lib.moe_fingerprint(_ptr(t), code, len(shape), arr, chunk_elems, _ptr(hashes), _ptr(total), _stream()),
           "moe_fingerprint")
    if not sync:
        return hashes[:m], total
    return hashes[:m], int(total.item()) & 0xFFFFFFFFFFFFFFFF


def moe_mfma_rate(blocks: int, iters: int, value: float = 0.125, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Enqueue the MFMA-rate loop on the current stream; returns the sink
    (float32 [256 * blocks] on the current device)."""
    lib = load_library()
    if sink is None:
        sink = torch.empty(256 * blocks, dtype=torch.float32, device="cuda")
    _check(lib.moe_mfma_rate(blocks, iters, value, _ptr(sink), _stream()), "moe_mfma_rate")
    return sink
