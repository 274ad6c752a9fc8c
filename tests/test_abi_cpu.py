"""The C-ABI library loads, exports every symbol declared in include/*.h, and
rejects invalid arguments before enqueuing anything (no GPU needed: these
paths return before any HIP call)."""
import ctypes
import glob
import os
import re

import pytest

import bitwise_deterministic_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(hdr).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M))
    return names


@pytest.fixture(scope="module")
def lib():
    return moe.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"moe_fwd", "moe_bwd_dgrad_dprob", "moe_bwd_wgrad", "moe_fingerprint"} <= names
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(moe.EXPORTED_SYMBOLS)
    assert lib.moe_abi_version() == 5


def test_library_is_built_from_the_tree(lib):
    # the loader refuses an in-tree library built from other sources; the
    # hash it carries is the build script's hash of the tree
    from bitwise_deterministic_moe_amd.build import source_hash
    assert len(source_hash()) == 16
    assert moe.moe_source_hash() == source_hash()


def test_status_strings(lib):
    for s in range(7):
        assert lib.moe_status_string(s)


BASE = dict(tokens=4096, d_model=1024, d_ffn=2048, num_experts=8, top_k=2)


@pytest.mark.parametrize("bad", [
    dict(top_k=0), dict(top_k=9), dict(num_experts=2000, top_k=2), dict(d_model=1000), dict(d_ffn=64),
    dict(tokens=-1), dict(expert_begin=7, num_local=2, combine=0), dict(num_local=4),  # combine=1 needs all experts
    dict(d_ffn=256 * 65), dict(top_k=65, num_experts=100),
    # token arrays [T, D] of 2 GiB; routed-row arrays [rows_cap, max(D, F)] of 32 GiB
    dict(tokens=1 << 20, d_model=1024), dict(tokens=1 << 19, d_model=256, d_ffn=4096, top_k=8),
])
def test_shape_validation(bad):
    p = moe.Problem(**{**BASE, **bad})
    with pytest.raises(moe.MoeError, match="status 2"):
        moe.moe_workspace_size(p)


def test_routed_row_arrays_beyond_2gib_are_accepted():
    # 65536 tokens top-8 of 8 experts at d_ffn 4096: h, dh and act_p are 4 GiB
    # each, addressed from each tile's first row
    p = moe.Problem(**{**BASE, "tokens": 1 << 16, "d_ffn": 4096, "top_k": 8})
    assert moe.moe_rows_cap(p) * 4096 * 2 == 4 << 30
    fwd, dgrad, wgrad = moe.moe_workspace_size(p)
    assert wgrad >= 4 << 30 and dgrad > 0 and fwd >= 4 << 30


def test_dtype_and_mode_validation(lib):
    p = moe.Problem(**BASE)
    cp = p.c()
    cp.dtype = 7
    sz = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(cp), 0, ctypes.byref(sz), None, None) == 3
    assert lib.moe_workspace_size(ctypes.byref(p.c()), 2, ctypes.byref(sz), None, None) == 5
    cp = p.c()
    cp.combine = 2
    assert lib.moe_workspace_size(ctypes.byref(cp), 0, ctypes.byref(sz), None, None) == 5


def test_null_and_workspace_errors_return_before_enqueue(lib):
    p = moe.Problem(**BASE)
    cp = p.c()
    fake = ctypes.c_void_p(0x1000)
    r = moe._CRouting(*([0x2000] * 9))
    # NULL x
    assert lib.moe_fwd(ctypes.byref(cp), fake, None, fake, fake, ctypes.byref(r), fake, fake, fake, 1 << 30, 0,
                       None) == 1
    # workspace too small
    assert lib.moe_fwd(ctypes.byref(cp), fake, fake, fake, fake, ctypes.byref(r), fake, fake, fake, 16, 0, None) == 4
    # misaligned workspace
    assert lib.moe_bwd_wgrad(ctypes.byref(cp), ctypes.byref(r), fake, fake, fake, fake, fake, fake,
                             ctypes.c_void_p(0x1008), 1 << 40, 0, None) == 4
    assert lib.moe_bwd_dgrad_dprob(None, ctypes.byref(r), fake, fake, fake, fake, fake, fake, fake, fake, 0,
                                   0, None) == 1
    # NULL dh
    assert lib.moe_bwd_dgrad_dprob(ctypes.byref(cp), ctypes.byref(r), fake, fake, fake, fake, fake, fake, None,
                                   fake, 1 << 40, 0, None) == 1
    # NULL h for the weight gradients
    assert lib.moe_bwd_wgrad(ctypes.byref(cp), ctypes.byref(r), fake, fake, None, fake, fake, fake, fake, 1 << 40, 0,
                             None) == 1
    # fingerprint argument checks
    shape = (ctypes.c_int64 * 1)(10)
    assert lib.moe_fingerprint(fake, 9, 1, shape, 4, fake, fake, None) == 3
    assert lib.moe_fingerprint(fake, 0, 1, shape, 0, fake, fake, None) == 2
    assert lib.moe_fingerprint(fake, 0, 9, shape, 4, fake, fake, None) == 2
    assert lib.moe_fingerprint(fake, 0, 1, shape, 4, fake, None, None) == 1


def test_workspace_sizes_and_rows_cap():
    p = moe.Problem(**BASE)
    fwd, dg, wg = moe.moe_workspace_size(p, moe.DETERMINISTIC)
    assert moe.moe_rows_cap(p) == 8192
    # dprob partials: rows_cap x (F / 256) floats
    assert dg >= 8192 * 8 * 4
    fa, da, wa = moe.moe_workspace_size(p, moe.ATOMIC)
    # chunk 4 * mean rows = 4096 >= tokens: no expert can split, no partial
    # slots; both modes hold act_p [rows_cap, F] bf16
    assert wa == wg and da >= 4096 * 1024 * 4
    assert wg >= 8192 * 2048 * 2
    assert moe.moe_stage_names(p, 0, 2) == ["wgrad_prep_act_p", "wgrad_fc1_fc2_ordered"]
    # 512 experts top-22: 32768 weight-gradient tiles, so no expert is split
    # (chunk 4096 = tokens): no slots, no ordered reduction
    latent = moe.Problem(4096, 2048, 2048, 512, 22)
    _, _, wl = moe.moe_workspace_size(latent, moe.DETERMINISTIC)
    _, _, wla = moe.moe_workspace_size(latent, moe.ATOMIC)
    assert wl == wla
    assert moe.moe_stage_names(latent, 0, 2) == ["wgrad_prep_act_p", "wgrad_fc1_fc2_ordered"]
    assert moe.moe_stage_names(latent, 1, 2) == ["wgrad_prep_act_p_zero", "wgrad_fc1_fc2"]
    # 8 experts, 16384 tokens top-2: 128 tiles, chunk 4096 < tokens: split
    # slots (rows_cap / chunk = 8 per weight gradient) in the deterministic workspace
    wide = moe.Problem(16384, 1024, 1024, 8, 2)
    _, _, ww = moe.moe_workspace_size(wide, moe.DETERMINISTIC)
    _, _, wwa = moe.moe_workspace_size(wide, moe.ATOMIC)
    assert ww - wwa >= 2 * 8 * 1024 * 1024 * 4
    # the ordered reduction rides in the pair launch: the same two launches
    # in both modes
    assert moe.moe_stage_names(wide, 0, 2) == ["wgrad_prep_act_p", "wgrad_fc1_fc2_ordered"]
    assert moe.moe_stage_names(wide, 1, 2) == ["wgrad_prep_act_p_zero", "wgrad_fc1_fc2"]
    # the float32 path keeps its separate ordered reduction
    wide32 = moe.Problem(16384, 64, 64, 8, 2, dtype="f32")
    assert moe.moe_stage_names(wide32, 0, 2) == ["wgrad_prep_act_p", "wgrad_fc1", "wgrad_fc2", "wgrad_reduce"]
    shard = moe.Problem(16384, 2048, 2048, 512, 22, 0, 4, "bf16", 0)
    assert moe.moe_rows_cap(shard) == 16384 * 4
    assert moe.moe_stage_names(p, 0, 1) == ["fc2_dgrad_dprob_partials", "fc1_dgrad_dprob_combine",
                                            "dx_combine_gather"]
    assert moe.moe_stage_names(p, 1, 2) == ["wgrad_prep_act_p_zero", "wgrad_fc1_fc2"]


def test_mfma_rate_validation_returns_before_enqueue(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_mfma_rate(0, 10, 0.125, fake, None) == 2          # no blocks
    assert lib.moe_mfma_rate(1 << 31, 10, 0.125, fake, None) == 2    # grid too large
    assert lib.moe_mfma_rate(4, 0, 0.125, fake, None) == 2           # no iterations
    assert lib.moe_mfma_rate(4, 10, 0.1, fake, None) == 2            # 0.1 is not a bf16 value
    assert lib.moe_mfma_rate(4, 10, 0.125, None, None) == 1          # NULL sink


def test_router_bwd_validation_returns_before_enqueue(lib):
    fake = ctypes.c_void_p(0x1000)
    r = moe._CRouting(*([0x2000] * 9))
    cp = moe.Problem(**BASE).c()
    ok_args = lambda: [fake] * 6
    # NULL dprob / x / outputs with tokens > 0
    assert lib.moe_router_bwd(ctypes.byref(cp), ctypes.byref(r), None, *ok_args()[:5], 0, None) == 1
    assert lib.moe_router_bwd(ctypes.byref(cp), ctypes.byref(r), fake, fake, fake, fake, None, fake, 0, None) == 1
    # bad mode
    assert lib.moe_router_bwd(ctypes.byref(cp), ctypes.byref(r), *ok_args(), 7, None) == 5
    # a shard (num_local < num_experts, row layout) is rejected
    sp = moe.Problem(**{**BASE, "expert_begin": 2, "num_local": 4, "combine": 0}).c()
    assert lib.moe_router_bwd(ctypes.byref(sp), ctypes.byref(r), *ok_args(), 0, None) == 2
    # NULL routing arrays
    r0 = moe._CRouting(*([0x2000] * 2 + [0] + [0x2000] * 6))
    assert lib.moe_router_bwd(ctypes.byref(cp), ctypes.byref(r0), *ok_args(), 0, None) == 1


def test_router_fwd_and_sgd_validation_return_before_enqueue(lib):
    fake = ctypes.c_void_p(0x1000)
    cp = moe.Problem(**BASE).c()
    assert lib.moe_router_fwd(ctypes.byref(cp), None, fake, fake, None) == 1
    bad = moe.Problem(**{**BASE, "top_k": 0}).c()
    assert lib.moe_router_fwd(ctypes.byref(bad), fake, fake, fake, None) == 2
    assert lib.moe_sgd_step(fake, fake, 10, 0.1, fake, 7, None) == 3      # dtype
    assert lib.moe_sgd_step(fake, fake, -1, 0.1, fake, 1, None) == 2      # n < 0
    assert lib.moe_sgd_step(None, fake, 10, 0.1, fake, 1, None) == 1      # NULL master
    assert lib.moe_sgd_step(None, None, 0, 0.1, None, 1, None) == 0       # nothing to do


def test_mx_quantize_validation_returns_before_enqueue(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_mx_quantize(fake, 7, 4, 64, fake, fake, 0, None) == 3          # dtype
    assert lib.moe_mx_quantize(fake, 1, 4, 48, fake, fake, 0, None) == 2          # cols not a multiple of 32
    assert lib.moe_mx_quantize(fake, 1, -1, 64, fake, fake, 0, None) == 2         # rows < 0
    assert lib.moe_mx_quantize(None, 1, 4, 64, fake, fake, 0, None) == 1          # NULL input
    assert lib.moe_mx_quantize(ctypes.c_void_p(0x1008), 1, 4, 64, fake, fake, 0, None) == 2   # misaligned
    assert lib.moe_mx_quantize(None, 1, 0, 64, None, None, 0, None) == 0          # empty


def test_mx_dgrad_fc1_validation_returns_before_enqueue(lib):
    fake = ctypes.c_void_p(0x1000)
    r = moe._CRouting(*([0x2000] * 9))
    big = moe.Problem(**{**BASE, "d_ffn": 4096}).c()
    assert lib.moe_mx_dgrad_fc1(ctypes.byref(big), ctypes.byref(r), fake, fake, fake, fake, fake, None) == 2
    f32 = moe.Problem(**{**BASE, "dtype": "f32"}).c()
    assert lib.moe_mx_dgrad_fc1(ctypes.byref(f32), ctypes.byref(r), fake, fake, fake, fake, fake, None) == 3
    cp = moe.Problem(**BASE).c()
    assert lib.moe_mx_dgrad_fc1(ctypes.byref(cp), ctypes.byref(r), None, fake, fake, fake, fake, None) == 1


def test_mx_dgrad_fc2_validation_returns_before_enqueue(lib):
    fake = ctypes.c_void_p(0x1000)
    r = moe._CRouting(*([0x2000] * 9))
    cp = moe.Problem(**BASE).c()

    def call(prob, dy=fake, mode=0, ws=ctypes.c_void_p(0x100000), ws_bytes=1 << 40):
        return lib.moe_mx_dgrad_fc2(ctypes.byref(prob), ctypes.byref(r), dy, fake, fake, fake, fake, fake, fake,
                                    ws, ws_bytes, mode, None)
    assert call(moe.Problem(**{**BASE, "d_model": 4096}).c()) == 2        # D beyond the staged scales
    assert call(moe.Problem(**{**BASE, "dtype": "f32"}).c()) == 3
    assert call(cp, mode=7) == 5
    assert call(cp, dy=None) == 1
    assert call(cp, ws_bytes=16) == 4                                      # workspace too small
    assert call(cp, ws=ctypes.c_void_p(0x100008)) == 4                     # misaligned


def test_mx_bindings_check_tensor_sizes_before_the_call():
    # CPU tensors of the wrong size: the binding raises before any pointer
    # reaches the library
    import torch
    p = moe.Problem(tokens=64, d_model=256, d_ffn=256, num_experts=4, top_k=2)
    rc, D, F, el = p.rows_cap, p.d_model, p.d_ffn, p.local
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8)  # noqa: E731
    r = moe.Routing(*[torch.zeros(1, dtype=torch.int32)] * 9)
    with pytest.raises(moe.MoeError, match="dh scales"):
        moe.moe_mx_dgrad_fc1(p, r, (u8(rc * F), u8(rc * F // 32 - 1)), (u8(el * D * F), u8(el * D * F // 32)))
    with pytest.raises(moe.MoeError, match="W2 codes"):
        moe.moe_mx_dgrad_fc2(p, r, (u8(64 * D), u8(64 * D // 32)), (u8(el * F * D + 1), u8(el * F * D // 32)),
                             torch.zeros(rc * F, dtype=torch.bfloat16))
    with pytest.raises(moe.MoeError, match="scales"):
        moe.moe_mx_quantize(torch.zeros(4, 64), scales=u8(3))


def test_nvfp4_quantize_validation_returns_before_enqueue(lib):
    fake, g = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x3000)
    assert lib.moe_nvfp4_quantize(fake, 2, 4, 64, fake, fake, g, 0, None) == 3             # i32 input
    assert lib.moe_nvfp4_quantize(fake, 1, 4, 40, fake, fake, g, 0, None) == 2             # cols % 16
    assert lib.moe_nvfp4_quantize(fake, 1, 4, 64, fake, fake, None, 0, None) == 1          # no tensor scale
    assert lib.moe_nvfp4_quantize(None, 1, 4, 64, fake, fake, g, 0, None) == 1
    assert lib.moe_nvfp4_quantize(ctypes.c_void_p(0x1008), 1, 4, 64, fake, fake, g, 0, None) == 2   # misaligned


def test_mx_forward_validation_returns_before_enqueue(lib):
    fake = ctypes.c_void_p(0x1000)
    r = moe._CRouting(*([0x2000] * 9))
    cp = moe.Problem(**BASE).c()
    # transposing quantiser: dtype, rows not a multiple of 32, NULL, misaligned codes, empty
    assert lib.moe_mx_quantize_t(fake, 2, 1, 64, 64, fake, fake, 0, None) == 3
    assert lib.moe_mx_quantize_t(fake, 1, 1, 48, 64, fake, fake, 0, None) == 2
    assert lib.moe_mx_quantize_t(None, 1, 1, 64, 64, fake, fake, 0, None) == 1
    assert lib.moe_mx_quantize_t(fake, 1, 1, 64, 64, ctypes.c_void_p(0x1008), fake, 0, None) == 2
    assert lib.moe_mx_quantize_t(None, 1, 0, 64, 64, None, None, 0, None) == 0
    # fc1: D beyond the staged scales, float32 problem, NULL operand
    big = moe.Problem(**{**BASE, "d_model": 4096}).c()
    assert lib.moe_mx_fwd_fc1(ctypes.byref(big), ctypes.byref(r), fake, fake, fake, fake, fake, fake, None) == 2
    f32 = moe.Problem(**{**BASE, "dtype": "f32"}).c()
    assert lib.moe_mx_fwd_fc1(ctypes.byref(f32), ctypes.byref(r), fake, fake, fake, fake, fake, fake, None) == 3
    assert lib.moe_mx_fwd_fc1(ctypes.byref(cp), ctypes.byref(r), None, fake, fake, fake, fake, fake, None) == 1
    # fc2: F beyond the staged scales, mode, workspace too small
    bigf = moe.Problem(**{**BASE, "d_ffn": 4096}).c()
    assert lib.moe_mx_fwd_fc2(ctypes.byref(bigf), ctypes.byref(r), fake, fake, fake, fake, fake, fake, 1 << 40, 0,
                              None) == 2
    assert lib.moe_mx_fwd_fc2(ctypes.byref(cp), ctypes.byref(r), fake, fake, fake, fake, fake,
                              ctypes.c_void_p(0x100000), 1 << 40, 7, None) == 5
    assert lib.moe_mx_fwd_fc2(ctypes.byref(cp), ctypes.byref(r), fake, fake, fake, fake, fake,
                              ctypes.c_void_p(0x100000), 16, 0, None) == 4


def test_mx_wgrad_rows_and_validation_return_before_enqueue(lib):
    p = moe.Problem(**BASE)
    rc, el = moe.moe_rows_cap(p), p.local
    # each expert's rows rounded up to 64: at most rows_cap + 63 per expert
    assert moe.moe_mx_wgrad_rows(p) == (rc + 63 * el + 63) // 64 * 64
    fake = ctypes.c_void_p(0x1000)
    r = moe._CRouting(*([0x2000] * 9))
    cp = p.c()
    f32 = moe.Problem(**{**BASE, "dtype": "f32"}).c()
    # quantiser: float32 problem, unknown kind, NULL source, NULL row_tok for
    # the token gather, misaligned codes
    assert lib.moe_mx_quantize_wgrad(ctypes.byref(f32), ctypes.byref(r), fake, 0, fake, fake, None) == 3
    assert lib.moe_mx_quantize_wgrad(ctypes.byref(cp), ctypes.byref(r), fake, 3, fake, fake, None) == 2
    assert lib.moe_mx_quantize_wgrad(ctypes.byref(cp), ctypes.byref(r), None, 1, fake, fake, None) == 1
    no_tok = moe._CRouting(*([0x2000] * 5 + [0] + [0x2000] * 3))
    assert lib.moe_mx_quantize_wgrad(ctypes.byref(cp), ctypes.byref(no_tok), fake, 0, fake, fake, None) == 1
    assert lib.moe_mx_quantize_wgrad(ctypes.byref(cp), ctypes.byref(r), fake, 1, ctypes.c_void_p(0x1008), fake,
                                     None) == 2
    # routed-row arrays of 32 GiB and more are rejected by every call
    huge = moe.Problem(**{**BASE, "tokens": 1 << 19, "d_model": 256, "d_ffn": 4096, "top_k": 8}).c()
    assert lib.moe_mx_quantize_wgrad(ctypes.byref(huge), ctypes.byref(r), fake, 1, fake, fake, None) == 2
    ops = [fake] * 8
    assert lib.moe_mx_wgrad(ctypes.byref(f32), ctypes.byref(r), *ops, fake, fake, None) == 3
    assert lib.moe_mx_wgrad(ctypes.byref(huge), ctypes.byref(r), *ops, fake, fake, None) == 2
    # a valid layer whose single expert could hold T rows of 2^31 encoded bytes
    wide = moe.Problem(**{**BASE, "tokens": 1 << 18, "d_model": 256, "d_ffn": 8192}).c()
    moe.moe_workspace_size(moe.Problem(**{**BASE, "tokens": 1 << 18, "d_model": 256, "d_ffn": 8192}))
    assert lib.moe_mx_quantize_wgrad(ctypes.byref(wide), ctypes.byref(r), fake, 1, fake, fake, None) == 2
    assert lib.moe_mx_wgrad(ctypes.byref(wide), ctypes.byref(r), *ops, fake, fake, None) == 2
    assert lib.moe_mx_wgrad(ctypes.byref(cp), ctypes.byref(r), *ops, None, fake, None) == 1
    assert lib.moe_mx_wgrad(ctypes.byref(cp), ctypes.byref(r), *([fake] * 7 + [None]), fake, fake, None) == 1
    # scales must be 16-byte aligned (they are streamed with 16-byte loads)
    assert lib.moe_mx_wgrad(ctypes.byref(cp), ctypes.byref(r), *([fake] * 3 + [ctypes.c_void_p(0x1002)] +
                                                                 [fake] * 4), fake, fake, None) == 2


def test_route_validation_and_stage_names(lib):
    p = moe.Problem(**BASE)
    assert moe.moe_stage_names(p, 0, 3) == ["route", "permute_scan", "permute_scatter"]
    assert moe.moe_stage_names(p, 1, 3) == ["route", "permute_scan", "permute_scatter_atomic"]
    fake = ctypes.c_void_p(0x1000)
    r = moe._CRouting(*([0x2000] * 9))
    cp = p.c()
    assert lib.moe_route(ctypes.byref(cp), fake, ctypes.byref(r), fake, 1 << 40, 9, None) == 5
    assert lib.moe_route(ctypes.byref(cp), None, ctypes.byref(r), fake, 1 << 40, 0, None) == 1
    assert lib.moe_route(ctypes.byref(cp), fake, ctypes.byref(r), ctypes.c_void_p(0x100000), 16, 0, None) == 4
    assert lib.moe_route(None, fake, ctypes.byref(r), fake, 1 << 40, 0, None) == 1


def test_mx_quantize_wgrad_needs_an_aligned_source(lib):
    r = moe._CRouting(*([0x2000] * 9))
    cp = moe.Problem(**BASE).c()
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_mx_quantize_wgrad(ctypes.byref(cp), ctypes.byref(r), ctypes.c_void_p(0x1002), 1, fake, fake,
                                     None) == 2
