"""The C-ABI library loads and exports every entry point include/ispa.h declares (CPU only: no compute)."""
import ctypes
import os
import re

import pytest

from kv_cache_absorption_ispa_amd import ispa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "ispa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ispa_[a-z_0-9]+)\s*\(", text)))


def test_header_lists_the_entry_points():
    names = header_functions()
    for n in ("ispa_decomp_attn", "ispa_gram_accum", "ispa_absorb_solve", "ispa_full_attn", "ispa_lse_merge",
              "ispa_layer_eps", "ispa_select_layers", "ispa_absorb_apply"):
        assert n in names
    assert sorted(ispa.EXPORTS) == names


@pytest.mark.skipif(not os.path.exists(ispa.LIB_PATH), reason="libispa.so not built")
def test_library_exports_every_declared_symbol():
    # RTLD_NOW: every symbol the library needs must resolve at load time (a kernel whose
    # launch stub went missing shows up here, not only at its first launch on a GPU)
    lib = ctypes.CDLL(ispa.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    for n in header_functions():
        assert hasattr(lib, n), n
    lib2 = ispa.load_library()
    assert lib2.ispa_version() >= 100
    assert lib2.ispa_status_string(0) == b"ISPA_OK"
    assert lib2.ispa_status_string(3) == b"ISPA_E_WORKSPACE"


@pytest.mark.skipif(not os.path.exists(ispa.LIB_PATH), reason="libispa.so not built")
def test_validation_errors_need_no_gpu():
    """Argument validation returns before any HIP call, so it is testable on the host."""
    lib = ispa.load_library()
    desc = ispa.AttnDesc(2, 96, 8, 8, 0, 0.1, 1)  # head_dim 96 unsupported
    st = lib.ispa_decomp_attn(ctypes.byref(desc), *([None] * 11), None, 0, None)
    assert st == ispa.ISPA_E_INVALID_ARG
    assert b"head_dim" in lib.ispa_last_error()
    desc = ispa.AttnDesc(2, 64, 8, 0, 0, 0.1, 1)  # n_loc = 0
    assert lib.ispa_decomp_attn(ctypes.byref(desc), *([None] * 11), None, 0, None) == ispa.ISPA_E_INVALID_ARG
    desc = ispa.AttnDesc(2, 64, 8, 4, 0, 0.1, 1)  # null Q
    assert lib.ispa_decomp_attn(ctypes.byref(desc), *([None] * 11), None, 0, None) == ispa.ISPA_E_INVALID_ARG
    misaligned = ctypes.c_void_p(0x1004)
    assert lib.ispa_decomp_attn(ctypes.byref(desc), misaligned, misaligned, misaligned,
                                *([None] * 8), None, 0, None) == ispa.ISPA_E_INVALID_ARG
    # a bf16 merge with history keys needs the float32 workspace
    d2 = ispa.AttnDesc(2, 128, 100, 50, 70, 0.1, 1)
    assert lib.ispa_decomp_attn_workspace_size(ctypes.byref(d2)) == 100 * 2 * 128 * 4
    d3 = ispa.AttnDesc(2, 128, 100, 50, 0, 0.1, 1)
    assert lib.ispa_decomp_attn_workspace_size(ctypes.byref(d3)) == 0
    ok = ctypes.c_void_p(0x10000)
    assert lib.ispa_decomp_attn(ctypes.byref(d2), ok, ok, ok, ok, ok, None, None, None, None, ok, None,
                                None, 0, None) == ispa.ISPA_E_WORKSPACE
    assert lib.ispa_absorb_solve(100, 64, 1, *([None] * 3), 0.01, *([None] * 4), 0, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_absorb_solve(128, 64, 1, *([None] * 3), -1.0, *([None] * 4), 0, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_gram_accum(10, 192, ispa.ISPA_BF16, *([None] * 5), 0, None, 0, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_gram_accum(10, 128, ispa.ISPA_BF16, *([None] * 5), 2, None, 0, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_lse_merge(0, None, None, 4, 2, 64, 1, None, None, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_lse_merge(17, None, None, 4, 2, 64, 1, None, None, None) == ispa.ISPA_E_INVALID_ARG
    # layer selection: k within [0, n_layers], at most 4096 layers, eps required
    assert lib.ispa_select_layers(30, ok, 31, ok, None, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_select_layers(30, ok, -1, ok, None, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_select_layers(4097, ok, 1, ok, None, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_select_layers(30, None, 15, ok, None, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_select_layers(30, ok, 15, None, None, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_absorb_apply(128, 128, 30, ok, 31, ok, ok, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_absorb_apply(128, 128, 30, None, 15, ok, ok, None) == ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_absorb_apply(3, 5, 30, ok, 15, ok, ok, None) == ispa.ISPA_E_INVALID_ARG
    # nothing to apply: succeeds without touching the device
    assert lib.ispa_absorb_apply(128, 128, 30, None, 0, None, None, None) == ispa.ISPA_OK


@pytest.mark.skipif(not os.path.exists(ispa.LIB_PATH), reason="libispa.so not built")
def test_workspace_queries():
    lib = ispa.load_library()
    # the absorb factor lives in the workspace: at least batch*d*d floats
    assert lib.ispa_absorb_workspace_size(1536, 1536, 30) >= 30 * 1536 * 1536 * 4
    assert lib.ispa_eps_workspace_size(1536, 1536, 2) == 3 * 2 * 1536 * 1536 * 4
    # bf16: the split D_hi, D_lo of the rows (2 x 2 bytes per element), a counter per output tile, and
    # partial sums only when the tiles alone cannot fill the GPU
    dsplit = 2 * 4680 * 5120 * 2
    assert dsplit <= lib.ispa_gram_workspace_size(4680, 5120, ispa.ISPA_BF16) < dsplit + (1 << 20)  # no split
    dsplit = 2 * 4680 * 1536 * 2
    assert lib.ispa_gram_workspace_size(4680, 1536, ispa.ISPA_BF16) >= dsplit + 2 * 3 * 1536 * 1536 * 4  # split rows
    # more rows than one block: the split is formed 32768 rows at a time
    assert lib.ispa_gram_workspace_size(10 ** 6, 1536, ispa.ISPA_BF16) == lib.ispa_gram_workspace_size(32768, 1536,
                                                                                                     ispa.ISPA_BF16)
    assert lib.ispa_gram_workspace_size(0, 1536, ispa.ISPA_BF16) == 0
    assert lib.ispa_gram_workspace_size(256, 128, ispa.ISPA_F32) == 0


@pytest.mark.skipif(not os.path.exists(ispa.LIB_PATH), reason="libispa.so not built")
def test_segment_validation_needs_no_gpu():
    """ispa_decomp_attn_segments rejects bad segment lists before any HIP call."""
    lib = ispa.load_library()
    ok = 0x10000

    def call(desc, segs, n_loc_segs, n_segs=None, o_full=None, ws=None, ws_bytes=0):
        arr = (ispa.KvSegment * max(len(segs), 1))(*[ispa.KvSegment(k, v, n) for k, v, n in segs])
        n_segs = len(segs) if n_segs is None else n_segs
        return lib.ispa_decomp_attn_segments(ctypes.byref(desc), ok, arr, n_segs, n_loc_segs, None, None, None,
                                             None, o_full, None, ws, ws_bytes, None)

    d = ispa.AttnDesc(2, 128, 100, 50, 70, 0.1, 1)
    good = [(ok, ok, 20), (ok, ok, 30), (ok, ok, 70)]
    bad = ispa.ISPA_E_INVALID_ARG
    assert call(d, good, 0) == bad                      # no local segment
    assert call(d, good, 4) == bad                      # more local segments than segments
    assert call(d, good, 1) == bad                      # local rows 20 != n_loc 50
    assert call(d, good, 3) == bad                      # history rows 0 != n_hist 70
    assert call(d, good, 2, n_segs=0) == bad
    assert call(d, good * 6, 2, n_segs=17) == bad       # above ISPA_MAX_KV_SEGMENTS
    assert call(d, [(ok, ok, 50), (ok, ok, 0), (ok, ok, 70)], 1) == bad  # empty segment
    assert call(d, [(ok, ok, 50), (ok + 8, ok, 70)], 1) == bad           # misaligned K
    assert call(d, [(ok, ok, 50), (ok, None, 70)], 1) == bad             # null V
    assert b"n_loc" in (call(d, good, 1) and lib.ispa_last_error())
    # the merge's float32 workspace is still required with history keys
    assert call(d, good, 2, o_full=ok) == ispa.ISPA_E_WORKSPACE
    assert call(d, good, 2, o_full=ok, ws=ok, ws_bytes=100 * 2 * 128 * 4 - 1) == ispa.ISPA_E_WORKSPACE
    assert ispa.ISPA_MAX_KV_SEGMENTS == 16
    hdr = open(os.path.join(ROOT, "include", "ispa.h")).read()
    assert "#define ISPA_MAX_KV_SEGMENTS 16" in hdr


@pytest.mark.skipif(not os.path.exists(ispa.LIB_PATH), reason="libispa.so not built")
def test_splitkv_validation_needs_no_gpu():
    lib = ispa.load_library()
    ok = 0x10000
    seg = (ispa.KvSegment * 2)(ispa.KvSegment(ok, ok, 50), ispa.KvSegment(ok, ok, 70))

    def call(desc, workers, n_loc_segs=1):
        return lib.ispa_decomp_attn_splitkv(ctypes.byref(desc), ok, seg, 2, n_loc_segs, workers, *([None] * 6),
                                            None, 0, None)

    bad = ispa.ISPA_E_INVALID_ARG
    d = ispa.AttnDesc(2, 128, 100, 50, 70, 0.1, 1)
    assert call(ispa.AttnDesc(2, 128, 100, 50, 70, 0.1, 0), 4) == bad  # float32: bf16 only
    assert b"bf16" in lib.ispa_last_error()
    assert call(d, -1) == bad
    assert call(d, 65536) == bad
    assert call(d, 4, n_loc_segs=2) == bad  # local rows 120 != 50
    # workspace: the merge's float32 O_loc (rounded up to 256 bytes) + 1 slot of 2*256*(128+1) floats per worker
    stash = (100 * 2 * 128 * 4 + 255) // 256 * 256
    slot = (2 * 256 * 128 + 2 * 256) * 4
    assert lib.ispa_decomp_attn_splitkv_workspace_size(ctypes.byref(d), 7) == stash + 7 * slot
    d0 = ispa.AttnDesc(2, 128, 100, 50, 0, 0.1, 1)
    assert lib.ispa_decomp_attn_splitkv_workspace_size(ctypes.byref(d0), 7) == 7 * slot
    assert lib.ispa_decomp_attn_splitkv_workspace_size(ctypes.byref(d), -3) == 0


@pytest.mark.skipif(not os.path.exists(ispa.LIB_PATH), reason="libispa.so not built")
def test_variant_validation_needs_no_gpu():
    lib = ispa.load_library()
    ok = 0x10000
    bad = ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_fit_error(100, 64, 1, ok, ok, ok, ok, None, ok, ok, None, 0, None) == bad  # d % 64
    assert lib.ispa_fit_error(128, 64, 1, ok, ok, None, ok, None, ok, ok, None, 0, None) == bad  # E required
    assert lib.ispa_fit_error_workspace_size(128, 64, 3) == 4 * 3 * 128 * 64 * 4
    assert lib.ispa_lambda_from_trace(128, 2, ok, -1.0, ok, None) == bad
    assert lib.ispa_lambda_from_trace(128, 0, ok, 1.0, ok, None) == bad
    assert lib.ispa_absorb_solve_lambdas(128, 64, 1, ok, ok, ok, None, ok, None, ok, None, 0, None) == bad
    assert lib.ispa_select_layers_below(30, ok, 0.5, 31, ok, ok, None, None) == bad  # k_max > n_layers
    assert lib.ispa_select_layers_below(30, ok, float("nan"), 3, ok, ok, None, None) == bad
    assert lib.ispa_select_layers_below(30, ok, 0.5, 3, ok, None, None, None) == bad  # count required
    assert lib.ispa_gather_layers(4, 0, ok, ok, 2, ok, None) == bad
    assert lib.ispa_gather_layers(4, 16, ok, ok, 0, None, None) == ispa.ISPA_OK  # nothing to gather
    assert lib.ispa_absorb_apply_compact(128, 64, 4, ok, 5, ok, ok, None) == bad
    assert lib.ispa_absorb_apply_compact(128, 64, 4, None, 0, None, None, None) == ispa.ISPA_OK


def test_every_entry_point_has_a_python_wrapper():
    skip = {"ispa_status_string", "ispa_last_error"}
    missing = [n for n in ispa.EXPORTS if n not in skip and not callable(getattr(ispa, n, None))]
    assert missing == []


@pytest.mark.skipif(not os.path.exists(ispa.LIB_PATH), reason="libispa.so not built")
def test_absorb_solve_ex_validation_needs_no_gpu():
    lib = ispa.load_library()
    ok = 0x10000
    bad = ispa.ISPA_E_INVALID_ARG
    assert lib.ispa_absorb_solve_ex(128, 64, 1, ok, ok, ok, 0.01, None, 2, ok, None, ok, None, 0, None, None) == bad
    assert lib.ispa_absorb_solve_ex(128, 64, 1, ok, ok, ok, -1.0, None, 0, ok, None, ok, None, 0, None, None) == bad
    assert lib.ispa_absorb_solve_ex(100, 64, 1, ok, ok, ok, 0.01, None, 1, ok, None, ok, None, 0, None, None) == bad
    # a side stream needs all three handles and must differ from the main stream
    part = ispa.SideStreamDesc(0x20000, None, 0x30000)
    assert lib.ispa_absorb_solve_ex(128, 64, 1, ok, ok, ok, 0.01, None, 0, ok, None, ok, None, 0,
                                    ctypes.byref(part), None) == bad
    assert b"side stream" in lib.ispa_last_error()
    same = ispa.SideStreamDesc(0x20000, 0x30000, 0x40000)
    assert lib.ispa_absorb_solve_ex(128, 64, 1, ok, ok, ok, 0.01, None, 0, ok, None, ok, None, 0,
                                    ctypes.byref(same), 0x20000) == bad
    assert b"differ" in lib.ispa_last_error()


def test_size_limits_are_rejected_without_a_gpu():
    """The documented size limits (fewer than 2^31 elements in each attention tensor, n_rows * d
    below 2^40 for the Gram) are checked before any HIP call.  Only the rejected side is exercised
    here: an accepted call would go on to the device.  (The LSE bound H * n_q < 2^31 follows from
    the bound on Q, since D >= 64.)"""
    lib = ispa.load_library()
    ok = ctypes.c_void_p(0x10000)
    args = [ok, ok, ok, ok, ok] + [None] * 6
    for n_q, n_loc, n_hist in ((1 << 20, 8, 0),             # Q: 2^20 * 16 * 128 = 2^31 elements
                               (8, (1 << 20) - 8, 8),       # keys: n_loc + n_hist = 2^20
                               (8, 8, 1 << 20)):
        desc = ispa.AttnDesc(16, 128, n_q, n_loc, n_hist, 0.1, ispa.ISPA_BF16)
        assert lib.ispa_decomp_attn(ctypes.byref(desc), *args, None, 0, None) == ispa.ISPA_E_INVALID_ARG
        assert b"too large" in lib.ispa_last_error()
    assert lib.ispa_gram_accum(1 << 30, 1024, ispa.ISPA_BF16, ok, ok, ok, ok, None, 0, None, 0,
                               None) == ispa.ISPA_E_INVALID_ARG
    assert b"too many rows" in lib.ispa_last_error()
