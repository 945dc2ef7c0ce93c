"""Thin ctypes binding of libispa.so (argument marshalling only).

Every function has the name of the C entry point it calls (see include/ispa.h
for the semantics).  Tensors are torch tensors on the current HIP device;
torch provides device memory and the stream, nothing else: all computation is
in the library's HIP kernels.  There is no fallback: if the library is not
built, or the device is not gfx950, calls raise :class:`IspaError`.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libispa.so")

ISPA_OK, ISPA_E_INVALID_ARG, ISPA_E_UNSUPPORTED, ISPA_E_WORKSPACE, ISPA_E_HIP = range(5)
ISPA_F32, ISPA_BF16 = 0, 1

EXPORTS = [
    "ispa_decomp_attn", "ispa_decomp_attn_noalloc", "ispa_decomp_attn_segments", "ispa_decomp_attn_splitkv",
    "ispa_decomp_attn_splitkv_workspace_size", "ispa_decomp_attn_workspace_size", "ispa_full_attn", "ispa_lse_merge", "ispa_gram_workspace_size", "ispa_gram_accum",
    "ispa_absorb_workspace_size", "ispa_absorb_solve", "ispa_eps_workspace_size", "ispa_layer_eps",
    "ispa_select_layers", "ispa_absorb_apply", "ispa_fit_error", "ispa_fit_error_workspace_size",
    "ispa_lambda_from_trace", "ispa_absorb_solve_lambdas", "ispa_select_layers_below", "ispa_gather_layers",
    "ispa_absorb_apply_compact", "ispa_absorb_solve_ex", "ispa_decomp_attn_fp8k", "ispa_quantize_fp8_heads",
    "ispa_quantize_fp8_heads_workspace_size", "ispa_quantize_fp8_rows", "ispa_quantize_fp8_cols", "ispa_w8a8_gemm", "ispa_status_string", "ispa_last_error", "ispa_version", "ispa_device_check",
]


class IspaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("n_q", ctypes.c_int64),
        ("n_loc", ctypes.c_int64),
        ("n_hist", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class KvSegment(ctypes.Structure):
    _fields_ = [("K", ctypes.c_void_p), ("V", ctypes.c_void_p), ("n_rows", ctypes.c_int64)]


class KvSegmentFp8k(ctypes.Structure):
    _fields_ = [("K8", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("V", ctypes.c_void_p),
                ("n_rows", ctypes.c_int64)]


class SideStreamDesc(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("ev_fork", ctypes.c_void_p), ("ev_join", ctypes.c_void_p)]


ISPA_MAX_KV_SEGMENTS = 16
ISPA_MAX_SPLITKV_WORKERS = 65535

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libispa.so and declare its signatures (no GPU needed to load)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise IspaError(-1, f"{path} is not built; run `python -m kv_cache_absorption_ispa_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, None
    sig = {
        "ispa_decomp_attn": (I32, [ctypes.POINTER(AttnDesc)] + [P] * 12 + [SZ, P]),
        "ispa_decomp_attn_noalloc": (I32, [ctypes.POINTER(AttnDesc)] + [P] * 11 + [P]),
        "ispa_decomp_attn_segments": (I32, [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(KvSegment), I32, I32]
                                      + [P] * 7 + [SZ, P]),
        "ispa_decomp_attn_splitkv": (I32, [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(KvSegment), I32, I32, I32]
                                     + [P] * 7 + [SZ, P]),
        "ispa_decomp_attn_splitkv_workspace_size": (SZ, [ctypes.POINTER(AttnDesc), I32]),
        "ispa_decomp_attn_workspace_size": (SZ, [ctypes.POINTER(AttnDesc)]),
        "ispa_full_attn": (I32, [ctypes.POINTER(AttnDesc), P, P, P, P, P, P]),
        "ispa_lse_merge": (I32, [I32, P, P, I64, I32, I32, I32, P, P, P]),
        "ispa_gram_workspace_size": (SZ, [I64, I32, I32]),
        "ispa_gram_accum": (I32, [I64, I32, I32, P, P, P, P, P, I32, P, SZ, P]),
        "ispa_absorb_workspace_size": (SZ, [I32, I32, I32]),
        "ispa_absorb_solve": (I32, [I32, I32, I32, P, P, P, F, P, P, P, P, SZ, P]),
        "ispa_eps_workspace_size": (SZ, [I32, I32, I32]),
        "ispa_layer_eps": (I32, [I32, I32, I32, P, P, P, P, P, F, P, P, P, SZ, P]),
        "ispa_select_layers": (I32, [I32, P, I32, P, P, P]),
        "ispa_absorb_apply": (I32, [I32, I32, I32, P, I32, P, P, P]),
        "ispa_fit_error_workspace_size": (SZ, [I32, I32, I32]),
        "ispa_fit_error": (I32, [I32, I32, I32, P, P, P, P, P, P, P, P, SZ, P]),
        "ispa_lambda_from_trace": (I32, [I32, I32, P, F, P, P]),
        "ispa_absorb_solve_lambdas": (I32, [I32, I32, I32, P, P, P, P, P, P, P, P, SZ, P]),
        "ispa_absorb_solve_ex": (I32, [I32, I32, I32, P, P, P, F, P, I32, P, P, P, P, SZ,
                                       ctypes.POINTER(SideStreamDesc), P]),
        "ispa_select_layers_below": (I32, [I32, P, ctypes.c_double, I32, P, P, P, P]),
        "ispa_gather_layers": (I32, [I32, I64, P, P, I32, P, P]),
        "ispa_absorb_apply_compact": (I32, [I32, I32, I32, P, I32, P, P, P]),
        "ispa_decomp_attn_fp8k": (I32, [ctypes.POINTER(AttnDesc), P, P, ctypes.POINTER(KvSegmentFp8k), I32, I32]
                                  + [P] * 7 + [SZ, P]),
        "ispa_quantize_fp8_heads_workspace_size": (SZ, [I64, I32]),
        "ispa_quantize_fp8_heads": (I32, [I64, I32, I32, I32, P, P, P, P, SZ, P]),
        "ispa_quantize_fp8_rows": (I32, [I64, I32, I32, P, P, P, P]),
        "ispa_quantize_fp8_cols": (I32, [I32, I32, P, P, P, P]),
        "ispa_w8a8_gemm": (I32, [I64, I32, I32, P, P, P, P, P, P]),
        "ispa_status_string": (ctypes.c_char_p, [I32]),
        "ispa_last_error": (ctypes.c_char_p, []),
        "ispa_version": (I32, []),
        "ispa_device_check": (I32, [I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != ISPA_OK:
        lib = load_library()
        raise IspaError(status, f"{lib.ispa_status_string(status).decode()}: {lib.ispa_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise IspaError(ISPA_E_INVALID_ARG, "tensor is not on the GPU")
    if not t.is_contiguous():
        raise IspaError(ISPA_E_INVALID_ARG, "tensor is not contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ISPA_BF16
    if t.dtype == torch.float32:
        return ISPA_F32
    raise IspaError(ISPA_E_INVALID_ARG, f"unsupported dtype {t.dtype}")


def _expect(t: Optional[torch.Tensor], shape, dtype, name: str) -> None:
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise IspaError(ISPA_E_INVALID_ARG, f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def make_desc(q: torch.Tensor, n_loc: int, n_hist: int, scale: Optional[float]) -> AttnDesc:
    n_q, H, D = q.shape
    return AttnDesc(H, D, n_q, n_loc, n_hist, float(scale if scale is not None else D ** -0.5), _dtype_code(q))


def ispa_decomp_attn_workspace_size(q, n_loc: int, n_hist: int, scale=None) -> int:
    desc = make_desc(q, n_loc, n_hist, scale)
    return int(load_library().ispa_decomp_attn_workspace_size(ctypes.byref(desc)))


def ispa_decomp_attn(q, k_loc, v_loc, k_hist=None, v_hist=None, *, scale=None, o_loc=None, lse_loc=None,
                     o_hist=None, lse_hist=None, o_full=None, lse_full=None, workspace=None, stream=None) -> None:
    """Dual-stream attention of one chunk; writes whichever outputs are given.

    `workspace` (bytes >= ispa_decomp_attn_workspace_size) is needed for o_full with history keys;
    when omitted here, one is allocated through torch for this call."""
    n_q, H, D = q.shape
    n_loc = k_loc.shape[0]
    n_hist = 0 if k_hist is None else k_hist.shape[0]
    for t, n in ((k_loc, "k_loc"), (v_loc, "v_loc")):
        _expect(t, (n_loc, H, D), q.dtype, n)
    if n_hist:
        _expect(k_hist, (n_hist, H, D), q.dtype, "k_hist")
        _expect(v_hist, (n_hist, H, D), q.dtype, "v_hist")
    for t, n in ((o_loc, "o_loc"), (o_hist, "o_hist"), (o_full, "o_full")):
        _expect(t, (n_q, H, D), q.dtype, n)
    for t, n in ((lse_loc, "lse_loc"), (lse_hist, "lse_hist"), (lse_full, "lse_full")):
        _expect(t, (H, n_q), torch.float32, n)
    desc = make_desc(q, n_loc, n_hist, scale)
    lib = load_library()
    if workspace is None and o_full is not None:
        workspace = _workspace(int(lib.ispa_decomp_attn_workspace_size(ctypes.byref(desc))), q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ispa_decomp_attn(ctypes.byref(desc), _ptr(q), _ptr(k_loc), _ptr(v_loc),
                                _ptr(k_hist) if n_hist else None, _ptr(v_hist) if n_hist else None,
                                _ptr(o_loc), _ptr(lse_loc), _ptr(o_hist), _ptr(lse_hist), _ptr(o_full),
                                _ptr(lse_full), _ptr(workspace), ws_bytes, _stream(stream)))


ISPA_NOALLOC_SCRATCH_BYTES = 128 << 20


def ispa_decomp_attn_noalloc(q, k_loc, v_loc, k_hist=None, v_hist=None, *, scale=None, o_loc=None, lse_loc=None,
                             o_hist=None, lse_hist=None, o_full=None, lse_full=None, stream=None) -> None:
    """ispa_decomp_attn with its scratch in the library's static device array: no workspace, nothing
    allocated (n_q * H * D * 4 <= ISPA_NOALLOC_SCRATCH_BYTES; calls overlapping on one GPU race)."""
    n_q, H, D = q.shape
    n_loc = k_loc.shape[0]
    n_hist = 0 if k_hist is None else k_hist.shape[0]
    for t, n in ((k_loc, "k_loc"), (v_loc, "v_loc")):
        _expect(t, (n_loc, H, D), q.dtype, n)
    if n_hist:
        _expect(k_hist, (n_hist, H, D), q.dtype, "k_hist")
        _expect(v_hist, (n_hist, H, D), q.dtype, "v_hist")
    for t, n in ((o_loc, "o_loc"), (o_hist, "o_hist"), (o_full, "o_full")):
        _expect(t, (n_q, H, D), q.dtype, n)
    for t, n in ((lse_loc, "lse_loc"), (lse_hist, "lse_hist"), (lse_full, "lse_full")):
        _expect(t, (H, n_q), torch.float32, n)
    desc = make_desc(q, n_loc, n_hist, scale)
    _check(load_library().ispa_decomp_attn_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k_loc), _ptr(v_loc), _ptr(k_hist) if n_hist else None,
        _ptr(v_hist) if n_hist else None, _ptr(o_loc), _ptr(lse_loc), _ptr(o_hist), _ptr(lse_hist), _ptr(o_full),
        _ptr(lse_full), _stream(stream)))


def _segments(q, loc_segs, hist_segs, o_loc, o_hist, o_full, lse_loc, lse_hist, lse_full):
    """Check shapes; marshal the (k, v) pairs into a KvSegment array."""
    n_q, H, D = q.shape
    segs = list(loc_segs) + list(hist_segs)
    arr = (KvSegment * max(len(segs), 1))()
    n_loc = n_hist = 0
    for i, (k, v) in enumerate(segs):
        n = int(k.shape[0])
        _expect(k, (n, H, D), q.dtype, f"segment {i} k")
        _expect(v, (n, H, D), q.dtype, f"segment {i} v")
        arr[i] = KvSegment(_ptr(k), _ptr(v), n)
        if i < len(loc_segs):
            n_loc += n
        else:
            n_hist += n
    for t, n in ((o_loc, "o_loc"), (o_hist, "o_hist"), (o_full, "o_full")):
        _expect(t, (n_q, H, D), q.dtype, n)
    for t, n in ((lse_loc, "lse_loc"), (lse_hist, "lse_hist"), (lse_full, "lse_full")):
        _expect(t, (H, n_q), torch.float32, n)
    return arr, len(segs), n_loc, n_hist


def ispa_decomp_attn_splitkv_workspace_size(q, n_loc: int, n_hist: int, n_workers: int = 0, scale=None) -> int:
    desc = make_desc(q, n_loc, n_hist, scale)
    return int(load_library().ispa_decomp_attn_splitkv_workspace_size(ctypes.byref(desc), n_workers))


def ispa_decomp_attn_splitkv(q, loc_segs: Sequence, hist_segs: Sequence = (), *, n_workers: int = 0, scale=None,
                             o_loc=None, lse_loc=None, o_hist=None, lse_hist=None, o_full=None, lse_full=None,
                             workspace=None, stream=None) -> None:
    """Split-KV form of ispa_decomp_attn_segments: the (head, query tile, key tile) steps are shared
    evenly by ``n_workers`` workgroups (0 = one per compute unit) and split units are merged through
    their LSE states.  ``workspace`` (bytes >= ispa_decomp_attn_splitkv_workspace_size) is allocated
    through torch for this call when omitted."""
    arr, n_segs, n_loc, n_hist = _segments(q, loc_segs, hist_segs, o_loc, o_hist, o_full, lse_loc, lse_hist,
                                           lse_full)
    desc = make_desc(q, n_loc, n_hist, scale)
    lib = load_library()
    if workspace is None:
        workspace = _workspace(int(lib.ispa_decomp_attn_splitkv_workspace_size(ctypes.byref(desc), n_workers)),
                               q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ispa_decomp_attn_splitkv(ctypes.byref(desc), _ptr(q), arr, n_segs, len(loc_segs), n_workers,
                                        _ptr(o_loc), _ptr(lse_loc), _ptr(o_hist), _ptr(lse_hist), _ptr(o_full),
                                        _ptr(lse_full), _ptr(workspace), ws_bytes, _stream(stream)))


def ispa_decomp_attn_segments(q, loc_segs: Sequence, hist_segs: Sequence = (), *, scale=None, o_loc=None,
                              lse_loc=None, o_hist=None, lse_hist=None, o_full=None, lse_full=None, workspace=None,
                              stream=None) -> None:
    """ispa_decomp_attn over K/V segments: ``loc_segs`` / ``hist_segs`` are sequences of (k, v) pairs,
    each [n_i, H, D] contiguous, attended in place (no concatenation)."""
    arr, n_segs, n_loc, n_hist = _segments(q, loc_segs, hist_segs, o_loc, o_hist, o_full, lse_loc, lse_hist,
                                           lse_full)
    desc = make_desc(q, n_loc, n_hist, scale)
    lib = load_library()
    if workspace is None and o_full is not None:
        workspace = _workspace(int(lib.ispa_decomp_attn_workspace_size(ctypes.byref(desc))), q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ispa_decomp_attn_segments(ctypes.byref(desc), _ptr(q), arr, n_segs, len(loc_segs),
                                         _ptr(o_loc), _ptr(lse_loc), _ptr(o_hist), _ptr(lse_hist), _ptr(o_full),
                                         _ptr(lse_full), _ptr(workspace), ws_bytes, _stream(stream)))


def ispa_full_attn(q, k, v, *, scale=None, o=None, lse=None, stream=None) -> None:
    """One online-softmax pass over all keys of k/v."""
    n_q, H, D = q.shape
    n = k.shape[0]
    _expect(k, (n, H, D), q.dtype, "k")
    _expect(v, (n, H, D), q.dtype, "v")
    _expect(o, (n_q, H, D), q.dtype, "o")
    _expect(lse, (H, n_q), torch.float32, "lse")
    desc = make_desc(q, n, 0, scale)
    lib = load_library()
    _check(lib.ispa_full_attn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(stream)))


def ispa_lse_merge(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor], o_out, lse_out=None,
                   stream=None) -> None:
    """Merge partial (O, LSE) results over disjoint key sets."""
    n = len(o_parts)
    n_q, H, D = o_parts[0].shape
    for o, l in zip(o_parts, lse_parts):
        _expect(o, (n_q, H, D), o_parts[0].dtype, "o_part")
        _expect(l, (H, n_q), torch.float32, "lse_part")
    _expect(o_out, (n_q, H, D), o_parts[0].dtype, "o_out")
    _expect(lse_out, (H, n_q), torch.float32, "lse_out")
    optrs = (ctypes.c_void_p * n)(*[_ptr(o) for o in o_parts])
    lptrs = (ctypes.c_void_p * n)(*[_ptr(l) for l in lse_parts])
    lib = load_library()
    _check(lib.ispa_lse_merge(n, optrs, lptrs, n_q, H, D, _dtype_code(o_parts[0]), _ptr(o_out), _ptr(lse_out),
                              _stream(stream)))


def ispa_gram_workspace_size(n_rows: int, d: int, dtype: torch.dtype) -> int:
    code = ISPA_BF16 if dtype == torch.bfloat16 else ISPA_F32
    return int(load_library().ispa_gram_workspace_size(n_rows, d, code))


def ispa_gram_accum(a_loc, a_full, G, C, E=None, *, accumulate: bool, workspace=None, stream=None) -> None:
    """With D = A_full - A_loc: G (+)= A_loc^T A_loc ; C (+)= A_loc^T D ; E (+)= D^T D (E optional).

    bf16 rows need ``workspace`` (bytes >= ispa_gram_workspace_size); when omitted here, one is allocated
    through torch for this call."""
    n = a_loc.shape[0]
    d = 1
    for s_ in a_loc.shape[1:]:
        d *= int(s_)
    a_loc2 = a_loc.reshape(n, d)
    a_full2 = a_full.reshape(a_full.shape[0], d)
    _expect(a_full2, (n, d), a_loc.dtype, "a_full")
    for t, nm in ((G, "G"), (C, "C"), (E, "E")):
        _expect(t, (d, d), torch.float32, nm)
    lib = load_library()
    if workspace is None:
        workspace = _workspace(int(lib.ispa_gram_workspace_size(n, d, _dtype_code(a_loc))), a_loc.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ispa_gram_accum(n, d, _dtype_code(a_loc), _ptr(a_loc2), _ptr(a_full2), _ptr(G), _ptr(C), _ptr(E),
                               1 if accumulate else 0, _ptr(workspace), ws_bytes, _stream(stream)))


def ispa_absorb_workspace_size(d: int, d_out: int, batch: int) -> int:
    return int(load_library().ispa_absorb_workspace_size(d, d_out, batch))


def ispa_absorb_solve(G, C, W, lam: float, dW, info, *, W_new=None, workspace=None, stream=None) -> None:
    """dW = (G + lam I)^-1 C W per batch entry; G, C [b,d,d] or [d,d]; W, dW [b,d,d_out] or [d,d_out]."""
    G3 = G if G.dim() == 3 else G[None]
    W3 = W if W.dim() == 3 else W[None]
    b, d, _ = G3.shape
    d_out = W3.shape[2]
    _expect(G3, (b, d, d), torch.float32, "G")
    _expect(C if C.dim() == 3 else C[None], (b, d, d), torch.float32, "C")
    _expect(W3, (b, d, d_out), torch.float32, "W")
    _expect(dW if dW.dim() == 3 else dW[None], (b, d, d_out), torch.float32, "dW")
    if W_new is not None:
        _expect(W_new if W_new.dim() == 3 else W_new[None], (b, d, d_out), torch.float32, "W_new")
    _expect(info.reshape(-1), (b,), torch.int32, "info")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    _check(lib.ispa_absorb_solve(d, d_out, b, _ptr(G), _ptr(C), _ptr(W), float(lam), _ptr(dW), _ptr(W_new),
                                 _ptr(info), _ptr(workspace), ws_bytes, _stream(stream)))


def ispa_eps_workspace_size(d: int, d_out: int, batch: int) -> int:
    return int(load_library().ispa_eps_workspace_size(d, d_out, batch))


def ispa_layer_eps(G, C, E, W, dW, lam: float, eps_abs, eps_rel, *, workspace=None, stream=None) -> None:
    """Reconstruction error of each layer from its Gram statistics (float64 outputs [batch])."""
    G3 = G if G.dim() == 3 else G[None]
    W3 = W if W.dim() == 3 else W[None]
    b, d, _ = G3.shape
    d_out = W3.shape[2]
    for t, nm in ((G, "G"), (C, "C"), (E, "E")):
        _expect(t if t.dim() == 3 else t[None], (b, d, d), torch.float32, nm)
    for t, nm in ((W, "W"), (dW, "dW")):
        _expect(t if t.dim() == 3 else t[None], (b, d, d_out), torch.float32, nm)
    _expect(eps_abs.reshape(-1), (b,), torch.float64, "eps_abs")
    _expect(eps_rel.reshape(-1), (b,), torch.float64, "eps_rel")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    _check(lib.ispa_layer_eps(d, d_out, b, _ptr(G), _ptr(C), _ptr(E), _ptr(W), _ptr(dW), float(lam),
                              _ptr(eps_abs), _ptr(eps_rel), _ptr(workspace), ws_bytes, _stream(stream)))


def ispa_select_layers(eps, k: int, selected, rank=None, *, stream=None) -> None:
    """selected[:k] = ids of the k layers with the lowest eps (ties to the lower id, NaN last)."""
    n = eps.numel()
    _expect(eps.reshape(-1), (n,), torch.float64, "eps")
    _expect(selected.reshape(-1), (k,), torch.int32, "selected")
    if rank is not None:
        _expect(rank.reshape(-1), (n,), torch.int32, "rank")
    lib = load_library()
    _check(lib.ispa_select_layers(n, _ptr(eps), int(k), _ptr(selected), _ptr(rank), _stream(stream)))


def ispa_absorb_apply(selected, dW, W, *, stream=None) -> None:
    """W[l] += dW[l] for every layer id l in `selected`; W, dW [n_layers, d, d_out] float32."""
    n, d, d_out = W.shape
    _expect(dW, (n, d, d_out), torch.float32, "dW")
    _expect(W, (n, d, d_out), torch.float32, "W")
    k = selected.numel()
    _expect(selected.reshape(-1), (k,), torch.int32, "selected")
    lib = load_library()
    _check(lib.ispa_absorb_apply(d, d_out, n, _ptr(selected), k, _ptr(dW), _ptr(W), _stream(stream)))


def _as3(t):
    return t if t.dim() == 3 else t[None]


def ispa_fit_error_workspace_size(d: int, d_out: int, batch: int) -> int:
    return int(load_library().ispa_fit_error_workspace_size(d, d_out, batch))


def ispa_fit_error(G, C, E, W, dW, eps_abs, eps_rel, *, workspace=None, stream=None) -> None:
    """||A_loc (W + dW) - A_full W||^2 over the rows summarised by (G, C, E), any dW (None: dW = 0)."""
    G3, W3 = _as3(G), _as3(W)
    b, d, _ = G3.shape
    d_out = W3.shape[2]
    for t, nm in ((G, "G"), (C, "C"), (E, "E")):
        _expect(_as3(t), (b, d, d), torch.float32, nm)
    _expect(W3, (b, d, d_out), torch.float32, "W")
    if dW is not None:
        _expect(_as3(dW), (b, d, d_out), torch.float32, "dW")
    _expect(eps_abs.reshape(-1), (b,), torch.float64, "eps_abs")
    _expect(eps_rel.reshape(-1), (b,), torch.float64, "eps_rel")
    lib = load_library()
    if workspace is None:
        workspace = _workspace(int(lib.ispa_fit_error_workspace_size(d, d_out, b)), G.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ispa_fit_error(d, d_out, b, _ptr(G), _ptr(C), _ptr(E), _ptr(W), _ptr(dW), _ptr(eps_abs),
                              _ptr(eps_rel), _ptr(workspace), ws_bytes, _stream(stream)))


def ispa_lambda_from_trace(G, lam_scale: float, lambdas, *, stream=None) -> None:
    """lambdas[b] = lam_scale * tr(G_b) / d (float32 [batch])."""
    G3 = _as3(G)
    b, d, _ = G3.shape
    _expect(G3, (b, d, d), torch.float32, "G")
    _expect(lambdas.reshape(-1), (b,), torch.float32, "lambdas")
    _check(load_library().ispa_lambda_from_trace(d, b, _ptr(G), float(lam_scale), _ptr(lambdas), _stream(stream)))


def ispa_absorb_solve_lambdas(G, C, W, lambdas, dW, info, *, W_new=None, workspace=None, stream=None) -> None:
    """ispa_absorb_solve with a per-layer lambda (device float32 [batch])."""
    G3, W3 = _as3(G), _as3(W)
    b, d, _ = G3.shape
    d_out = W3.shape[2]
    _expect(G3, (b, d, d), torch.float32, "G")
    _expect(_as3(C), (b, d, d), torch.float32, "C")
    _expect(W3, (b, d, d_out), torch.float32, "W")
    _expect(_as3(dW), (b, d, d_out), torch.float32, "dW")
    if W_new is not None:
        _expect(_as3(W_new), (b, d, d_out), torch.float32, "W_new")
    _expect(lambdas.reshape(-1), (b,), torch.float32, "lambdas")
    _expect(info.reshape(-1), (b,), torch.int32, "info")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ispa_absorb_solve_lambdas(d, d_out, b, _ptr(G), _ptr(C), _ptr(W), _ptr(lambdas), _ptr(dW),
                                                    _ptr(W_new), _ptr(info), _ptr(workspace), ws_bytes,
                                                    _stream(stream)))


ISPA_ABSORB_NO_REFINE = 1


class SideStream:
    """A caller-owned second stream and its fork / join events for ispa_absorb_solve_ex (created here,
    outside any hot-path call, and kept alive by this object)."""

    def __init__(self, device=None):
        self.stream = torch.cuda.Stream(device=device)
        self.ev_fork = torch.cuda.Event()
        self.ev_join = torch.cuda.Event()
        # torch creates an event's handle on its first record
        self.ev_fork.record(self.stream)
        self.ev_join.record(self.stream)
        self.desc = SideStreamDesc(self.stream.cuda_stream, self.ev_fork.cuda_event, self.ev_join.cuda_event)


def ispa_absorb_solve_ex(G, C, W, lam: float, dW, info, *, lambdas=None, refine: bool = True, W_new=None,
                         workspace=None, side: Optional[SideStream] = None, stream=None) -> None:
    """ispa_absorb_solve with a per-layer lambda (``lambdas``, device float32), the refinement optional and
    R = C W on a caller-owned side stream (``side``) beside the factorisation."""
    G3, W3 = _as3(G), _as3(W)
    b, d, _ = G3.shape
    d_out = W3.shape[2]
    _expect(G3, (b, d, d), torch.float32, "G")
    _expect(_as3(C), (b, d, d), torch.float32, "C")
    _expect(W3, (b, d, d_out), torch.float32, "W")
    _expect(_as3(dW), (b, d, d_out), torch.float32, "dW")
    if W_new is not None:
        _expect(_as3(W_new), (b, d, d_out), torch.float32, "W_new")
    if lambdas is not None:
        _expect(lambdas.reshape(-1), (b,), torch.float32, "lambdas")
    _expect(info.reshape(-1), (b,), torch.int32, "info")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ispa_absorb_solve_ex(d, d_out, b, _ptr(G), _ptr(C), _ptr(W), float(lam), _ptr(lambdas),
                                               0 if refine else ISPA_ABSORB_NO_REFINE, _ptr(dW), _ptr(W_new),
                                               _ptr(info), _ptr(workspace), ws_bytes,
                                               None if side is None else ctypes.byref(side.desc), _stream(stream)))


def ispa_select_layers_below(eps, tau: float, k_max: int, selected, count, rank=None, *, stream=None) -> None:
    """The layers with eps <= tau, lowest first, at most k_max; count[0] = how many."""
    n = eps.numel()
    _expect(eps.reshape(-1), (n,), torch.float64, "eps")
    _expect(selected.reshape(-1), (k_max,), torch.int32, "selected")
    _expect(count.reshape(-1), (1,), torch.int32, "count")
    if rank is not None:
        _expect(rank.reshape(-1), (n,), torch.int32, "rank")
    _check(load_library().ispa_select_layers_below(n, _ptr(eps), float(tau), int(k_max), _ptr(selected), _ptr(count),
                                                   _ptr(rank), _stream(stream)))


def ispa_gather_layers(src, selected, dst, *, stream=None) -> None:
    """dst[s] = src[selected[s]]; src [n_layers, ...], dst [k, ...] float32."""
    n = src.shape[0]
    k = selected.numel()
    per = src[0].numel() if n else 0
    _expect(src.reshape(n, -1), (n, per), torch.float32, "src")
    _expect(dst.reshape(k, -1) if k else dst, (k, per) if k else tuple(dst.shape), torch.float32, "dst")
    _check(load_library().ispa_gather_layers(n, per, _ptr(src), _ptr(selected), k, _ptr(dst), _stream(stream)))


def ispa_absorb_apply_compact(selected, dW, W, *, stream=None) -> None:
    """W[selected[s]] += dW[s]; W [n_layers, d, d_out], dW [k, d, d_out] float32."""
    n, d, d_out = W.shape
    k = selected.numel()
    _expect(dW, (k, d, d_out), torch.float32, "dW")
    _check(load_library().ispa_absorb_apply_compact(d, d_out, n, _ptr(selected), k, _ptr(dW), _ptr(W),
                                                    _stream(stream)))


def ispa_quantize_fp8_heads_workspace_size(n_rows: int, heads: int) -> int:
    return int(load_library().ispa_quantize_fp8_heads_workspace_size(n_rows, heads))


def ispa_quantize_fp8_heads(x, x8, scale, *, workspace=None, stream=None) -> None:
    """x [n, H, D] (bf16 / float32) -> codes x8 (uint8, same shape) and scale [H] (one per head)."""
    n, H, D = x.shape
    _expect(x8, (n, H, D), torch.uint8, "x8")
    _expect(scale.reshape(-1), (H,), torch.float32, "scale")
    lib = load_library()
    if workspace is None:
        workspace = _workspace(int(lib.ispa_quantize_fp8_heads_workspace_size(n, H)), x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ispa_quantize_fp8_heads(n, H, D, _dtype_code(x), _ptr(x), _ptr(x8), _ptr(scale), _ptr(workspace),
                                       ws_bytes, _stream(stream)))


def ispa_quantize_fp8_rows(x, x8, scale, *, stream=None) -> None:
    """x [n, d] -> codes x8 [n, d] (uint8) with scale [n] (one per row)."""
    n = x.shape[0]
    d = x[0].numel() if n else int(x.shape[-1])
    _expect(x8.reshape(n, -1) if n else x8, (n, d) if n else tuple(x8.shape), torch.uint8, "x8")
    _expect(scale.reshape(-1), (n,), torch.float32, "scale")
    _check(load_library().ispa_quantize_fp8_rows(n, d, _dtype_code(x), _ptr(x), _ptr(x8), _ptr(scale),
                                                 _stream(stream)))


def ispa_quantize_fp8_cols(W, w8t, scale, *, stream=None) -> None:
    """W [d, d_out] float32 -> codes w8t [d_out, d] (uint8, transposed) with scale [d_out] (one per column)."""
    d, d_out = W.shape
    _expect(W, (d, d_out), torch.float32, "W")
    _expect(w8t, (d_out, d), torch.uint8, "w8t")
    _expect(scale.reshape(-1), (d_out,), torch.float32, "scale")
    _check(load_library().ispa_quantize_fp8_cols(d, d_out, _ptr(W), _ptr(w8t), _ptr(scale), _stream(stream)))


def ispa_w8a8_gemm(a8, a_scale, w8t, w_scale, y, *, stream=None) -> None:
    """y [n, d_out] bf16 = (a8 [n, d] . w8t [d_out, d]^T) * a_scale[row] * w_scale[col]."""
    n, d = a8.shape
    d_out = w8t.shape[0]
    _expect(a8, (n, d), torch.uint8, "a8")
    _expect(w8t, (d_out, d), torch.uint8, "w8t")
    _expect(a_scale.reshape(-1), (n,), torch.float32, "a_scale")
    _expect(w_scale.reshape(-1), (d_out,), torch.float32, "w_scale")
    _expect(y, (n, d_out), torch.bfloat16, "y")
    _check(load_library().ispa_w8a8_gemm(n, d, d_out, _ptr(a8), _ptr(a_scale), _ptr(w8t), _ptr(w_scale), _ptr(y),
                                         _stream(stream)))


def ispa_decomp_attn_fp8k(q8, q_scale, loc_segs: Sequence, hist_segs: Sequence = (), *, scale=None, o_loc=None,
                          lse_loc=None, o_hist=None, lse_hist=None, o_full=None, lse_full=None, workspace=None,
                          stream=None) -> None:
    """Decomposable attention with fp8 queries and keys: q8 [n_q, H, D] codes (scale q_scale [H]); segments
    are (k8, k_scale, v) triples (k8 uint8 codes, k_scale [H] float32, v bf16).  Outputs bf16 / float32."""
    n_q, H, D = q8.shape
    _expect(q8, (n_q, H, D), torch.uint8, "q8")
    _expect(q_scale.reshape(-1), (H,), torch.float32, "q_scale")
    segs = list(loc_segs) + list(hist_segs)
    arr = (KvSegmentFp8k * max(len(segs), 1))()
    n_loc = n_hist = 0
    for i, (k8, ks, v) in enumerate(segs):
        n = int(k8.shape[0])
        _expect(k8, (n, H, D), torch.uint8, f"segment {i} k8")
        _expect(ks.reshape(-1), (H,), torch.float32, f"segment {i} k_scale")
        _expect(v, (n, H, D), torch.bfloat16, f"segment {i} v")
        arr[i] = KvSegmentFp8k(_ptr(k8), _ptr(ks), _ptr(v), n)
        if i < len(loc_segs):
            n_loc += n
        else:
            n_hist += n
    for t, nm in ((o_loc, "o_loc"), (o_hist, "o_hist"), (o_full, "o_full")):
        _expect(t, (n_q, H, D), torch.bfloat16, nm)
    for t, nm in ((lse_loc, "lse_loc"), (lse_hist, "lse_hist"), (lse_full, "lse_full")):
        _expect(t, (H, n_q), torch.float32, nm)
    desc = AttnDesc(H, D, n_q, n_loc, n_hist, float(scale if scale is not None else D ** -0.5), ISPA_BF16)
    lib = load_library()
    if workspace is None and o_full is not None:
        workspace = _workspace(int(lib.ispa_decomp_attn_workspace_size(ctypes.byref(desc))), q8.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ispa_decomp_attn_fp8k(ctypes.byref(desc), _ptr(q8), _ptr(q_scale), arr, len(segs), len(loc_segs),
                                     _ptr(o_loc), _ptr(lse_loc), _ptr(o_hist), _ptr(lse_hist), _ptr(o_full),
                                     _ptr(lse_full), _ptr(workspace), ws_bytes, _stream(stream)))


def ispa_version() -> int:
    return int(load_library().ispa_version())


def ispa_device_check(device: int = 0) -> None:
    _check(load_library().ispa_device_check(device))


def workspace(nbytes: int, device=None) -> Optional[torch.Tensor]:
    """A caller-owned device workspace of at least nbytes (None when 0)."""
    return _workspace(nbytes, device)


def _workspace(nbytes: int, device=None) -> Optional[torch.Tensor]:
    if nbytes <= 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
