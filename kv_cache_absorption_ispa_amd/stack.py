"""A stack of attention layers through warmup, transition and post-absorb chunks.

Source: "Technical Summary: Instance-Specific Parametric Absorption (ISPA) for
Memory-Efficient Video Generation", section 2 "Methodology": step 1 (every
layer runs the dual-stream warmup and collects A_loc / A_full), step 2 (closed
form absorb), step 3 (the converted layers use W + dW, drop their history KV
and attend locally from then on) and "Dynamic Layer Selection" (all layers are
ranked by reconstruction error; the lowest-error ones are converted).

This module is host orchestration only: it owns the per-layer device state
(stacked G, C, E, W, dW) and issues the library's calls; every arithmetic
step runs in the HIP kernels behind the C ABI.  Reading used for the ranking by
default: every layer is solved (batched), its post-fit error eps_rel comes from
the Gram statistics, and the k lowest (ties to the lower layer index) are
converted.  The pages leave the error, lambda and k open; the other readings:

* ``selection="prefit"``: rank by the error before the fit, ||(A_full - A_loc) W||^2,
  and solve only the chosen layers (gathered into a compact batch);
* ``selection="heldout"``: rows passed with ``heldout=True`` (say the last warmup
  chunk) are kept out of the fit; layers are ranked by the error of their fitted
  dW on those rows;
* ``lam_policy="trace"``: lambda_l = lam * tr(G_l) / d instead of lam;
* ``threshold=tau``: convert every layer with eps_rel <= tau, at most n_convert.
"""
from __future__ import annotations

import contextlib
import functools
from typing import List, Optional

import torch

from . import ispa


def _on_stack_stream(method):
    """Run a LayerStack method with its stream as torch's current stream: the library calls are then
    enqueued on it, temporaries come from that stream's pool (freed only behind its work), and host
    reads of device values (the converted set) wait for it."""

    @functools.wraps(method)
    def wrapper(self, *args, **kwargs):
        with self._stream_ctx():
            return method(self, *args, **kwargs)

    return wrapper


class LayerStack:
    """Per-layer state of an n_layers stack of attention layers with the same shape.

    ``W`` is the stacked output-projection weight [n_layers, d, d_out] (float32,
    device); it is updated in place for the converted layers at the transition.
    """

    SELECTIONS = ("postfit", "prefit", "heldout")
    LAM_POLICIES = ("absolute", "trace")

    def __init__(self, W: torch.Tensor, heads: int, head_dim: int, n_q: int, lam: float, n_convert: int,
                 dtype: torch.dtype = torch.bfloat16, stream=None, selection: str = "postfit",
                 lam_policy: str = "absolute", threshold: Optional[float] = None):
        if W.dim() != 3 or W.dtype != torch.float32 or not W.is_cuda:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "W must be a [n_layers, d, d_out] float32 device tensor")
        self.n_layers, self.d, self.d_out = (int(s) for s in W.shape)
        if self.d != heads * head_dim:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "W's d must equal heads * head_dim")
        if not 0 <= n_convert <= self.n_layers:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "n_convert must be in [0, n_layers]")
        if selection not in self.SELECTIONS or lam_policy not in self.LAM_POLICIES:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "unknown selection or lambda policy")
        if threshold is not None and not threshold == threshold:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "threshold is NaN")
        self.selection, self.lam_policy, self.threshold = selection, lam_policy, threshold
        self.heads, self.head_dim, self.n_q = heads, head_dim, n_q
        self.lam = float(lam)
        self.n_convert = n_convert
        self.dtype = dtype
        self.stream = stream
        dev = W.device
        L, d, do = self.n_layers, self.d, self.d_out
        self.W = W
        f32 = dict(dtype=torch.float32, device=dev)
        self.G = torch.zeros(L, d, d, **f32)
        self.C = torch.zeros(L, d, d, **f32)
        self.E = torch.zeros(L, d, d, **f32)
        self.dW = torch.zeros(L, d, do, **f32)
        self.info = torch.zeros(L, dtype=torch.int32, device=dev)
        self.eps_abs = torch.zeros(L, dtype=torch.float64, device=dev)
        self.eps_rel = torch.zeros(L, dtype=torch.float64, device=dev)
        self.selected = torch.zeros(max(n_convert, 1), dtype=torch.int32, device=dev)[:n_convert]
        self.rank = torch.zeros(L, dtype=torch.int32, device=dev)
        self.count = torch.zeros(1, dtype=torch.int32, device=dev)
        self.lambdas = torch.full((L,), self.lam, **f32)
        if selection == "heldout":
            self.G_h = torch.zeros(L, d, d, **f32)
            self.C_h = torch.zeros(L, d, d, **f32)
            self.E_h = torch.zeros(L, d, d, **f32)
            self.heldout_seen = [0] * L
        self.dW_compact: Optional[torch.Tensor] = None  # prefit: dW of the chosen layers, selection order
        self.info_compact: Optional[torch.Tensor] = None
        self.chunks_seen = [0] * L
        self.converted: Optional[List[int]] = None  # host copy after the transition
        # workspaces, sized once
        self._gram_ws = None
        self._attn_ws = None
        with self._stream_ctx():
            self._absorb_ws = ispa.workspace(ispa.ispa_absorb_workspace_size(d, do, L), dev)
            self._eps_ws = ispa.workspace(max(ispa.ispa_fit_error_workspace_size(d, do, L),
                                              ispa.ispa_eps_workspace_size(d, do, L)), dev)
        # R = C W of the absorb solves runs on this second stream beside the factorisation (owned here,
        # created once, outside the hot path)
        self.side = ispa.SideStream(dev)

    def _stream_ctx(self):
        return torch.cuda.stream(self.stream) if self.stream is not None else contextlib.nullcontext()

    def reset(self) -> None:
        """Start a new warmup with the same buffers (W is the caller's; restore it first if needed)."""
        self.chunks_seen = [0] * self.n_layers
        if self.selection == "heldout":
            self.heldout_seen = [0] * self.n_layers
        self.converted = None
        self.dW_compact = self.info_compact = None

    # ------------------------------------------------------------------ warmup
    @_on_stack_stream
    def warmup_chunk(self, layer: int, q, k_loc, v_loc, k_hist, v_hist, o_loc, o_full,
                     lse_loc=None, lse_full=None, heldout: bool = False) -> None:
        """Dual-stream attention of one chunk of `layer`, then its rows into the layer's G, C, E.

        ``o_loc`` / ``o_full`` [n_q, H, D] receive A_loc / A_full of this chunk."""
        if self.converted is not None:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "warmup is over (transition already ran)")
        n_hist = 0 if k_hist is None else int(k_hist.shape[0])
        need = ispa.ispa_decomp_attn_workspace_size(q, int(k_loc.shape[0]), n_hist)
        if need and (self._attn_ws is None or self._attn_ws.numel() < need):
            self._attn_ws = ispa.workspace(need, q.device)
        ispa.ispa_decomp_attn(q, k_loc, v_loc, k_hist, v_hist, o_loc=o_loc, lse_loc=lse_loc, o_full=o_full,
                              lse_full=lse_full, workspace=self._attn_ws)
        self.accumulate_rows(layer, o_loc, o_full, heldout=heldout)

    @_on_stack_stream
    def accumulate_rows(self, layer: int, a_loc, a_full, heldout: bool = False) -> None:
        """Add warmup rows computed elsewhere ([n, d] or [n, H, D]) to the layer's G, C, E (or, with
        ``heldout`` under selection="heldout", to the held-out statistics the ranking is measured on)."""
        if self.converted is not None:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "warmup is over (transition already ran)")
        if heldout and self.selection != "heldout":
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "held-out rows need selection='heldout'")
        n_rows = int(a_loc.shape[0])
        need = ispa.ispa_gram_workspace_size(n_rows, self.d, a_loc.dtype)
        if need and (self._gram_ws is None or self._gram_ws.numel() < need):
            self._gram_ws = ispa.workspace(need, a_loc.device)
        if heldout:
            ispa.ispa_gram_accum(a_loc, a_full, self.G_h[layer], self.C_h[layer], self.E_h[layer],
                                 accumulate=self.heldout_seen[layer] > 0, workspace=self._gram_ws)
            self.heldout_seen[layer] += 1
            return
        ispa.ispa_gram_accum(a_loc, a_full, self.G[layer], self.C[layer], self.E[layer],
                             accumulate=self.chunks_seen[layer] > 0, workspace=self._gram_ws)
        self.chunks_seen[layer] += 1

    # -------------------------------------------------------------- transition
    @_on_stack_stream
    def transition(self) -> List[int]:
        """Solve every layer (batched), rank by eps_rel, convert the n_convert lowest: W += dW there.

        Returns the converted layer ids (lowest error first); this is the one host sync of the
        transition (the host needs the set to launch the post-absorb chunks)."""
        if self.converted is not None:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "transition already ran")
        if min(self.chunks_seen) == 0:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "every layer needs at least one warmup chunk")
        if self.selection == "heldout" and min(self.heldout_seen) == 0:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "every layer needs held-out rows")
        self.solve_and_rank()
        return self.convert()

    def _select(self) -> None:
        if self.threshold is None:
            ispa.ispa_select_layers(self.eps_rel, self.n_convert, self.selected, self.rank)
        else:
            ispa.ispa_select_layers_below(self.eps_rel, self.threshold, self.n_convert, self.selected, self.count,
                                          self.rank)

    def _solve(self, G, C, W, dW, info, lambdas, workspace) -> None:
        if self.lam_policy == "trace":
            ispa.ispa_lambda_from_trace(G, self.lam, lambdas)
            ispa.ispa_absorb_solve_ex(G, C, W, 0.0, dW, info, lambdas=lambdas, workspace=workspace, side=self.side)
        else:
            ispa.ispa_absorb_solve_ex(G, C, W, self.lam, dW, info, workspace=workspace, side=self.side)

    @_on_stack_stream
    def solve_and_rank(self) -> None:
        """The transition's device work before the weights change: solves, errors, ranking.

        prefit: errors at dW = 0 and ranking first; the chosen layers are solved in convert()."""
        if self.selection == "prefit":
            ispa.ispa_fit_error(self.G, self.C, self.E, self.W, None, self.eps_abs, self.eps_rel,
                                workspace=self._eps_ws)
            self._select()
            return
        self._solve(self.G, self.C, self.W, self.dW, self.info, self.lambdas, self._absorb_ws)
        if self.selection == "heldout":
            ispa.ispa_fit_error(self.G_h, self.C_h, self.E_h, self.W, self.dW, self.eps_abs, self.eps_rel,
                                workspace=self._eps_ws)
        elif self.lam_policy == "trace":  # per-layer lambda: the general form (no normal-equation shortcut)
            ispa.ispa_fit_error(self.G, self.C, self.E, self.W, self.dW, self.eps_abs, self.eps_rel,
                                workspace=self._eps_ws)
        else:
            ispa.ispa_layer_eps(self.G, self.C, self.E, self.W, self.dW, self.lam, self.eps_abs, self.eps_rel,
                                workspace=self._eps_ws)
        self._select()

    @_on_stack_stream
    def convert(self) -> List[int]:
        """W += dW on the selected layers; returns their ids (a host sync)."""
        if self.converted is not None:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "layers already converted")
        k = self.n_convert if self.threshold is None else int(self.count.item())
        sel = self.selected[:k]
        if self.selection == "prefit":
            # solve only the chosen layers: gather their statistics and weights into a compact batch
            d, do = self.d, self.d_out
            dev = self.W.device
            f32 = dict(dtype=torch.float32, device=dev)
            if k:
                Gs, Cs = torch.empty(k, d, d, **f32), torch.empty(k, d, d, **f32)
                Ws, dWs = torch.empty(k, d, do, **f32), torch.empty(k, d, do, **f32)
                ispa.ispa_gather_layers(self.G, sel, Gs)
                ispa.ispa_gather_layers(self.C, sel, Cs)
                ispa.ispa_gather_layers(self.W, sel, Ws)
                info = torch.empty(k, dtype=torch.int32, device=dev)
                lambdas = torch.empty(k, **f32)
                ws = ispa.workspace(ispa.ispa_absorb_workspace_size(d, do, k), dev)
                self._solve(Gs, Cs, Ws, dWs, info, lambdas, ws)
                ispa.ispa_absorb_apply_compact(sel, dWs, self.W)
                self.dW_compact, self.info_compact = dWs, info
        else:
            ispa.ispa_absorb_apply(sel, self.dW, self.W)
        self.converted = [int(x) for x in sel.cpu().tolist()]
        return self.converted

    # ------------------------------------------------------------- post-absorb
    def is_converted(self, layer: int) -> bool:
        if self.converted is None:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "transition has not run")
        return layer in self.converted

    @_on_stack_stream
    def post_chunk(self, layer: int, q, k_loc, v_loc, k_hist, v_hist, o_full, lse_full=None) -> None:
        """Attention of one post-absorb chunk: local keys only for a converted layer (its history is
        evicted; ``k_hist`` / ``v_hist`` are ignored and may be None), all keys otherwise.
        ``o_full`` receives the layer's attention output."""
        if self.is_converted(layer):
            ispa.ispa_decomp_attn(q, k_loc, v_loc, None, None, o_full=o_full, lse_full=lse_full)
            return
        need = ispa.ispa_decomp_attn_workspace_size(q, int(k_loc.shape[0]), int(k_hist.shape[0]))
        if need and (self._attn_ws is None or self._attn_ws.numel() < need):
            self._attn_ws = ispa.workspace(need, q.device)
        ispa.ispa_decomp_attn(q, k_loc, v_loc, k_hist, v_hist, o_full=o_full, lse_full=lse_full,
                              workspace=self._attn_ws)

    # ------------------------------------------------------- streaming K/V cache
    def _attn_ws_for(self, q, n_loc: int, n_hist: int):
        need = ispa.ispa_decomp_attn_workspace_size(q, n_loc, n_hist)
        if need and (self._attn_ws is None or self._attn_ws.numel() < need):
            self._attn_ws = ispa.workspace(need, q.device)
        return self._attn_ws

    @_on_stack_stream
    def warmup_chunk_cached(self, layer: int, q, cache, o_loc, o_full, heldout: bool = False) -> None:
        """warmup_chunk with the keys taken from a StreamingKVCache: the layer's sink and current slot
        (local) and its history runs, attended in place.  The caller writes the chunk's K/V into
        ``cache.current(layer)`` before and calls ``cache.commit(layer)`` after."""
        if self.converted is not None:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "warmup is over (transition already ran)")
        loc, hist = cache.segments(layer)
        n_loc = sum(int(k.shape[0]) for k, _ in loc)
        n_hist = sum(int(k.shape[0]) for k, _ in hist)
        ispa.ispa_decomp_attn_segments(q, loc, hist, o_loc=o_loc, o_full=o_full,
                                       workspace=self._attn_ws_for(q, n_loc, n_hist))
        self.accumulate_rows(layer, o_loc, o_full, heldout=heldout)

    @_on_stack_stream
    def post_chunk_cached(self, layer: int, q, cache, o_full, lse_full=None) -> None:
        """Attention of a post-absorb chunk from the cache (a converted layer's cache holds no history
        once evict_converted ran, so it attends locally)."""
        if self.converted is None:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "transition has not run")
        loc, hist = cache.segments(layer)
        if self.is_converted(layer) and hist:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "converted layer still holds history (evict_converted)")
        n_loc = sum(int(k.shape[0]) for k, _ in loc)
        n_hist = sum(int(k.shape[0]) for k, _ in hist)
        ispa.ispa_decomp_attn_segments(q, loc, hist, o_full=o_full, lse_full=lse_full,
                                       workspace=self._attn_ws_for(q, n_loc, n_hist))

    def evict_converted(self, cache) -> int:
        """Drop the converted layers' history K/V from the cache; returns the bytes released."""
        if self.converted is None:
            raise ispa.IspaError(ispa.ISPA_E_INVALID_ARG, "transition has not run")
        before = cache.resident_bytes()
        for layer in self.converted:
            cache.evict(layer)
        return before - cache.resident_bytes()

    def evicted_kv_bytes(self, n_hist: int) -> int:
        """History K and V bytes the converted layers no longer hold (n_hist keys per layer)."""
        if self.converted is None:
            return 0
        elt = 2 if self.dtype == torch.bfloat16 else 4
        return len(self.converted) * 2 * n_hist * self.heads * self.head_dim * elt
