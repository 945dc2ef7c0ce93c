"""Streaming K/V cache of a chunk-wise generation, handed to the attention as segment lists.

Source: "Technical Summary: Instance-Specific Parametric Absorption (ISPA) for
Memory-Efficient Video Generation", section 2 "Methodology": step 1 (the local
stream sees the sink tokens and the current chunk, the full stream the whole
context generated so far), step 3 (a converted layer evicts its history K/V
and keeps attending locally).  The video is generated chunk after chunk, so the
history of chunk c is the K/V of the chunks before it.

Layout per layer (device memory, allocated once):

* ``sink``  [n_sink, H, D] K and V: the fixed sink tokens (written once).
* ``ring``  [(max_hist_chunks + 1) * chunk_tokens, H, D] K and V: one slot per
  chunk.  ``max_hist_chunks`` slots hold the history, oldest first from
  ``head`` (wrapping), and the free slot after them takes the current chunk.
  The model writes the current chunk's K/V straight into that slot
  (:meth:`current`), so nothing is concatenated or copied: the attention call
  gets the sink, the slot and the history's one or two contiguous runs as
  segments.  :meth:`commit` turns the slot into history; once the history
  holds ``max_hist_chunks`` chunks the oldest is dropped (a rolling window; the
  pages keep the whole context, which is ``max_hist_chunks`` >= the number of
  chunks generated).
* A converted layer (:meth:`evict`) gives back its ring and keeps one chunk
  slot: from then on its segment list is the sink and the current chunk only.

Host bookkeeping only: the attention runs in the library's kernels
(``ispa_decomp_attn_segments``); torch provides the device memory.
"""
from __future__ import annotations

from typing import List, Tuple

import torch

Seg = Tuple[torch.Tensor, torch.Tensor]


class StreamingKVCache:
    def __init__(self, n_layers: int, heads: int, head_dim: int, n_sink: int, chunk_tokens: int,
                 max_hist_chunks: int, dtype: torch.dtype = torch.bfloat16, device="cuda"):
        if n_layers < 1 or heads < 1 or head_dim < 1 or n_sink < 0 or chunk_tokens < 1 or max_hist_chunks < 0:
            raise ValueError("bad cache shape")
        self.n_layers, self.heads, self.head_dim = n_layers, heads, head_dim
        self.n_sink, self.chunk_tokens, self.max_hist_chunks = n_sink, chunk_tokens, max_hist_chunks
        self.dtype, self.device = dtype, torch.device(device)
        self.n_slots = max_hist_chunks + 1
        H, D = heads, head_dim
        kw = dict(dtype=dtype, device=self.device)
        self.sink_k = [torch.empty(n_sink, H, D, **kw) for _ in range(n_layers)]
        self.sink_v = [torch.empty(n_sink, H, D, **kw) for _ in range(n_layers)]
        self.ring_k = [torch.empty(self.n_slots * chunk_tokens, H, D, **kw) for _ in range(n_layers)]
        self.ring_v = [torch.empty(self.n_slots * chunk_tokens, H, D, **kw) for _ in range(n_layers)]
        self.head = [0] * n_layers    # ring slot of the oldest history chunk
        self.count = [0] * n_layers   # history chunks held
        self.evicted = [False] * n_layers
        self.chunks_committed = [0] * n_layers

    # ------------------------------------------------------------------ slots
    def _slot(self, layer: int, slot: int) -> Seg:
        ct = self.chunk_tokens
        return self.ring_k[layer][slot * ct:(slot + 1) * ct], self.ring_v[layer][slot * ct:(slot + 1) * ct]

    def sink(self, layer: int) -> Seg:
        """Views of the layer's sink K and V (write them once, before the first chunk)."""
        return self.sink_k[layer], self.sink_v[layer]

    def current(self, layer: int) -> Seg:
        """Views the current chunk's K and V are written into ([chunk_tokens, H, D] each)."""
        if self.evicted[layer]:
            return self._slot(layer, 0)
        return self._slot(layer, (self.head[layer] + self.count[layer]) % self.n_slots)

    def write_current(self, layer: int, k: torch.Tensor, v: torch.Tensor) -> None:
        """Copy K/V computed elsewhere into the current slot (a device copy)."""
        ck, cv = self.current(layer)
        ck.copy_(k)
        cv.copy_(v)

    # --------------------------------------------------------------- segments
    def history_runs(self, layer: int) -> List[Tuple[int, int]]:
        """The history as at most two (first slot, slots) runs of the ring, oldest first."""
        if self.evicted[layer] or self.count[layer] == 0:
            return []
        h, c, n = self.head[layer], self.count[layer], self.n_slots
        if h + c <= n:
            return [(h, c)]
        return [(h, n - h), (0, h + c - n)]

    def segments(self, layer: int) -> Tuple[List[Seg], List[Seg]]:
        """(local segments, history segments) of the current chunk: sink then chunk, history oldest first."""
        loc: List[Seg] = []
        if self.n_sink > 0:
            loc.append(self.sink(layer))
        loc.append(self.current(layer))
        ct = self.chunk_tokens
        hist = [(self.ring_k[layer][s * ct:(s + n) * ct], self.ring_v[layer][s * ct:(s + n) * ct])
                for s, n in self.history_runs(layer)]
        return loc, hist

    def history_tokens(self, layer: int) -> int:
        return 0 if self.evicted[layer] else self.count[layer] * self.chunk_tokens

    # ------------------------------------------------------------- lifecycle
    def commit(self, layer: int) -> None:
        """The current chunk is done: it joins the history (oldest dropped beyond the window)."""
        self.chunks_committed[layer] += 1
        if self.evicted[layer]:
            return
        if self.max_hist_chunks == 0:
            return
        self.count[layer] += 1
        if self.count[layer] > self.max_hist_chunks:
            self.head[layer] = (self.head[layer] + 1) % self.n_slots
            self.count[layer] -= 1

    def evict(self, layer: int) -> None:
        """Drop the layer's history K/V (a converted layer); one chunk slot stays for its current chunk."""
        if self.evicted[layer]:
            return
        H, D = self.heads, self.head_dim
        kw = dict(dtype=self.dtype, device=self.device)
        self.ring_k[layer] = torch.empty(self.chunk_tokens, H, D, **kw)
        self.ring_v[layer] = torch.empty(self.chunk_tokens, H, D, **kw)
        self.evicted[layer] = True
        self.head[layer] = self.count[layer] = 0

    def resident_bytes(self, layer: int | None = None) -> int:
        """Device bytes of K/V held (sink + ring) for one layer or all."""
        layers = range(self.n_layers) if layer is None else [layer]
        elt = torch.empty(0, dtype=self.dtype).element_size()
        tot = 0
        for l in layers:
            rows = self.sink_k[l].shape[0] + self.ring_k[l].shape[0]
            tot += 2 * rows * self.heads * self.head_dim * elt
        return tot
