"""Host model of the attention kernel's lazy rescale, for choosing and checking test inputs.

The bf16 kernel walks a branch's keys in tiles of 128 (in segment order, each segment ending in its
own ragged tile; a split-KV piece starts a fresh state at its first tile).  It keeps a reference
maximum m of the log2-domain scores c2 * s (c2 = scale * log2 e) and raises it only when a tile's
maximum beats it by more than 8, for all 32 queries of a wave at once; the accumulator and the row
sum are then multiplied by alpha = 2^(m_old - m_new).  At a branch's first tile m_old = -inf and
alpha = 0; at any later tile 0 < alpha < 1.

``rescale_events`` counts the (head, query) pairs whose reference moves at a later tile with a
margin (so float32 rounding on the GPU cannot change the decision).  ``lazy_branch`` runs the same
recurrence in float64 with optional planted mistakes; it exists to show that inputs which trigger
such moves make a wrong rescale fail the parity gates (see tests/test_rescale_cases.py).
"""
from __future__ import annotations

import numpy as np

TILE = 128
THRESH = 8.0
LOG2E = 1.4426950408889634


def tile_bounds(seg_rows):
    """[start, end) of the key tiles of a branch given as consecutive segments of these sizes."""
    out, base = [], 0
    for n in seg_rows:
        for t in range(0, n, TILE):
            out.append((base + t, base + min(n, t + TILE)))
        base += n
    return out


def scores_log2(q, k, scale):
    """c2 * <q, k> per head: [H, n_q, n_k] float64 (q [n_q, H, D], k [n_k, H, D])."""
    return np.einsum("qhd,khd->hqk", q, k) * (scale * LOG2E)


def rescale_events(q, k, scale, seg_rows=None, margin=1.0):
    """(head, query) pairs whose reference maximum is raised at a non-first tile of the branch by more
    than THRESH + margin (so the kernel certainly rescales there with 0 < alpha < 2^-THRESH)."""
    s = scores_log2(q, k, scale)
    bounds = tile_bounds([k.shape[0]] if seg_rows is None else seg_rows)
    m = np.full(s.shape[:2], -np.inf)
    events = np.zeros(s.shape[:2], dtype=bool)
    for i, (a, b) in enumerate(bounds):
        mx = s[:, :, a:b].max(axis=2)
        if i > 0:
            events |= mx > m + THRESH + margin
        # the wave raises its reference when any of its 32 queries needs it
        need = mx > m + THRESH
        H, nq = need.shape
        blk = np.zeros_like(need)
        for w in range(0, nq, 32):
            blk[:, w:w + 32] = need[:, w:w + 32].any(axis=1, keepdims=True)
        m = np.where(blk, np.maximum(m, mx), m)
    return events


def lazy_branch(q, k, v, scale, mistake=None):
    """The kernel's recurrence for one branch, float64: returns (O [n_q, H, D], LSE natural [H, n_q]).
    mistake: None, "no_l_rescale", "no_acc_rescale", "alpha_one" (the reference moves but nothing is
    rescaled), "inverse_alpha"."""
    s = scores_log2(q, k, scale)
    H, nq, nk = s.shape
    D = v.shape[2]
    m = np.full((H, nq), -np.inf)
    l = np.zeros((H, nq))
    acc = np.zeros((H, nq, D))
    for a, b in tile_bounds([nk]):
        st = s[:, :, a:b]
        mx = st.max(axis=2)
        need = mx > m + THRESH
        blk = np.zeros_like(need)
        for w in range(0, nq, 32):
            blk[:, w:w + 32] = need[:, w:w + 32].any(axis=1, keepdims=True)
        mnew = np.where(blk, np.maximum(m, mx), m)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isneginf(m), 0.0, np.exp2(m - mnew))
        if mistake == "alpha_one":
            alpha = np.where(np.isneginf(m), 0.0, 1.0)
        elif mistake == "inverse_alpha":
            alpha = np.where(np.isneginf(m), 0.0, np.exp2(mnew - m))
        if mistake != "no_l_rescale":
            l = l * alpha
        if mistake != "no_acc_rescale":
            acc = acc * alpha[:, :, None]
        m = mnew
        p = np.exp2(st - m[:, :, None])
        l = l + p.sum(axis=2)
        acc = acc + np.einsum("hqk,khd->hqd", p, v[a:b])
    o = acc / l[:, :, None]
    lse = (m + np.log2(l)) / LOG2E
    return np.transpose(o, (1, 0, 2)), lse
