"""Oracle: softmax attention over a key set, the two branches, and their merge.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "Technical Summary: Instance-Specific Parametric Absorption (ISPA) for
Memory-Efficient Video Generation", section 2 "Methodology", step 1 "Dual-Stream
Warmup": A_full is attention over the entire context, A_loc is attention over
the current chunk plus the sink tokens, and the decomposable form computes a
local and a historical branch and fuses them after the fact from their
log-sum-exp (LSE) states.

Readings of what the page leaves open:

* scores are scale * <q, k> with scale = 1/sqrt(head_dim); no mask: every query
  sees every sink, chunk and history key;
* LSE is the natural log of sum_j exp(score_ij), scale included;
* the merge is the standard LSE merge: LSE = logaddexp(LSE_a, LSE_b) and
  O = exp(LSE_a - LSE) O_a + exp(LSE_b - LSE) O_b;
* a branch with no keys has LSE = -inf and O = 0, so it drops out of the merge.

Layouts: Q, K, V are [tokens, heads, head_dim]; O is [tokens, heads, head_dim];
LSE is [heads, tokens].  All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np


def attention(q, k, v, scale, row_block: int = 512):
    """Softmax attention of every query over every key, per head (direct, not online).

    For head h and query i: s_ij = scale * sum_e q_ihe k_jhe, m_i = max_j s_ij,
    p_ij = exp(s_ij - m_i), l_i = sum_j p_ij, O_i = sum_j p_ij v_jh / l_i,
    LSE_i = m_i + ln l_i.  Returns (O [Nq,H,D], LSE [H,Nq]).  With no keys,
    O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, H, D = q.shape
    nk = k.shape[0]
    out = np.zeros((nq, H, D), dtype=np.float64)
    lse = np.full((H, nq), -np.inf, dtype=np.float64)
    if nk == 0 or nq == 0:
        return out, lse
    for h in range(H):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for r0 in range(0, nq, row_block):
            qh = q[r0:r0 + row_block, h, :]
            s = scale * (qh @ kh.T)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            out[r0:r0 + row_block, h, :] = (p @ vh) / l
            lse[h, r0:r0 + row_block] = (m + np.log(l))[:, 0]
    return out, lse


def merge(o_a, lse_a, o_b, lse_b):
    """Fuse two branches' (O, LSE) into the output over the union of their keys.

    LSE = logaddexp(LSE_a, LSE_b); O = exp(LSE_a - LSE) O_a + exp(LSE_b - LSE) O_b.
    O is [Nq,H,D] and LSE is [H,Nq].  If both LSEs are -inf the result is O = 0,
    LSE = -inf."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - lse))
        wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - lse))
    # weights are [H, Nq]; outputs are [Nq, H, D]
    return wa.T[:, :, None] * o_a + wb.T[:, :, None] * o_b, lse


def branch_outputs(q, k_loc, v_loc, k_hist, v_hist, scale):
    """The dual-stream quantities of one chunk, each computed directly.

    Returns dict with O_loc/LSE_loc (keys = sink + chunk), O_hist/LSE_hist
    (keys = history) and O_full/LSE_full (keys = all of them, computed as one
    softmax over the concatenated key set, not by merging)."""
    o_loc, lse_loc = attention(q, k_loc, v_loc, scale)
    o_hist, lse_hist = attention(q, k_hist, v_hist, scale)
    k_all = np.concatenate([np.asarray(k_loc), np.asarray(k_hist)], axis=0)
    v_all = np.concatenate([np.asarray(v_loc), np.asarray(v_hist)], axis=0)
    o_full, lse_full = attention(q, k_all, v_all, scale)
    return dict(O_loc=o_loc, LSE_loc=lse_loc, O_hist=o_hist, LSE_hist=lse_hist,
                O_full=o_full, LSE_full=lse_full)
