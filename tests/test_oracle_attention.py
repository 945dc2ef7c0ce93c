"""Pins for the oracle's attention, branch split and LSE merge (CPU only).

Each pin ties the oracle to something other than itself: pure-Python brute
force with a different formula (no max subtraction, exact summation), torch's
float64 scaled-dot-product attention and logsumexp (library routines), closed
forms for special cases, and invariants the mathematics fixes (the merge of
the local and historical branches equals one softmax over all keys, however
the keys are split; permuting keys changes nothing).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from kv_cache_absorption_ispa_amd import inputs


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_attention(q, k, v, scale):
    """Scalar loops: p_ij = exp(s_ij) / sum_j exp(s_ij) with exact (fsum) sums; no max shift."""
    nq, H, D = q.shape
    nk = k.shape[0]
    out = np.zeros((nq, H, D))
    lse = np.zeros((H, nq))
    for h in range(H):
        for i in range(nq):
            e = []
            for j in range(nk):
                s = scale * math.fsum(float(q[i, h, c]) * float(k[j, h, c]) for c in range(D))
                e.append(math.exp(s))
            z = math.fsum(e)
            lse[h, i] = math.log(z)
            for c in range(D):
                out[i, h, c] = math.fsum(e[j] * float(v[j, h, c]) for j in range(nk)) / z
    return out, lse


@pytest.mark.parametrize("nq,nk,H,D", [(3, 5, 1, 4), (4, 9, 2, 8), (1, 1, 2, 4), (5, 33, 1, 6)])
def test_brute_force_tiny(nq, nk, H, D):
    q, k, v = _rand(1, nq, H, D), _rand(2, nk, H, D), _rand(3, nk, H, D)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale)
    ob, lseb = brute_attention(q, k, v, scale)
    assert np.max(np.abs(o - ob)) <= 1e-13
    assert np.max(np.abs(lse - lseb)) <= 1e-13


def test_torch_sdpa_and_logsumexp_float64():
    """Library routine pin: torch's attention (float64, CPU) and logsumexp."""
    nq, nk, H, D = 37, 150, 3, 16
    q, k, v = _rand(4, nq, H, D), _rand(5, nk, H, D), _rand(6, nk, H, D)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0].permute(1, 0, 2).numpy()
    s = scale * torch.einsum("qhd,khd->hqk", torch.from_numpy(q), torch.from_numpy(k))
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-13
    assert np.max(np.abs(lse - ref_lse)) <= 1e-13


def test_single_key_gives_value_and_score():
    q, k, v = _rand(7, 6, 2, 8), _rand(8, 1, 2, 8), _rand(9, 1, 2, 8)
    o, lse = oracle.attention(q, k, v, 0.5)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))
    s = 0.5 * np.einsum("qhd,hd->hq", q, k[0])
    assert np.max(np.abs(lse - s)) <= 1e-15


def test_equal_scores_give_mean_and_log_n():
    nk = 77
    q = np.zeros((4, 2, 8))
    k, v = _rand(10, nk, 2, 8), _rand(11, nk, 2, 8)
    o, lse = oracle.attention(q, k, v, 0.125)
    assert np.max(np.abs(o - v.mean(axis=0)[None])) <= 1e-15
    assert np.max(np.abs(lse - math.log(nk))) <= 1e-14


def test_constant_values_give_constant():
    q, k = _rand(12, 5, 2, 8), _rand(13, 40, 2, 8)
    c = _rand(14, 2, 8)
    v = np.broadcast_to(c, (40, 2, 8)).copy()
    o, _ = oracle.attention(q, k, v, 0.3)
    assert np.max(np.abs(o - c[None])) <= 1e-14


def test_score_shift_moves_lse_only():
    """Adding the same vector w to every key shifts query i's scores by scale*<q_i, w>:
    O must not change and LSE must move by exactly that amount."""
    q, k, v = _rand(15, 9, 2, 8), _rand(16, 30, 2, 8), _rand(17, 30, 2, 8)
    w = 3.0 * _rand(18, 2, 8)
    scale = 0.35
    o1, l1 = oracle.attention(q, k, v, scale)
    o2, l2 = oracle.attention(q, k + w[None], v, scale)
    shift = scale * np.einsum("qhd,hd->hq", q, w)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs((l2 - l1) - shift)) <= 1e-12


def test_huge_scores_stay_finite():
    q, k, v = 40.0 * _rand(19, 5, 1, 8), 40.0 * _rand(20, 50, 1, 8), _rand(21, 50, 1, 8)
    o, lse = oracle.attention(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    # the output is a convex combination of value rows
    assert np.all(o <= v.max(axis=0)[None] + 1e-12) and np.all(o >= v.min(axis=0)[None] - 1e-12)


def test_key_permutation_invariance():
    q, k, v = _rand(22, 11, 2, 8), _rand(23, 60, 2, 8), _rand(24, 60, 2, 8)
    perm = np.random.default_rng(25).permutation(60)
    o1, l1 = oracle.attention(q, k, v, 0.4)
    o2, l2 = oracle.attention(q, k[perm], v[perm], 0.4)
    assert np.max(np.abs(o1 - o2)) <= 1e-14
    assert np.max(np.abs(l1 - l2)) <= 1e-13


def test_empty_key_set():
    q = _rand(26, 3, 2, 4)
    o, lse = oracle.attention(q, np.zeros((0, 2, 4)), np.zeros((0, 2, 4)), 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("cuts", [[40], [1], [99], [10, 50], [3, 30, 70]])
def test_merge_equals_full_softmax_for_any_split(cuts):
    """The decomposition is exact: merging the branches' (O, LSE) reproduces one softmax
    over the union of keys, however the keys are split (2-way, 3-way, 4-way)."""
    q, k, v = _rand(27, 13, 2, 8), 2.0 * _rand(28, 100, 2, 8), _rand(29, 100, 2, 8)
    scale = 0.3
    o_full, l_full = oracle.attention(q, k, v, scale)
    bounds = [0] + cuts + [100]
    o_m, l_m = oracle.attention(q, k[:0], v[:0], scale)
    for a, b in zip(bounds[:-1], bounds[1:]):
        o_p, l_p = oracle.attention(q, k[a:b], v[a:b], scale)
        o_m, l_m = oracle.merge(o_m, l_m, o_p, l_p)
    assert np.max(np.abs(o_m - o_full)) <= 1e-13
    assert np.max(np.abs(l_m - l_full)) <= 1e-13


def test_merge_weights_and_empty_branch():
    q, k, v = _rand(30, 7, 2, 8), _rand(31, 20, 2, 8), _rand(32, 20, 2, 8)
    o, l = oracle.attention(q, k, v, 0.3)
    oe, le = oracle.attention(q, k[:0], v[:0], 0.3)
    om, lm = oracle.merge(o, l, oe, le)
    assert np.array_equal(om, o) and np.array_equal(lm, l)
    om2, lm2 = oracle.merge(oe, le, o, l)
    assert np.array_equal(om2, o) and np.array_equal(lm2, l)
    # merge weights exp(LSE_a - LSE) + exp(LSE_b - LSE) sum to one
    o1, l1 = oracle.attention(q, k[:8], v[:8], 0.3)
    o2, l2 = oracle.attention(q, k[8:], v[8:], 0.3)
    _, lm3 = oracle.merge(o1, l1, o2, l2)
    assert np.max(np.abs(np.exp(l1 - lm3) + np.exp(l2 - lm3) - 1.0)) <= 1e-14


def test_branch_outputs_on_seeded_tiny_layer():
    """The dual-stream quantities on the seeded fp32 layer: full = merge(local, history)."""
    cfg = inputs.TINY_F32
    x = inputs.chunk_inputs(cfg, 0, 0, n_q=48, n_hist=200)
    b = oracle.branch_outputs(x.q.f64, x.k_loc.f64, x.v_loc.f64, x.k_hist.f64, x.v_hist.f64, cfg.scale)
    om, lm = oracle.merge(b["O_loc"], b["LSE_loc"], b["O_hist"], b["LSE_hist"])
    assert np.max(np.abs(om - b["O_full"])) <= 1e-13
    assert np.max(np.abs(lm - b["LSE_full"])) <= 1e-13
    # local branch alone differs from the full output (the history matters)
    assert np.max(np.abs(b["O_loc"] - b["O_full"])) > 1e-2
