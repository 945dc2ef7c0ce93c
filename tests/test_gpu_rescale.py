"""GPU parity of the online softmax's lazy rescale: keys that dominate late in a branch.

The attention kernel moves its reference maximum only when a key tile beats it by more than 2^8
(log2 domain), scaling the row sum and the accumulator by alpha = 2^(m_old - m_new).  With plain
N(0, 1) keys this never happens after a branch's first tile, so these cases plant keys with 24x the
usual norm in the LAST tile of the local branch, the last tile of the history branch, a middle
segment, and a non-first split-KV piece, for bf16 and fp8 keys, at ragged sizes.  Before each GPU
call the host model in tests/rescale_util.py confirms from the inputs that many (head, query) pairs
must rescale there with 0 < alpha < 2^-8; tests/test_rescale_cases.py shows on the CPU that a wrong
or missing rescale then fails the gates.  Everything is compared with the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_absorption_ispa_amd import inputs, ispa
from tests import rescale_util as ru
from tests.gpu_util import TOL_BF16_LSE, TOL_BF16_O, dev, say
from tests.test_gpu_attention import check_against_oracle, run_decomp
from tests.test_gpu_fp8 import _check, _fp8k_inputs, _run_fp8k
from tests.test_gpu_segments import run_segments
from tests.test_gpu_splitkv import run_splitkv

pytestmark = pytest.mark.gpu

# (seed, n_q, n_loc, n_hist, H, D): local and history each span several 128-key tiles and end ragged
CASES = [(201, 300, 700, 900, 2, 128), (202, 257, 390, 645, 3, 64)]
MIN_EVENTS = 40  # (head, query) pairs that must rescale late in each planted branch


def planted(case):
    seed, n_q, n_loc, n_hist, H, D = case
    return inputs.planted_inputs(seed, n_q, n_loc, n_hist, H, D, "bf16",
                                 loc_rows=(n_loc - 1, n_loc - 37), hist_rows=(n_hist - 1, n_hist - 2))


def assert_late_rescales(q, k, scale, seg_rows=None, what=""):
    ev = ru.rescale_events(q, k, scale, seg_rows)
    n = int(ev.sum())
    say(f"late rescales {what}: {n} of {ev.size} (head, query) pairs")
    assert n >= MIN_EVENTS, (what, n)


@pytest.mark.parametrize("case", CASES)
def test_rescale_in_last_local_and_history_tiles(case):
    x = planted(case)
    D = case[5]
    scale = D ** -0.5
    assert_late_rescales(x.q.f64, x.k_loc.f64, scale, what="local")
    assert_late_rescales(x.q.f64, x.k_hist.f64, scale, what="history")
    out = run_decomp(x, scale)
    say("report", check_against_oracle(x, out, scale, TOL_BF16_O, TOL_BF16_LSE))


def test_rescale_in_a_middle_segment():
    """History given as three segments, the dominant keys in the second one's second tile; the local
    branch as sink + chunk with a dominant key in the chunk's last tile."""
    seed, n_q, H, D = 203, 300, 2, 128
    ls, hs = (100, 600), (300, 350, 250)
    x = inputs.planted_inputs(seed, n_q, sum(ls), sum(hs), H, D, "bf16", loc_rows=(sum(ls) - 5,),
                              hist_rows=(300 + 200, 300 + 201))
    scale = D ** -0.5
    assert_late_rescales(x.q.f64, x.k_loc.f64, scale, seg_rows=ls, what="local segments")
    assert_late_rescales(x.q.f64, x.k_hist.f64, scale, seg_rows=hs, what="history segments")
    out = run_segments(x, scale, ls, hs)
    say("report", check_against_oracle(x, out, scale, TOL_BF16_O, TOL_BF16_LSE))


def _sk_pieces(n_wg, n_units, T):
    """Pieces per unit of the split-KV launch (the kernel's rule: the most workgroups every XCD can
    give each of its units, at most T)."""
    pc = T
    for x in range(8):
        wx = n_wg // 8 + (1 if x < n_wg % 8 else 0)
        nx = n_units // 8 + (1 if x < n_units % 8 else 0)
        if nx > 0:
            pc = min(pc, wx // nx)
    return max(pc, 1)


@pytest.mark.parametrize("workers", [16, 32])
def test_rescale_inside_a_later_split_kv_piece(workers):
    """Split-KV: each piece starts a fresh softmax state; the dominant keys sit in the last tile of a
    piece that is not the unit's first and has earlier tiles of its own."""
    seed, n_q, n_loc, n_hist, H, D = 204, 300, 700, 900, 2, 128
    x = inputs.planted_inputs(seed, n_q, n_loc, n_hist, H, D, "bf16", loc_rows=(n_loc - 1,),
                              hist_rows=(n_hist - 1,))
    scale = D ** -0.5
    Tl, T = -(-n_loc // 128), -(-n_loc // 128) - (-n_hist // 128)
    P = _sk_pieces(workers, H * -(-n_q // 256), T)
    cuts = [i * T // P for i in range(P + 1)]
    assert P >= 2, P
    piece_of = lambda tile: max(j for j in range(P) if cuts[j] <= tile)
    for tile in (Tl - 1, T - 1):  # the tiles holding the dominant keys: never a piece's first tile
        assert cuts[piece_of(tile)] < tile, (P, cuts, tile)
    assert piece_of(T - 1) > 0, (P, cuts)  # the history plant lies in a later piece
    # within its piece the history plant follows earlier history tiles of the same piece
    p_last = max(j for j in range(P) if cuts[j] <= T - 1)
    first_hist_tile_of_piece = max(cuts[p_last], Tl)
    keys = x.k_hist.f64[(first_hist_tile_of_piece - Tl) * 128:]
    assert_late_rescales(x.q.f64, keys, scale, what=f"history part of the last piece (P = {P})")
    out = run_splitkv(x, scale, workers)
    say("report", check_against_oracle(x, out, scale, TOL_BF16_O, TOL_BF16_LSE))


@pytest.mark.parametrize("case", CASES[:1])
def test_rescale_with_fp8_keys(case):
    seed, n_q, n_loc, n_hist, H, D = case
    x = planted(case)
    scale = D ** -0.5
    q8, qs, segs, kd = _fp8k_inputs(x, (n_loc,), (n_hist,))
    from oracle import fp8 as ofp8
    qd = ofp8.dequantize(q8, qs[None, :, None])
    assert_late_rescales(qd, kd[0], scale, what="fp8 local")
    assert_late_rescales(qd, kd[1], scale, what="fp8 history")
    out = _run_fp8k(q8, qs, segs, H, D, n_q, scale)
    say("report", _check(x, q8, qs, kd, out, H, scale, 1))
