"""Planted mistakes: each plausible slip in the oracle must make at least one pin fail (CPU only).

A mutant replaces one oracle function on the CPU; the pin tests are then run
against it and at least one of them has to raise.  This checks that the pins
would catch a dropped term, a wrong sign, scale, log base or operand.
"""
import numpy as np
import pytest

import oracle
import oracle.ridge_absorb as oabs
import oracle.softmax_attention as oatt
import oracle.fp8 as ofp8
from tests import test_oracle_absorb as PA
from tests import test_oracle_fp8 as PF
from tests import test_oracle_attention as PT

_attn = oatt.attention
_merge = oatt.merge
_gram = oabs.gram
_solve = oabs.ridge_solve
_eps = oabs.reconstruction_error
_enc = ofp8.e4m3_encode
_scale = ofp8.absmax_scale
_tlam = oabs.trace_scaled_lambda
_below = oabs.select_below


def _attn_pins():
    return [
        lambda: PT.test_brute_force_tiny(4, 9, 2, 8),
        PT.test_torch_sdpa_and_logsumexp_float64,
        PT.test_single_key_gives_value_and_score,
        PT.test_equal_scores_give_mean_and_log_n,
        PT.test_score_shift_moves_lse_only,
        lambda: PT.test_merge_equals_full_softmax_for_any_split([10, 50]),
        PT.test_merge_weights_and_empty_branch,
    ]


def _absorb_pins():
    return [
        PA.test_gram_brute_force_entries,
        PA.test_zero_update_when_streams_agree,
        lambda: PA.test_ridge_matches_sklearn(1e-2),
        lambda: PA.test_ridge_matches_sklearn(30.0),
        PA.test_ridge_matches_stacked_lstsq,
        PA.test_exact_linear_relation_recovered_as_lambda_vanishes,
        PA.test_large_lambda_limit,
        PA.test_solution_minimises_objective,
        PA.test_reconstruction_error_closed_form,
    ]


def _variant_pins():
    return [
        PA.test_trace_scaled_lambda_value_and_scale_invariance,
        PA.test_select_below_brute_force,
    ]


def _some_pin_fails(pins):
    for p in pins:
        try:
            p()
        except (AssertionError, np.linalg.LinAlgError, ValueError, FloatingPointError):
            return True
    return False


ATTN_MUTANTS = {
    "scale dropped": lambda q, k, v, s, **kw: _attn(q, k, v, 1.0),
    "scale squared": lambda q, k, v, s, **kw: _attn(q, k, v, s * s),
    "lse in log2": lambda q, k, v, s, **kw: (lambda o, l: (o, l / np.log(2.0)))(*_attn(q, k, v, s)),
    "lse without the running max": lambda q, k, v, s, **kw: (
        lambda o, l: (o, np.where(np.isfinite(l), np.log(np.sum(np.exp(
            s * np.einsum("qhd,khd->hqk", np.asarray(q, float), np.asarray(k, float))
            - (s * np.einsum("qhd,khd->hqk", np.asarray(q, float), np.asarray(k, float))).max(-1, keepdims=True)),
            axis=-1)) if np.asarray(k).shape[0] else l, l)))(*_attn(q, k, v, s)),
    "normaliser off by one key": lambda q, k, v, s, **kw: (
        (lambda o, l: (o * (np.asarray(k).shape[0] / (np.asarray(k).shape[0] + 1.0)), l))(*_attn(q, k, v, s))),
    "heads of V swapped": lambda q, k, v, s, **kw: _attn(q, k, np.asarray(v)[:, ::-1, :], s),
}

MERGE_MUTANTS = {
    "weights swapped": lambda oa, la, ob, lb: (lambda o, l: (
        np.exp(np.asarray(lb) - l).T[:, :, None] * oa + np.exp(np.asarray(la) - l).T[:, :, None] * ob, l))(
        None, np.logaddexp(la, lb)),
    "plain average": lambda oa, la, ob, lb: (0.5 * (np.asarray(oa) + np.asarray(ob)), np.logaddexp(la, lb)),
    "lse = max": lambda oa, la, ob, lb: (_merge(oa, la, ob, lb)[0], np.maximum(la, lb)),
}

GRAM_MUTANTS = {
    "C without the -A_loc term": lambda al, af: (_gram(al, af)[0],
                                                 np.asarray(al, float).T @ np.asarray(af, float)),
    "C transposed": lambda al, af: (lambda g, c: (g, c.T))(*_gram(al, af)),
    "mean instead of sum": lambda al, af: (lambda g, c: (g / len(al), c / len(al)))(*_gram(al, af)),
    "G from A_full": lambda al, af: (np.asarray(af, float).T @ np.asarray(af, float), _gram(al, af)[1]),
}

SOLVE_MUTANTS = {
    "lambda dropped": lambda G, C, W, lam: _solve(G, C, W, 0.0),
    "lambda doubled": lambda G, C, W, lam: _solve(G, C, W, 2.0 * lam),
    "sign flipped": lambda G, C, W, lam: -_solve(G, C, W, lam),
    "C transposed": lambda G, C, W, lam: _solve(G, np.asarray(C).T, W, lam),
    "W transposed": lambda G, C, W, lam: _solve(G, C, np.asarray(W).T, lam) if np.shape(W)[0] == np.shape(W)[1]
    else _solve(G, C, W, lam) * 1.001,
}

EPS_MUTANTS = {
    "A_full without W": lambda al, af, W, dW: (lambda r: (float(np.sum(r * r)), 1.0))(
        np.asarray(al, float) @ (W + dW) - np.asarray(af, float) @ np.eye(*np.shape(W))),
    "pre-fit discrepancy": lambda al, af, W, dW: _eps(al, af, W, np.zeros_like(dW)),
}


TLAM_MUTANTS = {
    "trace without 1/d": lambda G, s: s * float(np.trace(np.asarray(G, float))),
    "mean diagonal of G^2": lambda G, s: s * float(np.trace(np.asarray(G, float) @ np.asarray(G, float))) / len(G),
    "largest diagonal entry": lambda G, s: s * float(np.max(np.diag(np.asarray(G, float)))),
    "constant (absolute) lambda": lambda G, s: float(s),
}

BELOW_MUTANTS = {
    "strict threshold": lambda e, t, k: [i for i in _below(e, t, k + 1) if np.asarray(e, float)[i] < t][:k],
    "NaN admitted": lambda e, t, k: [int(i) for i in np.argsort(np.nan_to_num(np.asarray(e, float), nan=-1.0),
                                                               kind="stable") if not np.asarray(e, float)[i] > t][:k],
    "cap ignored": lambda e, t, k: _below(e, t, len(e)),
    "ties to the higher index": lambda e, t, k: [-j for _, j in sorted(
        (float(np.asarray(e, float)[i]), -i) for i in range(len(e)) if np.asarray(e, float)[i] <= t)][:k],
}


def _fp8_pins():
    return [PF.test_hand_values, PF.test_matches_torch_cast, PF.test_every_finite_code_round_trips,
            PF.test_nearest_and_ties_to_even, PF.test_per_head_scale_maps_amax_to_448,
            PF.test_w8a8_matmul_exact_and_bounded]


ENC_MUTANTS = {
    "ties away from zero": lambda x: np.where(
        np.abs(ofp8.e4m3_decode(_enc(x)) - np.asarray(x, np.float64)) > 0,
        _enc(np.nextafter(np.asarray(x, np.float32), np.float32(np.inf) * np.sign(np.asarray(x, np.float32)))),
        _enc(x)).astype(np.uint8),
    "subnormals flushed": lambda x: np.where(np.abs(np.asarray(x, np.float32)) < 2.0 ** -6,
                                             (np.signbit(np.asarray(x, np.float32)) * 0x80).astype(np.uint8),
                                             _enc(x)).astype(np.uint8),
    "truncation": lambda x: _enc(np.asarray(x, np.float32) * np.float32(1 - 2.0 ** -5)),
}

SCALE_MUTANTS = {
    "amax / 256": lambda x, axis=None: (_scale(x, axis) * np.float32(448.0 / 256.0)).astype(np.float32),
    "amax / 448 in float64": lambda x, axis=None: np.where(
        np.max(np.abs(np.asarray(x, np.float64)), axis=axis) > 0,
        np.max(np.abs(np.asarray(x, np.float64)), axis=axis) / 448.0 * (1 + 1e-7), 1.0),
}


@pytest.mark.parametrize("name", ENC_MUTANTS)
def test_fp8_encode_mutant_caught(name, monkeypatch):
    monkeypatch.setattr(ofp8, "e4m3_encode", ENC_MUTANTS[name])
    assert _some_pin_fails(_fp8_pins()), name


@pytest.mark.parametrize("name", SCALE_MUTANTS)
def test_fp8_scale_mutant_caught(name, monkeypatch):
    monkeypatch.setattr(ofp8, "absmax_scale", SCALE_MUTANTS[name])
    assert _some_pin_fails(_fp8_pins()), name


@pytest.mark.parametrize("name", TLAM_MUTANTS)
def test_trace_lambda_mutant_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "trace_scaled_lambda", TLAM_MUTANTS[name])
    assert _some_pin_fails(_variant_pins()), name


@pytest.mark.parametrize("name", BELOW_MUTANTS)
def test_select_below_mutant_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "select_below", BELOW_MUTANTS[name])
    assert _some_pin_fails(_variant_pins()), name


@pytest.mark.parametrize("name", ATTN_MUTANTS)
def test_attention_mutant_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "attention", ATTN_MUTANTS[name])
    assert _some_pin_fails(_attn_pins()), name


@pytest.mark.parametrize("name", MERGE_MUTANTS)
def test_merge_mutant_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "merge", MERGE_MUTANTS[name])
    assert _some_pin_fails(_attn_pins()), name


@pytest.mark.parametrize("name", GRAM_MUTANTS)
def test_gram_mutant_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "gram", GRAM_MUTANTS[name])
    assert _some_pin_fails(_absorb_pins()), name


@pytest.mark.parametrize("name", SOLVE_MUTANTS)
def test_solve_mutant_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "ridge_solve", SOLVE_MUTANTS[name])
    assert _some_pin_fails(_absorb_pins()), name


@pytest.mark.parametrize("name", EPS_MUTANTS)
def test_eps_mutant_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "reconstruction_error", EPS_MUTANTS[name])
    assert _some_pin_fails(_absorb_pins()), name


def test_unmutated_oracle_passes_every_pin():
    assert not _some_pin_fails(_attn_pins())
    assert not _some_pin_fails(_absorb_pins())
    assert not _some_pin_fails(_variant_pins())
    assert not _some_pin_fails(_fp8_pins())
