"""The lazy-rescale GPU cases have teeth (CPU only).

On the planted inputs of tests/test_gpu_rescale.py, the kernel's recurrence (tests/rescale_util.py:
128-key tiles, reference raised only past 2^8, wave-wide decision) run in float64 matches the
oracle, while each plausible mistake in the rescale (row sum not scaled, accumulator not scaled,
alpha = 1, alpha inverted) moves the outputs or the LSE far past the bf16 gates.  So a GPU kernel
with such a mistake cannot pass the GPU cases."""
import numpy as np
import pytest

import oracle
from kv_cache_absorption_ispa_amd import inputs
from tests import rescale_util as ru
from tests.gpu_util import TOL_BF16_LSE, TOL_BF16_O
from tests.test_gpu_rescale import CASES, MIN_EVENTS, planted

MISTAKES = ("no_l_rescale", "no_acc_rescale", "alpha_one", "inverse_alpha")


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("branch", ["local", "history"])
def test_planted_cases_rescale_late_and_catch_mistakes(case, branch):
    x = planted(case)
    D = case[5]
    scale = D ** -0.5
    k, v = (x.k_loc, x.v_loc) if branch == "local" else (x.k_hist, x.v_hist)
    q = x.q.f64
    ev = ru.rescale_events(q, k.f64, scale)
    assert int(ev.sum()) >= MIN_EVENTS
    ref_o, ref_l = oracle.attention(q, k.f64, v.f64, scale)
    o, l = ru.lazy_branch(q, k.f64, v.f64, scale)
    assert np.max(np.abs(o - ref_o)) <= 1e-10 and np.max(np.abs(l - ref_l)) <= 1e-10
    for m in MISTAKES:
        with np.errstate(all="ignore"):
            o, l = ru.lazy_branch(q, k.f64, v.f64, scale, mistake=m)
        eo = np.nanmax(np.abs(o - ref_o)) if np.isfinite(o).any() else np.inf
        el = np.nanmax(np.abs(l - ref_l)) if np.isfinite(l).any() else np.inf
        assert eo > 10 * TOL_BF16_O or el > 10 * TOL_BF16_LSE, (m, eo, el)


def test_plain_inputs_never_rescale_late():
    """Why the planted cases exist: with N(0,1) keys (and the usual 4x boost in the first local tile)
    no query's reference moves after a branch's first tile."""
    x = inputs.custom_inputs(201, 300, 700, 900, 2, 128, "bf16", boost_rows=8)
    for k in (x.k_loc, x.k_hist):
        assert int(ru.rescale_events(x.q.f64, k.f64, 128 ** -0.5, margin=0.0).sum()) == 0
