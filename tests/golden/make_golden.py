"""Writes tests/golden/oracle_tiny.json: the oracle's outputs on a tiny seeded case.

The pages print no worked example, so there is no page-printed value to store.
This fixture is a regression pin of the oracle against itself over time (an
accidental edit to its arithmetic changes these numbers); it calls only
``oracle`` and the seeded input generator.  Run from the repo root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from kv_cache_absorption_ispa_amd import inputs  # noqa: E402


def case():
    cfg = inputs.TINY_F32
    x = inputs.chunk_inputs(cfg, 0, 0, n_q=4, n_hist=16)
    b = oracle.branch_outputs(x.q.f64, x.k_loc.f64, x.v_loc.f64, x.k_hist.f64, x.v_hist.f64, cfg.scale)
    a_loc, a_full = inputs.absorb_rows(0, 0, 64, 8, "f32")
    W = inputs.normal(0, 0, inputs.LAYER_CHUNK, inputs.T_W, (8, 8)) * np.float32(1 / np.sqrt(8))
    G, C = oracle.gram(a_loc.f64, a_full.f64)
    dW = oracle.ridge_solve(G, C, W.astype(np.float64), 1e-2)
    eps, eps_rel = oracle.reconstruction_error(a_loc.f64, a_full.f64, W.astype(np.float64), dW)
    out = {k: np.asarray(v).tolist() for k, v in b.items()}
    out.update(G=G.tolist(), C=C.tolist(), dW=dW.tolist(), eps=eps, eps_rel=eps_rel)
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump({"what": "oracle outputs, tiny seeded case (see make_golden.py)", "values": case()}, f)
    print("wrote", path)
