"""Oracle: Gram statistics, the closed-form ridge absorb, reconstruction error, selection.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "Technical Summary: Instance-Specific Parametric Absorption (ISPA) for
Memory-Efficient Video Generation", section 2 "Methodology":

* step 2 "Layer Absorb": the objective
  min_dW ||A_loc (W + dW) - A_full W||^2 + lambda ||dW||^2 and its minimiser
  dW = (A_loc^T A_loc + lambda I)^-1 A_loc^T (A_full - A_loc) W;
* step 3 "Memory-Efficient Inference": W_new = W + dW for the converted layers;
* "Dynamic Layer Selection": layers are ranked by their reconstruction error
  and the lowest-error ones are converted.

The pages leave the error measure, lambda and the number of converted layers
open; besides the reading used by default (below) the variants are: ranking by
the error before the fit (``reconstruction_error`` with dW = 0), by the error on
held-out rows (``reconstruction_error`` on rows the fit did not see), lambda
proportional to the mean eigenvalue of G (:func:`trace_scaled_lambda`), and
converting every layer whose error is under a threshold (:func:`select_below`).

Readings taken here: the norm is Frobenius and the objective
is a sum (not a mean) over all warmup rows, every row weighted equally; lambda
is absolute; W is the attention output projection in the row-vector convention
y = a W with W of shape [d, d_out]; the reconstruction error is the post-fit
data residual ||A_loc (W + dW) - A_full W||_F^2 (lambda term excluded), and the
ranking uses it relative to ||A_full W||_F^2, ties going to the lower layer
index.
"""
from __future__ import annotations

import numpy as np


def gram(a_loc, a_full):
    """G = A_loc^T A_loc and C = A_loc^T (A_full - A_loc) over the given rows ([N, d] each)."""
    a_loc = np.asarray(a_loc, dtype=np.float64)
    a_full = np.asarray(a_full, dtype=np.float64)
    return a_loc.T @ a_loc, a_loc.T @ (a_full - a_loc)


def gram_from_chunks(chunks):
    """Sum of :func:`gram` over an iterable of (A_loc, A_full) chunks (the warmup rows)."""
    G = C = None
    for a_loc, a_full in chunks:
        g, c = gram(a_loc, a_full)
        G = g if G is None else G + g
        C = c if C is None else C + c
    return G, C


def ridge_solve(G, C, W, lam):
    """dW = (G + lambda I)^-1 (C W), by LAPACK's general solve in float64."""
    G = np.asarray(G, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    d = G.shape[0]
    return np.linalg.solve(G + lam * np.eye(d), C @ W)


def objective(a_loc, a_full, W, dW, lam):
    """||A_loc (W + dW) - A_full W||_F^2 + lambda ||dW||_F^2."""
    r = np.asarray(a_loc, np.float64) @ (np.asarray(W, np.float64) + dW) - np.asarray(a_full, np.float64) @ W
    return float(np.sum(r * r) + lam * np.sum(np.asarray(dW) ** 2))


def reconstruction_error(a_loc, a_full, W, dW):
    """(eps, eps_rel): eps = ||A_loc (W + dW) - A_full W||_F^2, eps_rel = eps / ||A_full W||_F^2.

    Computed explicitly from the stored rows."""
    a_loc = np.asarray(a_loc, np.float64)
    a_full = np.asarray(a_full, np.float64)
    W = np.asarray(W, np.float64)
    y_full = a_full @ W
    r = a_loc @ (W + np.asarray(dW, np.float64)) - y_full
    eps = float(np.sum(r * r))
    return eps, eps / float(np.sum(y_full * y_full))


def select_layers(eps_rel, k):
    """Indices of the k layers with the lowest eps_rel (ties to the lower index), ascending by error."""
    eps_rel = np.asarray(eps_rel, dtype=np.float64)
    order = np.argsort(eps_rel, kind="stable")
    return [int(i) for i in order[:k]]


def trace_scaled_lambda(G, lam_scale):
    """lambda = lam_scale * tr(G) / d: the ridge weight as a fraction of G's mean eigenvalue."""
    G = np.asarray(G, dtype=np.float64)
    return float(lam_scale) * float(np.trace(G)) / G.shape[0]


def select_below(eps_rel, tau, k_max):
    """Layers with eps_rel <= tau, lowest first (ties to the lower index), at most k_max; NaN never."""
    eps_rel = np.asarray(eps_rel, dtype=np.float64)
    order = [int(i) for i in np.argsort(eps_rel, kind="stable")]
    return [i for i in order if eps_rel[i] <= tau][:k_max]
