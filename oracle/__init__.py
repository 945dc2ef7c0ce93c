"""Oracle: a plain, slow, obviously correct float64 CPU implementation of the ISPA hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

Sources (the pages this follows):

* "Towards Memory-Efficient Autoregressive Video Generation via
  Instance-Specific Parametric Absorption" (mlsanity.com paper card), section
  "Abstract (arXiv)": the F-layer / L-layer split and the closed-form absorb.
* "Technical Summary: Instance-Specific Parametric Absorption (ISPA) for
  Memory-Efficient Video Generation" (gist.science), section 2
  "Methodology": Dual-Stream Warmup (A_full, A_loc, decomposable attention
  fused after the fact through log-sum-exp states), Layer Absorb (the ridge
  objective and its closed-form minimiser), Memory-Efficient Inference
  (W_new = W + dW, history eviction) and Dynamic Layer Selection (ranking by
  reconstruction error); section 3 "Key Contributions" (online softmax).

Every function computes the plain definition of its quantity (the method reaches
these exact results, up to rounding order), in float64, with numpy/LAPACK
primitives and no blocking or reordering beyond the definition.
"""
from . import fp8
from .softmax_attention import attention, branch_outputs, merge
from .ridge_absorb import (gram, gram_from_chunks, ridge_solve, objective, reconstruction_error, select_layers,
                           select_below, trace_scaled_lambda)

__all__ = [
    "fp8",
    "attention",
    "branch_outputs",
    "merge",
    "gram",
    "gram_from_chunks",
    "ridge_solve",
    "objective",
    "reconstruction_error",
    "select_layers",
    "select_below",
    "trace_scaled_lambda",
]
