"""Helpers for GPU tests: move seeded host arrays to the device and compare with the oracle."""
import sys

import numpy as np
import torch

from kv_cache_absorption_ispa_amd import inputs


def dev(t: inputs.Tensor) -> torch.Tensor:
    """Device copy with the exact bits the generator made (bf16 patterns or float32)."""
    if t.dtype == "bf16":
        return torch.from_numpy(t.raw.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(t.raw).cuda()


def host64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def poisoned(shape, dtype) -> torch.Tensor:
    """Output buffer filled with NaN, so an unwritten element fails any comparison."""
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def nan_workspace(nbytes: int):
    """A caller workspace whose previous contents are NaN (None when nbytes is 0): a kernel that reads
    any part of it before writing that part shows in the results."""
    from kv_cache_absorption_ispa_amd import ispa
    ws = ispa.workspace(nbytes)
    if ws is not None:
        ws[: nbytes // 4 * 4].view(torch.float32).fill_(float("nan"))
    return ws


def maxabs(a, b) -> float:
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    return float(np.nanmax(d)) if not np.isnan(d).any() else float("inf")


def relfro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def say(*msg):
    print(*msg, flush=True)
    sys.stdout.flush()


# tolerances from the parity contract
TOL_F32 = 1e-4            # outputs and LSE, float32 configurations (max-abs)
TOL_BF16_O = 2e-2         # outputs, bf16 configurations (max-abs)
TOL_BF16_LSE = 2e-3       # LSE, bf16 configurations (max-abs)
TOL_DW = 1e-3             # dW (relative Frobenius)
