"""GPU parity of the split-KV attention (ispa_decomp_attn_splitkv) against the float64 oracle.

Each (head, query tile) unit is cut into P equal pieces of key tiles on P
workgroups, whose states merge through their LSEs; the cases put piece
boundaries inside the local branch, at its end and inside the history, go down
to one key tile per piece, and include worker counts that give P = 1 (the
unsplit launch, which must be ispa_decomp_attn_segments bit for bit)."""
import numpy as np
import pytest
import torch

from kv_cache_absorption_ispa_amd import inputs
from kv_cache_absorption_ispa_amd import ispa
from tests.gpu_util import TOL_BF16_LSE, TOL_BF16_O, dev, say
from tests.test_gpu_attention import check_against_oracle, run_decomp
from tests.test_gpu_segments import NAMES, _outputs, _split

pytestmark = pytest.mark.gpu


def run_splitkv(x: inputs.ChunkInputs, scale, n_workers, loc_sizes=None, hist_sizes=None):
    q = dev(x.q)
    n_q, H, D = q.shape
    kl, vl = dev(x.k_loc), dev(x.v_loc)
    ls = loc_sizes or (kl.shape[0],)
    loc = list(zip(_split(kl, ls), _split(vl, ls)))
    hist = []
    if x.k_hist.shape[0]:
        hs = hist_sizes or (x.k_hist.shape[0],)
        kh, vh = dev(x.k_hist), dev(x.v_hist)
        hist = list(zip(_split(kh, hs), _split(vh, hs)))
    out = _outputs(n_q, H, D, q.dtype)
    ws = ispa.workspace(ispa.ispa_decomp_attn_splitkv_workspace_size(q, sum(ls), x.k_hist.shape[0], n_workers))
    if ws is not None:
        ws.view(torch.float32).fill_(float("nan"))  # every slot value the merge reads must have been written
    ispa.ispa_decomp_attn_splitkv(q, loc, hist, n_workers=n_workers, scale=scale, o_loc=out["O_loc"],
                                  lse_loc=out["LSE_loc"], o_hist=out["O_hist"], lse_hist=out["LSE_hist"],
                                  o_full=out["O_full"], lse_full=out["LSE_full"], workspace=ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case", [
    # (seed, n_q, loc sizes, hist sizes, H, D, workers); units = H x ceil(n_q / 256), P pieces each
    (51, 300, (200,), (333,), 2, 128, 16),     # 4 units, T = 5 (Tl = 2): P = 2, cut at tile 2
    (52, 300, (400,), (100,), 2, 128, 64),     # T = 5 (Tl = 4): P = 5, one key tile per piece
    (53, 300, (200,), (333,), 2, 128, 8),      # one workgroup per XCD: P = 1, unsplit
    (54, 600, (300,), (700,), 8, 128, 96),     # 24 units, T = 9: P = 4
    (55, 257, (64, 66), (), 2, 128, 16),       # no history: O_full is the merged O_loc
    (56, 129, (1, 130), (129, 1, 200), 3, 128, 24),  # T = 8 over 5 segments: P = 3
    (57, 200, (97,), (250,), 2, 64, 16),
    (58, 1, (1,), (1,), 1, 128, 16),           # T = 2: P = 2, one piece per branch
])
def test_splitkv_parity(case):
    seed, n_q, ls, hs, H, D, w = case
    say("case", case)
    x = inputs.custom_inputs(seed, n_q, sum(ls), sum(hs), H, D, "bf16", boost_rows=min(8, sum(ls)))
    scale = D ** -0.5
    out = run_splitkv(x, scale, w, ls, hs)
    for n in NAMES:
        assert not torch.isnan(out[n]).any().item(), n
    say("report", check_against_oracle(x, out, scale, TOL_BF16_O, TOL_BF16_LSE))


def test_one_unit_per_workgroup_is_bitwise_decomp():
    """With one workgroup per (head, query tile) unit nothing is split (P = 1): the outputs are
    those of ispa_decomp_attn bit for bit."""
    H, D, n_q = 3, 128, 600  # 3 query tiles of 256 -> 9 units
    x = inputs.custom_inputs(61, n_q, 300, 500, H, D, "bf16", boost_rows=8)
    out = run_splitkv(x, D ** -0.5, 9)
    ref = run_decomp(x, D ** -0.5)
    for n in NAMES:
        assert torch.equal(out[n], ref[n]), n


@pytest.mark.parametrize("cfg_name,n_q", [("wan1.3b-layer", 256), ("wan1.3b-layer", 4680),
                                          ("wan1.3b-long-history", 512)])
def test_splitkv_full_size_sampled_rows(cfg_name, n_q):
    """Full-size keys with one workgroup per compute unit: a short query chunk (12 or 24 units, so
    10-16 pieces each) and the full chunk (228 units: P = 1).  Sampled rows against the oracle,
    every element against the unsplit call within the bf16 output bound."""
    cfg = inputs.BY_NAME[cfg_name]
    say("config", cfg.name, "n_q", n_q)
    x = inputs.chunk_inputs(cfg, 0, 0, n_q=n_q)
    out = run_splitkv(x, cfg.scale, 0, (cfg.n_sink, cfg.n_chunk))
    for name, t in out.items():
        assert not torch.isnan(t).any().item(), f"{name} has unwritten (NaN) elements"
    g = np.random.default_rng(cfg.cfg_id)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(n_q - 80, n_q), g.choice(n_q, 24, replace=False)]))
    say("report", check_against_oracle(x, out, cfg.scale, TOL_BF16_O, TOL_BF16_LSE, rows=rows))
    ref = run_decomp(x, cfg.scale)
    for n in ("O_loc", "O_hist", "O_full"):
        d = (out[n].float() - ref[n].float()).abs().max().item()
        say(n, "max |split - unsplit|", d)
        assert d <= 2 * TOL_BF16_O
