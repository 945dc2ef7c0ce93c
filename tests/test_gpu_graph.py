"""One warmup-and-absorb step (decomposable attention, Gram accumulation, absorb solve) captured
into a HIP graph through torch.cuda.graph and replayed: every replay, with eager work and
synchronisation between them, must reproduce the eager step bit for bit.

The absorb solve forks R = C W onto the library's own second stream and joins it back with events;
capture follows that fork and join.  The library creates that stream on its first solve, so the
step runs eagerly once before capture.  Inputs are seeded draws; the comparison is GPU against GPU
(same computation, so exact), the step's parity with the oracle being covered elsewhere."""
import pytest
import torch

from kv_cache_absorption_ispa_amd import inputs, ispa
from tests.gpu_util import dev, nan_workspace

pytestmark = pytest.mark.gpu


def test_step_captured_in_a_graph_replays_like_eager():
    H, D, n_q, n_loc, n_hist = 2, 128, 384, 320, 512
    d = H * D
    x = inputs.custom_inputs(91, n_q, n_loc, n_hist, H, D, "bf16", boost_rows=8)
    q, kl, vl, kh, vh = dev(x.q), dev(x.k_loc), dev(x.v_loc), dev(x.k_hist), dev(x.v_hist)
    W = torch.from_numpy(inputs.normal(91, 0, inputs.LAYER_CHUNK, inputs.T_W, (d, d)) * d ** -0.5).cuda()
    o_loc = torch.empty(n_q, H, D, dtype=torch.bfloat16, device="cuda")
    o_full = torch.empty_like(o_loc)
    lse = torch.empty(H, n_q, device="cuda")
    G = torch.empty(d, d, device="cuda")
    C = torch.empty(d, d, device="cuda")
    dW = torch.empty(d, d, device="cuda")
    info = torch.empty(1, dtype=torch.int32, device="cuda")
    aws = nan_workspace(ispa.ispa_decomp_attn_workspace_size(q, n_loc, n_hist))
    gws = nan_workspace(ispa.ispa_gram_workspace_size(n_q, d, torch.bfloat16))
    sws = nan_workspace(ispa.ispa_absorb_workspace_size(d, d, 1))

    def step():
        ispa.ispa_decomp_attn(q, kl, vl, kh, vh, o_loc=o_loc, o_full=o_full, lse_full=lse, workspace=aws)
        ispa.ispa_gram_accum(o_loc, o_full, G, C, accumulate=False, workspace=gws)
        ispa.ispa_absorb_solve(G, C, W, 1e-2, dW, info, workspace=sws)

    outs = (o_loc, o_full, lse, G, C, dW)
    step()
    torch.cuda.synchronize()
    assert info.item() == 0
    eager = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm the capture stream as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))  # eager work between replays; every output must be rewritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert info.item() == 0, rep
        for name, t, e in zip(("O_loc", "O_full", "LSE_full", "G", "C", "dW"), outs, eager):
            assert torch.equal(t, e), (rep, name)
