"""GPU parity of the segment-list attention (ispa_decomp_attn_segments) and of a streaming
loop over the K/V cache, against the float64 oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_absorption_ispa_amd import inputs
from kv_cache_absorption_ispa_amd import ispa
from kv_cache_absorption_ispa_amd.kv_cache import StreamingKVCache
from tests.gpu_util import (TOL_BF16_LSE, TOL_BF16_O, TOL_F32, dev, host64, maxabs, poisoned, say)
from tests.test_gpu_attention import check_against_oracle, run_decomp

pytestmark = pytest.mark.gpu

NAMES = ("O_loc", "LSE_loc", "O_hist", "LSE_hist", "O_full", "LSE_full")


def _outputs(n_q, H, D, dt):
    return dict(O_loc=poisoned((n_q, H, D), dt), LSE_loc=poisoned((H, n_q), torch.float32),
                O_hist=poisoned((n_q, H, D), dt), LSE_hist=poisoned((H, n_q), torch.float32),
                O_full=poisoned((n_q, H, D), dt), LSE_full=poisoned((H, n_q), torch.float32))


def _split(t: torch.Tensor, sizes):
    """Separate device buffers holding consecutive row ranges of t."""
    assert sum(sizes) == t.shape[0]
    out, r = [], 0
    for n in sizes:
        out.append(t[r:r + n].clone())
        r += n
    return out


def run_segments(x: inputs.ChunkInputs, scale, loc_sizes, hist_sizes):
    q = dev(x.q)
    n_q, H, D = q.shape
    kl, vl = dev(x.k_loc), dev(x.v_loc)
    loc = list(zip(_split(kl, loc_sizes), _split(vl, loc_sizes)))
    hist = []
    if hist_sizes:
        kh, vh = dev(x.k_hist), dev(x.v_hist)
        hist = list(zip(_split(kh, hist_sizes), _split(vh, hist_sizes)))
    out = _outputs(n_q, H, D, q.dtype)
    ispa.ispa_decomp_attn_segments(q, loc, hist, scale=scale, o_loc=out["O_loc"], lse_loc=out["LSE_loc"],
                                   o_hist=out["O_hist"], lse_hist=out["LSE_hist"], o_full=out["O_full"],
                                   lse_full=out["LSE_full"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case", [
    # (seed, n_q, loc segment sizes, hist segment sizes, H, D, dtype): ragged segments, several tiles
    (21, 300, (37, 100, 200), (5, 128, 77, 300), 2, 128, "bf16"),
    (22, 129, (1, 64, 1), (129, 1), 3, 128, "bf16"),
    (23, 200, (97,), (250,), 2, 64, "bf16"),
    (24, 257, (64, 66), (), 2, 128, "bf16"),
    (25, 130, (1,) * 5 + (40,), (3,) * 10, 2, 128, "bf16"),  # 16 segments
    (26, 150, (33, 31), (70, 1, 64), 2, 64, "f32"),
    (27, 77, (45,), (33, 12), 2, 128, "f32"),
])
def test_segments_parity(case):
    seed, n_q, ls, hs, H, D, dt = case
    say("case", case)
    x = inputs.custom_inputs(seed, n_q, sum(ls), sum(hs), H, D, dt, boost_rows=min(8, sum(ls)))
    scale = D ** -0.5
    out = run_segments(x, scale, ls, hs)
    tol_o, tol_l = (TOL_BF16_O, TOL_BF16_LSE) if dt == "bf16" else (TOL_F32, TOL_F32)
    say("report", check_against_oracle(x, out, scale, tol_o, tol_l))


@pytest.mark.parametrize("dt,unit", [("bf16", 128), ("f32", 32)])
def test_tile_aligned_segments_are_bitwise_the_two_buffer_call(dt, unit):
    """Segments whose sizes are multiples of the key tile give the same tiles in the same
    order as one local and one history buffer, so the results are identical bit for bit."""
    H, D = 2, 128
    ls, hs = (unit, 2 * unit), (unit, unit, 3 * unit)
    x = inputs.custom_inputs(31, 190, sum(ls), sum(hs), H, D, dt, boost_rows=8)
    seg = run_segments(x, D ** -0.5, ls, hs)
    ref = run_decomp(x, D ** -0.5)
    for n in NAMES:
        assert torch.equal(seg[n], ref[n]), n


def test_streaming_loop_with_rolling_history_and_eviction():
    """Chunks of one layer through the K/V cache: the history is the previous chunks (a rolling
    window of 3 that wraps the ring), each chunk attended in place; after eviction the layer
    attends to sink + chunk only and its full output is the local one."""
    seed, H, D, n_sink, ct, max_hist, dt = 41, 2, 128, 64, 192, 3, "bf16"
    scale = D ** -0.5
    cache = StreamingKVCache(1, H, D, n_sink, ct, max_hist, dtype=torch.bfloat16, device="cuda")
    sk, sv = inputs.stream_sink(seed, n_sink, H, D, dt)
    cache.sink(0)[0].copy_(dev(sk))
    cache.sink(0)[1].copy_(dev(sv))
    host_k, host_v = [], []  # every chunk's K/V as the generator drew them (oracle side)
    evict_at = 5
    for c in range(8):
        if c == evict_at:
            cache.evict(0)
        ch = inputs.stream_chunk(seed, c, ct, ct, H, D, dt)
        host_k.append(ch.k.f64)
        host_v.append(ch.v.f64)
        cache.write_current(0, dev(ch.k), dev(ch.v))
        loc, hist = cache.segments(0)
        q = dev(ch.q)
        out = _outputs(ct, H, D, q.dtype)
        ispa.ispa_decomp_attn_segments(q, loc, hist, scale=scale, o_loc=out["O_loc"], lse_loc=out["LSE_loc"],
                                       o_hist=out["O_hist"], lse_hist=out["LSE_hist"], o_full=out["O_full"],
                                       lse_full=out["LSE_full"])
        torch.cuda.synchronize()
        first = 0 if c >= evict_at else max(0, c - max_hist)
        n_hist_chunks = 0 if c >= evict_at else c - first
        say("chunk", c, "history chunks", n_hist_chunks, "runs", cache.history_runs(0))
        kl = np.concatenate([sk.f64, host_k[c]], axis=0)
        vl = np.concatenate([sv.f64, host_v[c]], axis=0)
        if n_hist_chunks:
            kh = np.concatenate(host_k[first:c], axis=0)
            vh = np.concatenate(host_v[first:c], axis=0)
        else:
            kh = np.zeros((0, H, D))
            vh = np.zeros((0, H, D))
        ref = oracle.branch_outputs(ch.q.f64, kl, vl, kh, vh, scale)
        for n in ("O_loc", "O_full") + (("O_hist",) if n_hist_chunks else ()):
            assert maxabs(host64(out[n]), ref[n]) <= TOL_BF16_O, (c, n)
        for n in ("LSE_loc", "LSE_full") + (("LSE_hist",) if n_hist_chunks else ()):
            got = out[n].cpu().numpy().astype(np.float64)
            assert maxabs(got, ref[n]) <= TOL_BF16_LSE, (c, n)
        if not n_hist_chunks:
            assert torch.equal(out["O_full"], out["O_loc"])
            assert torch.all(torch.isneginf(out["LSE_hist"]))
        cache.commit(0)
