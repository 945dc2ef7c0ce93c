"""Host bookkeeping of the streaming K/V cache (CPU tensors; no attention is computed here).

Each chunk's K is filled with its chunk number (V with that + 0.5), so the segment lists can be
checked against the history the streaming loop must see: the last
``max_hist_chunks`` chunks, oldest first, then the sink and the current chunk."""
import pytest
import torch

from kv_cache_absorption_ispa_amd.kv_cache import StreamingKVCache


def _chunk_ids(segs, ct):
    """Chunk number of every chunk-sized block in the concatenated segments."""
    if not segs:
        return []
    k = torch.cat([s[0] for s in segs], dim=0)
    v = torch.cat([s[1] for s in segs], dim=0)
    assert torch.equal(k, v - 0.5)
    assert k.shape[0] % ct == 0
    blocks = k.reshape(-1, ct, *k.shape[1:])
    ids = []
    for b in blocks:
        assert torch.all(b == b.flatten()[0])
        ids.append(int(b.flatten()[0]))
    return ids


@pytest.mark.parametrize("max_hist", [0, 1, 3, 5])
def test_history_window_and_order(max_hist):
    ct, H, D = 6, 2, 4
    cache = StreamingKVCache(2, H, D, n_sink=3, chunk_tokens=ct, max_hist_chunks=max_hist, dtype=torch.float32,
                             device="cpu")
    for layer in range(2):
        sk, sv = cache.sink(layer)
        sk.fill_(-1.0)
        sv.fill_(-0.5)
    for c in range(12):
        for layer in range(2):
            ck, cv = cache.current(layer)
            cache.write_current(layer, torch.full((ct, H, D), float(c)), torch.full((ct, H, D), float(c + 0.5)))
            loc, hist = cache.segments(layer)
            assert len(loc) == 2 and len(hist) <= 2
            assert torch.all(loc[0][0] == -1.0) and torch.all(loc[0][1] == -0.5)
            assert _chunk_ids([loc[1]], ct) == [c]
            want = list(range(max(0, c - max_hist), c))
            assert _chunk_ids(hist, ct) == want
            assert cache.history_tokens(layer) == len(want) * ct
            # segments are views of the cache's storage: no copies
            assert loc[1][0].data_ptr() == ck.data_ptr()
            for s in hist:
                base = cache.ring_k[layer]
                assert base.data_ptr() <= s[0].data_ptr() < base.data_ptr() + base.numel() * base.element_size()
            cache.commit(layer)


def test_ring_wraps_into_two_runs():
    cache = StreamingKVCache(1, 1, 4, n_sink=0, chunk_tokens=2, max_hist_chunks=3, dtype=torch.float32, device="cpu")
    seen_two = False
    for c in range(9):
        cache.write_current(0, torch.full((2, 1, 4), float(c)), torch.full((2, 1, 4), float(c + 0.5)))
        loc, hist = cache.segments(0)
        assert len(loc) == 1  # no sink
        runs = cache.history_runs(0)
        assert sum(n for _, n in runs) == min(c, 3)
        seen_two |= len(runs) == 2
        assert _chunk_ids(hist, 2) == list(range(max(0, c - 3), c))
        cache.commit(0)
    assert seen_two


def test_evict_keeps_sink_and_current_only():
    ct, H, D = 4, 2, 8
    cache = StreamingKVCache(3, H, D, n_sink=5, chunk_tokens=ct, max_hist_chunks=4, dtype=torch.bfloat16,
                             device="cpu")
    full = cache.resident_bytes()
    per_layer = 2 * (5 + 5 * ct) * H * D * 2
    assert full == 3 * per_layer
    for c in range(3):
        for layer in range(3):
            cache.write_current(layer, torch.full((ct, H, D), float(c)), torch.full((ct, H, D), float(c + 0.5)))
            cache.commit(layer)
    cache.evict(1)
    assert cache.resident_bytes(1) == 2 * (5 + ct) * H * D * 2
    assert cache.resident_bytes() == full - 2 * 4 * ct * H * D * 2
    loc, hist = cache.segments(1)
    assert hist == [] and len(loc) == 2 and cache.history_tokens(1) == 0
    cache.write_current(1, torch.full((ct, H, D), 7.0), torch.full((ct, H, D), 7.5))
    assert _chunk_ids([cache.segments(1)[0][1]], ct) == [7]
    cache.commit(1)
    assert cache.segments(1)[1] == [] and cache.chunks_committed[1] == 4
    # the other layers keep their history
    assert _chunk_ids(cache.segments(0)[1], ct) == [0, 1, 2]


def test_bad_shapes_rejected():
    with pytest.raises(ValueError):
        StreamingKVCache(0, 1, 4, 0, 2, 1, device="cpu")
    with pytest.raises(ValueError):
        StreamingKVCache(1, 1, 4, 0, 0, 1, device="cpu")
