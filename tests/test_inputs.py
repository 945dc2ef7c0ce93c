"""The seeded input generator: determinism, shapes, the sink boost, and the bf16 encoding (CPU only)."""
import numpy as np
import torch

from kv_cache_absorption_ispa_amd import inputs


def test_bf16_rne_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32),
        (g.standard_normal(20000) * 1e-30).astype(np.float32),
        (g.standard_normal(20000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 1.00390625, 1.01171875], dtype=np.float32),
    ])
    # exact ties (halfway between two bf16 values) in both directions
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_distinct():
    cfg = inputs.TINY_F32
    a = inputs.chunk_inputs(cfg, 0, 0)
    b = inputs.chunk_inputs(cfg, 0, 0)
    c = inputs.chunk_inputs(cfg, 0, 1)
    assert np.array_equal(a.q.raw, b.q.raw) and np.array_equal(a.v_hist.raw, b.v_hist.raw)
    assert not np.array_equal(a.q.raw, c.q.raw)
    # sink rows are per layer: shared by the chunks of a layer
    assert np.array_equal(a.k_loc.raw[: cfg.n_sink], c.k_loc.raw[: cfg.n_sink])
    assert not np.array_equal(a.k_loc.raw[cfg.n_sink:], c.k_loc.raw[cfg.n_sink:])


def test_shapes_and_boost():
    cfg = inputs.WAN13B_LAYER
    x = inputs.chunk_inputs(cfg, 0, 0, n_hist=64)
    assert x.q.shape == (4680, 12, 128) and x.q.raw.dtype == np.uint16
    assert x.k_loc.shape == (cfg.n_loc, 12, 128)
    assert x.k_hist.shape == (64, 12, 128)
    ks, vs = inputs.sink_kv(cfg, 0)
    kraw = inputs.normal(1, 0, inputs.LAYER_CHUNK, inputs.T_KS, (cfg.n_sink, 12, 128))
    assert np.array_equal(ks[:8], 4 * kraw[:8]) and np.array_equal(ks[8:], kraw[8:])
    assert np.array_equal(x.k_loc.raw[:cfg.n_sink], inputs.f32_to_bf16_bits(ks))


def test_weight_scale():
    cfg = inputs.WAN13B_LAYER
    W = inputs.weight(cfg, 0)
    assert W.shape == (1536, 1536) and W.dtype == np.float32
    assert abs(W.std() * np.sqrt(1536) - 1) < 0.01


def test_flop_counts():
    cfg = inputs.WAN13B_LAYER
    assert abs(cfg.attn_flops() - 5.83e11) / 5.83e11 < 0.01
    assert cfg.gram_rows == 18720
