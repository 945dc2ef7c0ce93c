"""Seeded synthetic inputs shared by the GPU path's callers and by the oracle's tests.

This module draws data and encodes it; it holds none of the method's arithmetic
(no attention, no merge, no Gram, no solve).  Every array is a pure function of
(config, layer, chunk, tensor id), so the GPU path and the oracle see the same bits.

Recipe (the pages give no data; the shapes are the Wan-shaped layers the
benchmark names, the distributions are stated here):

* Seeds: ``SeedSequence([2607, cfg, layer, chunk, tensor_id])`` feeding PCG64.
  tensor ids: 0 Q, 1 K_chunk, 2 V_chunk, 3 K_hist, 4 V_hist, 5 K_sink, 6 V_sink,
  7 W, 8..12 the stand-in attention rows for the Gram/solve step (see
  :func:`absorb_rows`).  Per-layer tensors (sink K/V, W, stand-in rows) use
  chunk id 255; the post-absorb chunk is chunk 4.
* Q, K, V ~ N(0, 1), drawn float32 in [tokens, heads, head_dim] order.  In the
  bf16 configurations the first 8 sink keys (all heads) are multiplied by 4
  before rounding; V is never boosted.
* The sink block is drawn once per layer and is shared by that layer's chunks;
  Q, the chunk K/V and the history K/V are fresh per chunk.  The local key set
  handed to the attention call is the sink rows followed by the chunk rows.
* W ~ N(0, 1/d), float32, kept float32.
* Streaming sequences (:func:`stream_sink`, :func:`stream_chunk`) use
  cfg id 300 + seed: a sink drawn once, then per chunk Q and the chunk's own
  K/V; a chunk's history is the K/V of the chunks before it.
* bf16 values are made from the float32 draws by round-to-nearest-even on the
  host (:func:`f32_to_bf16_bits`); the GPU receives the 16-bit patterns and the
  oracle receives the exact same values widened to float64.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_ROOT = 2607
LAYER_CHUNK = 255  # chunk id used for per-layer tensors

T_Q, T_KC, T_VC, T_KH, T_VH, T_KS, T_VS, T_W = range(8)
T_AROW_BASE = 8  # 8..12: stand-in rows for the Gram / solve step


# --------------------------------------------------------------------------- #
# Workload shapes
# --------------------------------------------------------------------------- #
@dataclass(frozen=True)
class LayerConfig:
    """One attention layer's warmup workload."""

    cfg_id: int
    name: str
    heads: int
    head_dim: int
    n_q: int  # queries per chunk
    n_sink: int
    n_chunk: int  # keys of the current chunk (== n_q here)
    n_hist: int
    dtype: str  # "f32" or "bf16"
    n_chunks: int = 4  # warmup chunks (12 latent frames at 3 frames / chunk)
    lam: float = 1e-2
    sink_boost: float = 4.0
    n_boost: int = 8  # number of boosted sink keys (bf16 configs only)
    n_layers: int = 1
    n_absorb: int = 0  # layers converted to local attention (stack only)

    @property
    def d(self) -> int:
        return self.heads * self.head_dim

    @property
    def n_loc(self) -> int:
        return self.n_sink + self.n_chunk

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def gram_rows(self) -> int:
        return self.n_chunks * self.n_q

    def attn_flops(self, n_hist: int | None = None) -> float:
        """Matmul FLOPs of one pass over local+history keys (4 * Nq * Nk * D * H)."""
        nh = self.n_hist if n_hist is None else n_hist
        return 4.0 * self.n_q * (self.n_loc + nh) * self.head_dim * self.heads


CONFIGS = {
    # tiny fp32 layer the oracle finishes in seconds
    0: LayerConfig(0, "tiny-fp32", heads=2, head_dim=64, n_q=256, n_sink=64, n_chunk=256,
                   n_hist=1024, dtype="f32"),
    # Wan-1.3B-shaped layer: 3 latent frames x 1560 tokens per chunk, 1 sink frame, 9 history frames
    1: LayerConfig(1, "wan1.3b-layer", heads=12, head_dim=128, n_q=4680, n_sink=1560, n_chunk=4680,
                   n_hist=14040, dtype="bf16"),
    # same layer with 21 history frames
    2: LayerConfig(2, "wan1.3b-long-history", heads=12, head_dim=128, n_q=4680, n_sink=1560,
                   n_chunk=4680, n_hist=32760, dtype="bf16"),
    # Wan-14B-shaped layer
    3: LayerConfig(3, "wan14b-layer", heads=40, head_dim=128, n_q=4680, n_sink=1560, n_chunk=4680,
                   n_hist=14040, dtype="bf16"),
    # 30-layer stack of the 1.3B layer, half of them absorbed
    4: LayerConfig(4, "wan1.3b-stack30", heads=12, head_dim=128, n_q=4680, n_sink=1560, n_chunk=4680,
                   n_hist=14040, dtype="bf16", n_layers=30, n_absorb=15),
}
BY_NAME = {c.name: c for c in CONFIGS.values()}
TINY_F32 = BY_NAME["tiny-fp32"]
WAN13B_LAYER = BY_NAME["wan1.3b-layer"]
WAN13B_LONG_HISTORY = BY_NAME["wan1.3b-long-history"]
WAN14B_LAYER = BY_NAME["wan14b-layer"]
WAN13B_STACK30 = BY_NAME["wan1.3b-stack30"]


# --------------------------------------------------------------------------- #
# Encoding
# --------------------------------------------------------------------------- #
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the uint16 patterns.

    Finite inputs only (the draws here are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 patterns to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """A host array in the representation the GPU receives plus its exact float64 value.

    ``raw`` is float32 (fp32 configs) or the uint16 bf16 patterns (bf16 configs)."""

    raw: np.ndarray
    dtype: str

    @property
    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.raw).astype(np.float64)
        return self.raw.astype(np.float64)

    @property
    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.raw)
        return self.raw

    @property
    def shape(self):
        return self.raw.shape


def _encode(x32: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        return Tensor(f32_to_bf16_bits(x32), "bf16")
    return Tensor(np.ascontiguousarray(x32, dtype=np.float32), "f32")


def rng_for(cfg_id: int, layer: int, chunk: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, cfg_id, layer, chunk, tensor_id]))


def normal(cfg_id: int, layer: int, chunk: int, tensor_id: int, shape) -> np.ndarray:
    return rng_for(cfg_id, layer, chunk, tensor_id).standard_normal(shape, dtype=np.float32)


# --------------------------------------------------------------------------- #
# Attention inputs
# --------------------------------------------------------------------------- #
@dataclass
class ChunkInputs:
    q: Tensor  # [n_q, H, D]
    k_loc: Tensor  # [n_loc, H, D]  (sink rows, then chunk rows)
    v_loc: Tensor
    k_hist: Tensor  # [n_hist, H, D]
    v_hist: Tensor


def sink_kv(cfg: LayerConfig, layer: int = 0, cfg_id: int | None = None):
    """Per-layer sink K and V (float32 before rounding), boost applied to K only."""
    cid = cfg.cfg_id if cfg_id is None else cfg_id
    shp = (cfg.n_sink, cfg.heads, cfg.head_dim)
    ks = normal(cid, layer, LAYER_CHUNK, T_KS, shp)
    vs = normal(cid, layer, LAYER_CHUNK, T_VS, shp)
    if cfg.dtype == "bf16" and cfg.n_boost > 0:
        ks[: cfg.n_boost] *= np.float32(cfg.sink_boost)
    return ks, vs


def chunk_inputs(cfg: LayerConfig, layer: int = 0, chunk: int = 0, *, n_q: int | None = None,
                 n_hist: int | None = None, cfg_id: int | None = None) -> ChunkInputs:
    """Q, local K/V (sink + chunk) and history K/V of one chunk of one layer.

    ``n_q`` / ``n_hist`` override the sizes (the prefix of the full draw is NOT
    used; a different size is a different draw)."""
    cid = cfg.cfg_id if cfg_id is None else cfg_id
    H, D = cfg.heads, cfg.head_dim
    nq = cfg.n_q if n_q is None else n_q
    nh = cfg.n_hist if n_hist is None else n_hist
    q = normal(cid, layer, chunk, T_Q, (nq, H, D))
    kc = normal(cid, layer, chunk, T_KC, (cfg.n_chunk, H, D))
    vc = normal(cid, layer, chunk, T_VC, (cfg.n_chunk, H, D))
    kh = normal(cid, layer, chunk, T_KH, (nh, H, D))
    vh = normal(cid, layer, chunk, T_VH, (nh, H, D))
    ks, vs = sink_kv(cfg, layer, cid)
    k_loc = np.concatenate([ks, kc], axis=0)
    v_loc = np.concatenate([vs, vc], axis=0)
    return ChunkInputs(_encode(q, cfg.dtype), _encode(k_loc, cfg.dtype), _encode(v_loc, cfg.dtype),
                       _encode(kh, cfg.dtype), _encode(vh, cfg.dtype))


def custom_inputs(seed: int, n_q: int, n_loc: int, n_hist: int, heads: int, head_dim: int,
                  dtype: str, boost_rows: int = 0) -> ChunkInputs:
    """Free-shape inputs for parity sweeps (ragged sizes, edge cases); same recipe."""
    H, D = heads, head_dim
    q = normal(100 + seed, 0, 0, T_Q, (n_q, H, D))
    kl = normal(100 + seed, 0, 0, T_KC, (n_loc, H, D))
    vl = normal(100 + seed, 0, 0, T_VC, (n_loc, H, D))
    kh = normal(100 + seed, 0, 0, T_KH, (n_hist, H, D))
    vh = normal(100 + seed, 0, 0, T_VH, (n_hist, H, D))
    if boost_rows:
        kl[:boost_rows] *= np.float32(4.0)
    return ChunkInputs(_encode(q, dtype), _encode(kl, dtype), _encode(vl, dtype),
                       _encode(kh, dtype), _encode(vh, dtype))


def planted_inputs(seed: int, n_q: int, n_loc: int, n_hist: int, heads: int, head_dim: int, dtype: str,
                   loc_rows=(), hist_rows=(), factor: float = 24.0, boost_rows: int = 8) -> ChunkInputs:
    """custom_inputs with some keys made dominant late in a branch: the K rows listed in ``loc_rows``
    (local) and ``hist_rows`` (history), all heads, are multiplied by ``factor`` before rounding.
    Their scores spread over ``factor`` times the usual range, so for many queries such a key beats
    every earlier key of its branch by a wide margin (the online softmax then has to move its
    reference maximum in the middle of the branch)."""
    x = custom_inputs(seed, n_q, n_loc, n_hist, heads, head_dim, "f32", boost_rows=boost_rows)
    kl = x.k_loc.raw.copy()
    kh = x.k_hist.raw.copy()
    for r in loc_rows:
        kl[r] *= np.float32(factor)
    for r in hist_rows:
        kh[r] *= np.float32(factor)
    return ChunkInputs(_encode(x.q.raw, dtype), _encode(kl, dtype), _encode(x.v_loc.raw, dtype),
                       _encode(kh, dtype), _encode(x.v_hist.raw, dtype))


@dataclass
class StreamChunk:
    q: Tensor  # [n_q, H, D]
    k: Tensor  # [n_chunk, H, D]: this chunk's own keys (history of the later chunks)
    v: Tensor


def stream_sink(seed: int, n_sink: int, heads: int, head_dim: int, dtype: str):
    """Sink K and V of a streaming sequence (first 8 keys boosted x4 in bf16, as in the configs)."""
    shp = (n_sink, heads, head_dim)
    ks = normal(300 + seed, 0, LAYER_CHUNK, T_KS, shp)
    vs = normal(300 + seed, 0, LAYER_CHUNK, T_VS, shp)
    if dtype == "bf16":
        ks[:8] *= np.float32(4.0)
    return _encode(ks, dtype), _encode(vs, dtype)


def stream_chunk(seed: int, chunk: int, n_q: int, n_chunk: int, heads: int, head_dim: int,
                 dtype: str) -> StreamChunk:
    """Queries and own K/V of chunk ``chunk`` of a streaming sequence.  The history
    a chunk attends to is the K/V of the chunks before it, so these draws are
    all a streaming test needs."""
    H, D = heads, head_dim
    q = normal(300 + seed, 0, chunk, T_Q, (n_q, H, D))
    k = normal(300 + seed, 0, chunk, T_KC, (n_chunk, H, D))
    v = normal(300 + seed, 0, chunk, T_VC, (n_chunk, H, D))
    return StreamChunk(_encode(q, dtype), _encode(k, dtype), _encode(v, dtype))


def weight(cfg: LayerConfig, layer: int = 0, d_out: int | None = None, cfg_id: int | None = None) -> np.ndarray:
    """Output-projection weight W [d, d_out], N(0, 1/d), float32 (row-vector convention y = a W)."""
    cid = cfg.cfg_id if cfg_id is None else cfg_id
    dout = cfg.d if d_out is None else d_out
    return normal(cid, layer, LAYER_CHUNK, T_W, (cfg.d, dout)) * np.float32(1.0 / np.sqrt(cfg.d))


# --------------------------------------------------------------------------- #
# Stand-in attention rows for the Gram / solve step
# --------------------------------------------------------------------------- #
def absorb_rows(cfg_id: int, layer: int, n_rows: int, d: int, dtype: str, mismatch: float = 1.0,
                diff_scale: float = 1.0):
    """Stand-in rows (A_loc, A_full), each [n_rows, d], for testing the Gram and solve step.

    The Gram/solve step consumes attention outputs; a test of it may not take its
    inputs from the GPU attention, and the oracle's own attention at full size
    takes minutes.  These rows reproduce what matters to that step, calibrated
    against the oracle's attention rows of the Wan-1.3B layer (one 4680-row
    chunk: condition number of G + lambda*I 1.8e5, eigenvalues 0.13..2.4e4, rms
    0.25): per-column scales spread over 1.85 decades plus a shared rank-one
    component give, at that size, condition number 1.9e5, eigenvalues
    0.16..3.1e4 and rms 0.20.  A_full is A_loc plus a per-column modulation and
    independent noise (so the ridge solution is non-trivial).  ``mismatch`` scales the noise part, giving
    layers of a stack different reconstruction errors.  ``diff_scale`` scales the whole difference
    A_full - A_loc (modulation and noise): small values give layers whose full and local rows nearly
    agree (the layers a stack converts first).
    """
    g = rng_for(cfg_id, layer, LAYER_CHUNK, T_AROW_BASE)
    perm = g.permutation(d).astype(np.float32)
    s = (0.55 * 10.0 ** (-1.85 * perm / max(d - 1, 1))).astype(np.float32)
    b = (0.065 * g.standard_normal(d)).astype(np.float32)
    m = (0.1 * g.standard_normal(d)).astype(np.float32)
    z = normal(cfg_id, layer, LAYER_CHUNK, T_AROW_BASE + 1, (n_rows, d))
    u = normal(cfg_id, layer, LAYER_CHUNK, T_AROW_BASE + 2, (n_rows, 1))
    e = normal(cfg_id, layer, LAYER_CHUNK, T_AROW_BASE + 3, (n_rows, d))
    a_loc = z * s + u * b
    if diff_scale == 1.0:
        a_full = a_loc * (np.float32(1.0) + m) + np.float32(0.3 * mismatch) * e * s
    else:
        a_full = a_loc + np.float32(diff_scale) * (a_loc * m + np.float32(0.3 * mismatch) * e * s)
    return _encode(a_loc.astype(np.float32), dtype), _encode(a_full.astype(np.float32), dtype)
