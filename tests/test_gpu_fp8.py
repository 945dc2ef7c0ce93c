"""GPU parity of the fp8 path against the float64 oracle: E4M3 quantisers (bit-exact codes and
scales), the W8A8 product, and the decomposable attention with fp8 queries and keys.

Inputs are seeded draws; the quantised operands handed to the product and the attention are the
oracle's codes and scales, never GPU outputs."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
from kv_cache_absorption_ispa_amd import inputs, ispa
from tests.gpu_util import TOL_BF16_LSE, TOL_BF16_O, dev, host64, maxabs, poisoned, relfro, say

pytestmark = pytest.mark.gpu


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("n,H,D,boost", [(300, 3, 128, True), (257, 2, 64, False), (1, 1, 128, False),
                                         (4680, 12, 128, True)])
def test_quantize_heads_bit_exact(n, H, D, boost):
    x = inputs.custom_inputs(71 + n, n, 1, 0, H, D, "bf16", boost_rows=0).q  # bf16 patterns
    raw = x.raw.copy()
    if boost:
        raw[: min(8, n)] = inputs.f32_to_bf16_bits(x.f32[: min(8, n)] * np.float32(4.0))
    t = inputs.Tensor(raw, "bf16")
    codes, scale = ofp8.quantize_per_head(t.f32)
    x8 = torch.full((n, H, D), 0xFF, dtype=torch.uint8, device="cuda")
    s = torch.full((H,), float("nan"), dtype=torch.float32, device="cuda")
    ispa.ispa_quantize_fp8_heads(dev(t), x8, s)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), scale)
    assert np.array_equal(x8.cpu().numpy(), codes)


def test_quantize_rows_and_cols_bit_exact():
    g = np.random.default_rng(4)
    a = inputs.Tensor(inputs.f32_to_bf16_bits((g.standard_normal((333, 256)) * g.uniform(0.1, 5, (333, 1)))
                                              .astype(np.float32)), "bf16")
    a8 = torch.full((333, 256), 0xFF, dtype=torch.uint8, device="cuda")
    sa = torch.full((333,), float("nan"), dtype=torch.float32, device="cuda")
    ispa.ispa_quantize_fp8_rows(dev(a), a8, sa)
    W = (g.standard_normal((256, 384)) / 16).astype(np.float32)
    W[:, 7] = 0.0  # an all-zero column: scale 1, codes 0
    w8t = torch.full((384, 256), 0xFF, dtype=torch.uint8, device="cuda")
    sw = torch.full((384,), float("nan"), dtype=torch.float32, device="cuda")
    ispa.ispa_quantize_fp8_cols(_f32(W), w8t, sw)
    torch.cuda.synchronize()
    sa_ref = ofp8.absmax_scale(a.f32, axis=1)
    sw_ref = ofp8.absmax_scale(W, axis=0)
    assert np.array_equal(sa.cpu().numpy(), sa_ref)
    assert np.array_equal(a8.cpu().numpy(), ofp8.quantize(a.f32, sa_ref[:, None]))
    assert np.array_equal(sw.cpu().numpy(), sw_ref) and sw_ref[7] == 1.0
    assert np.array_equal(w8t.cpu().numpy(), ofp8.quantize(W, sw_ref[None, :]).T)


@pytest.mark.parametrize("n,d,d_out", [(300, 256, 384), (1, 64, 128), (4680, 1536, 1536)])
def test_w8a8_gemm_parity(n, d, d_out):
    g = np.random.default_rng(n + d)
    a = (g.standard_normal((n, d)) * 0.3).astype(np.float32)
    W = (g.standard_normal((d, d_out)) / np.sqrt(d)).astype(np.float32)
    sa, sw = ofp8.absmax_scale(a, axis=1), ofp8.absmax_scale(W, axis=0)
    a8, w8 = ofp8.quantize(a, sa[:, None]), ofp8.quantize(W, sw[None, :])
    ad, wd = ofp8.dequantize(a8, sa[:, None]), ofp8.dequantize(w8, sw[None, :])
    ref = ad @ wd
    assert np.array_equal(ref, ofp8.w8a8_matmul(a, W))
    y = poisoned((n, d_out), torch.bfloat16)
    ispa.ispa_w8a8_gemm(_u8(a8), _f32(sa), _u8(w8.T), _f32(sw), y)
    torch.cuda.synchronize()
    got = host64(y)
    # bf16 rounding of the output (half an ulp: <= 2^-8 relative) plus the float32 summation of d exact
    # code products (the textbook bound d * 2^-24 * sum |a_k w_k|; the scale products round once more)
    bound = 2.0 ** -8 * np.abs(ref) + (d + 2) * 2.0 ** -24 * (np.abs(ad) @ np.abs(wd))
    err = np.abs(got - ref)
    say("w8a8 max err / bound", float(np.max(err / bound)), "relfro", relfro(got, ref))
    assert np.all(err <= bound)


def _fp8k_inputs(x: inputs.ChunkInputs, loc_sizes, hist_sizes):
    """Oracle quantisation: Q per head, K per head within each segment; V stays bf16."""
    q8, qs = ofp8.quantize_per_head(x.q.f32)
    segs, kd = [], []
    for kt, vt, sizes in ((x.k_loc, x.v_loc, loc_sizes), (x.k_hist, x.v_hist, hist_sizes)):
        r = 0
        part = []
        for n in sizes:
            k8, ks = ofp8.quantize_per_head(kt.f32[r:r + n])
            part.append((k8, ks, vt.raw[r:r + n]))
            kd.append(ofp8.dequantize(k8, ks[None, :, None]))
            r += n
        segs.append(part)
    return q8, qs, segs, kd


def _run_fp8k(q8, qs, segs, H, D, n_q, scale):
    dv = lambda raw: torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()
    loc = [(_u8(k8), _f32(ks), dv(v)) for k8, ks, v in segs[0]]
    hist = [(_u8(k8), _f32(ks), dv(v)) for k8, ks, v in segs[1]]
    out = dict(O_loc=poisoned((n_q, H, D), torch.bfloat16), LSE_loc=poisoned((H, n_q), torch.float32),
               O_hist=poisoned((n_q, H, D), torch.bfloat16), LSE_hist=poisoned((H, n_q), torch.float32),
               O_full=poisoned((n_q, H, D), torch.bfloat16), LSE_full=poisoned((H, n_q), torch.float32))
    ispa.ispa_decomp_attn_fp8k(_u8(q8), _f32(qs), loc, hist, scale=scale, o_loc=out["O_loc"], lse_loc=out["LSE_loc"],
                               o_hist=out["O_hist"], lse_hist=out["LSE_hist"], o_full=out["O_full"],
                               lse_full=out["LSE_full"])
    torch.cuda.synchronize()
    return out


def _check(x, q8, qs, kd, out, H, scale, n_loc_kd, rows=None):
    qd = ofp8.dequantize(q8, qs[None, :, None])
    kl = np.concatenate(kd[:n_loc_kd]) if n_loc_kd else np.zeros((0,) + qd.shape[1:])
    kh = np.concatenate(kd[n_loc_kd:]) if len(kd) > n_loc_kd else np.zeros((0,) + qd.shape[1:])
    if rows is not None:
        qd = qd[rows]
    ref = oracle.branch_outputs(qd, kl, x.v_loc.f64, kh, x.v_hist.f64, scale)
    rep = {}
    for nm in ("O_loc", "O_hist", "O_full"):
        got = host64(out[nm]) if rows is None else host64(out[nm])[rows]
        rep[nm] = maxabs(got, ref[nm])
        assert rep[nm] <= TOL_BF16_O, (nm, rep[nm])
    for nm in ("LSE_loc", "LSE_hist", "LSE_full"):
        got = out[nm].cpu().numpy().astype(np.float64)
        got = got if rows is None else got[:, rows]
        if kh.shape[0] == 0 and nm == "LSE_hist":
            assert np.all(np.isneginf(got))
            continue
        rep[nm] = maxabs(got, ref[nm])
        assert rep[nm] <= TOL_BF16_LSE, (nm, rep[nm])
    return rep


@pytest.mark.parametrize("case", [
    # (seed, n_q, loc sizes, hist sizes, H, D)
    (81, 300, (200,), (333,), 2, 128),
    (82, 129, (64, 1, 66), (129, 300), 3, 128),
    (83, 200, (97,), (250,), 2, 64),
    (84, 257, (130,), (), 2, 128),
    (85, 1, (1,), (1,), 1, 128),
])
def test_fp8k_attention_parity(case):
    seed, n_q, ls, hs, H, D = case
    say("case", case)
    x = inputs.custom_inputs(seed, n_q, sum(ls), sum(hs), H, D, "bf16", boost_rows=min(8, sum(ls)))
    scale = D ** -0.5
    q8, qs, segs, kd = _fp8k_inputs(x, ls, hs)
    out = _run_fp8k(q8, qs, segs, H, D, n_q, scale)
    for nm, t in out.items():
        assert not torch.isnan(t).any().item(), nm
    say("report", _check(x, q8, qs, kd, out, H, scale, len(ls)))


def test_fp8k_attention_full_size_sampled_rows():
    """The Wan-1.3B layer with fp8 Q and K (sink, chunk and a 3-chunk history as separate segments)."""
    cfg = inputs.WAN13B_LAYER
    x = inputs.chunk_inputs(cfg, 0, 0)
    ls, hs = (cfg.n_sink, cfg.n_chunk), (cfg.n_chunk,) * (cfg.n_hist // cfg.n_chunk)
    q8, qs, segs, kd = _fp8k_inputs(x, ls, hs)
    out = _run_fp8k(q8, qs, segs, cfg.heads, cfg.head_dim, cfg.n_q, cfg.scale)
    for nm, t in out.items():
        assert not torch.isnan(t).any().item(), nm
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(cfg.n_q - 80, cfg.n_q),
                                     g.choice(cfg.n_q, 24, replace=False)]))
    say("report", _check(x, q8, qs, kd, out, cfg.heads, cfg.scale, len(ls), rows=rows))
