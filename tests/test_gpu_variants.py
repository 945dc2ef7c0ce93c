"""GPU parity of the selection and lambda variants (ispa_fit_error, ispa_lambda_from_trace,
ispa_absorb_solve_lambdas, ispa_select_layers_below, ispa_gather_layers,
ispa_absorb_apply_compact) and of the layer stack under each policy, against the float64 oracle.

Inputs are the seeded stand-in rows or the oracle's own attention rows, never GPU outputs."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_absorption_ispa_amd import inputs, ispa
from kv_cache_absorption_ispa_amd.stack import LayerStack
from tests.gpu_util import TOL_DW, dev, host64, nan_workspace, poisoned, relfro, say
from tests.test_gpu_absorb import gpu_gram, gpu_solve

pytestmark = pytest.mark.gpu

D = 256


def _weight(seed, layer):
    return inputs.normal(seed, layer, inputs.LAYER_CHUNK, inputs.T_W, (D, D)) * np.float32(D ** -0.5)


def _eps(out_abs, out_rel):
    torch.cuda.synchronize()
    return out_abs.cpu().numpy(), out_rel.cpu().numpy()


def test_fit_error_before_the_fit_and_on_held_out_rows():
    """dW = 0: ||(A_full - A_loc) W||^2 on the fitted rows.  dW fitted on other rows: the residual on
    rows the fit did not see.  Both against the oracle's explicit residual."""
    b = 3
    Gs, Cs, Qs, Hg, Hc, Hq, Ws, dWs, pre_ref, ho_ref = ([] for _ in range(10))
    for layer in range(b):
        al, af = inputs.absorb_rows(12, layer, 3000, D, "bf16", mismatch=0.5 + layer)
        hl, hf = inputs.absorb_rows(13, layer, 1000, D, "bf16", mismatch=0.5 + layer)
        G, C, Q = gpu_gram([(al, af)], D, qff=True)
        G2, C2, Q2 = gpu_gram([(hl, hf)], D, qff=True)
        W = _weight(12, layer)
        Gr, Cr = oracle.gram(al.f64, af.f64)
        dWr = oracle.ridge_solve(Gr, Cr, W.astype(np.float64), 1e-2).astype(np.float32)
        for lst, v in ((Gs, G), (Cs, C), (Qs, Q), (Hg, G2), (Hc, C2), (Hq, Q2)):
            lst.append(v)
        Ws.append(torch.from_numpy(W).cuda())
        dWs.append(torch.from_numpy(dWr).cuda())
        pre_ref.append(oracle.reconstruction_error(al.f64, af.f64, W.astype(np.float64), np.zeros((D, D))))
        ho_ref.append(oracle.reconstruction_error(hl.f64, hf.f64, W.astype(np.float64), dWr.astype(np.float64)))
    G, C, Q, G2, C2, Q2, W, dW = (torch.stack(x) for x in (Gs, Cs, Qs, Hg, Hc, Hq, Ws, dWs))
    ea = torch.full((b,), float("nan"), dtype=torch.float64, device="cuda")
    er = torch.full_like(ea, float("nan"))
    ispa.ispa_fit_error(G, C, Q, W, None, ea, er)
    pa, pr = _eps(ea, er)
    ispa.ispa_fit_error(G2, C2, Q2, W, dW, ea, er)
    ha, hr = _eps(ea, er)
    for i in range(b):
        say("pre-fit eps_rel gpu / oracle", pr[i], pre_ref[i][1], "held-out", hr[i], ho_ref[i][1])
        assert abs(pr[i] - pre_ref[i][1]) <= 1e-4 * pre_ref[i][1]
        assert abs(pa[i] - pre_ref[i][0]) <= 1e-4 * pre_ref[i][0]
        assert abs(hr[i] - ho_ref[i][1]) <= 1e-3 * ho_ref[i][1] + 1e-5
        assert abs(ha[i] - ho_ref[i][0]) <= 1e-3 * ho_ref[i][0] + 1e-5 * ho_ref[i][0] / max(ho_ref[i][1], 1e-30)
    # on the fitted rows with the fitted dW the general form agrees with the normal-equation form
    dWg, info = gpu_solve(G, C, W, 1e-2)
    ispa.ispa_fit_error(G, C, Q, W, dWg, ea, er)
    _, gen = _eps(ea, er)
    ea2, er2 = torch.empty_like(ea), torch.empty_like(er)
    ispa.ispa_layer_eps(G, C, Q, W, dWg, 1e-2, ea2, er2,
                        workspace=nan_workspace(ispa.ispa_eps_workspace_size(D, D, b)))
    _, ne = _eps(ea2, er2)
    assert np.all(np.abs(gen - ne) <= 1e-3 * ne + 1e-6)


def test_trace_lambda_and_per_layer_solve():
    """lambda_b = scale * tr(G_b) / d, then the solve with that lambda per layer, against the oracle's
    solve with the oracle's lambda on the same (float32-rounded) statistics."""
    b, scale = 3, 1e-3
    Gs, Cs, Ws, refs, lam_ref = [], [], [], [], []
    for layer in range(b):
        al, af = inputs.absorb_rows(14, layer, 2000, D, "f32", mismatch=1.0 + layer)
        Gr, Cr = oracle.gram(al.f64, af.f64)
        G32, C32 = Gr.astype(np.float32), Cr.astype(np.float32)
        W = _weight(14, layer)
        lam = oracle.trace_scaled_lambda(G32.astype(np.float64), scale)
        lam_ref.append(lam)
        refs.append(oracle.ridge_solve(G32.astype(np.float64), C32.astype(np.float64), W.astype(np.float64), lam))
        Gs.append(torch.from_numpy(G32).cuda())
        Cs.append(torch.from_numpy(C32).cuda())
        Ws.append(torch.from_numpy(W).cuda())
    G, C, W = (torch.stack(x) for x in (Gs, Cs, Ws))
    lam = torch.full((b,), float("nan"), dtype=torch.float32, device="cuda")
    ispa.ispa_lambda_from_trace(G, scale, lam)
    dW = poisoned(W.shape, torch.float32)
    info = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    ispa.ispa_absorb_solve_lambdas(G, C, W, lam, dW, info,
                                   workspace=nan_workspace(ispa.ispa_absorb_workspace_size(D, D, b)))
    torch.cuda.synchronize()
    assert info.cpu().tolist() == [0] * b
    for i in range(b):
        say("lambda gpu / oracle", lam[i].item(), lam_ref[i], "dW relfro", relfro(host64(dW[i]), refs[i]))
        assert abs(lam[i].item() - lam_ref[i]) <= 1e-6 * lam_ref[i]
        assert relfro(host64(dW[i]), refs[i]) <= TOL_DW
    # a constant per-layer lambda is the scalar solve, bit for bit
    const = torch.full((b,), 0.25, dtype=torch.float32, device="cuda")
    dW2 = poisoned(W.shape, torch.float32)
    ispa.ispa_absorb_solve_lambdas(G, C, W, const, dW2, info,
                                   workspace=nan_workspace(ispa.ispa_absorb_workspace_size(D, D, b)))
    dW3, _ = gpu_solve(G, C, W, 0.25)
    torch.cuda.synchronize()
    assert torch.equal(dW2, dW3)


@pytest.mark.parametrize("n,tau,k_max", [(8, 1.0, 8), (8, 1.0, 2), (40, 20.0, 40), (4096, 10.0, 1000),
                                         (4096, 10.0, 4096), (30, -1.0, 30)])
def test_select_below_matches_oracle(n, tau, k_max):
    g = np.random.default_rng(n + k_max)
    e_h = g.integers(0, 50, size=n).astype(np.float64)
    e_h[g.random(n) < 0.05] = np.nan
    if n == 8:
        e_h = np.array([3.0, 1.0, np.nan, 1.0, 0.5, 2.0, np.nan, 1.0])
    e = torch.from_numpy(e_h).cuda()
    sel = torch.full((k_max,), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rank = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    ispa.ispa_select_layers_below(e, tau, k_max, sel, cnt, rank)
    torch.cuda.synchronize()
    want = oracle.select_below(e_h, tau, k_max)
    c = cnt.item()
    assert c == len(want)
    assert sel.cpu().tolist()[:c] == want
    assert rank.cpu().tolist() == [int(r) for r in np.argsort(np.argsort(e_h, kind="stable"), kind="stable")]


def test_gather_and_compact_apply():
    n, d, do = 6, 128, 64
    g = np.random.default_rng(3)
    W_h = g.standard_normal((n, d, do)).astype(np.float32)
    dWc_h = g.standard_normal((3, d, do)).astype(np.float32)
    sel_h = [5, 0, 3]
    W = torch.from_numpy(W_h.copy()).cuda()
    sel = torch.tensor(sel_h, dtype=torch.int32, device="cuda")
    out = poisoned((3, d, do), torch.float32)
    ispa.ispa_gather_layers(W, sel, out)
    ispa.ispa_absorb_apply_compact(sel, torch.from_numpy(dWc_h).cuda(), W)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), W_h[sel_h])
    want = W_h.copy()
    for s, l in enumerate(sel_h):
        want[l] = W_h[l] + dWc_h[s]  # one float32 addition, as on the device
    assert np.array_equal(W.cpu().numpy(), want)


# ------------------------------------------------------------------ the stack under each policy
STACK = inputs.LayerConfig(15, "stack8-small", heads=1, head_dim=128, n_q=256, n_sink=64, n_chunk=256,
                           n_hist=512, dtype="bf16", n_layers=8, n_absorb=3)


def _oracle_rows(cfg, layer, chunk):
    x = inputs.chunk_inputs(cfg, layer, chunk)
    ref = oracle.branch_outputs(x.q.f64, x.k_loc.f64, x.v_loc.f64, x.k_hist.f64, x.v_hist.f64, cfg.scale)
    enc = lambda a: inputs.Tensor(inputs.f32_to_bf16_bits(a.reshape(cfg.n_q, cfg.d).astype(np.float32)), "bf16")
    return enc(ref["O_loc"]), enc(ref["O_full"])


@pytest.fixture(scope="module")
def stack_rows():
    cfg = STACK
    return {(l, c): _oracle_rows(cfg, l, c) for l in range(cfg.n_layers) for c in range(cfg.n_chunks)}


@pytest.mark.parametrize("selection,lam_policy,threshold", [
    ("prefit", "absolute", None), ("heldout", "absolute", None), ("postfit", "trace", None),
    ("postfit", "absolute", "median"), ("prefit", "trace", "median")])
def test_stack_policy_matches_oracle(stack_rows, selection, lam_policy, threshold):
    cfg = STACK
    L, K, d = cfg.n_layers, cfg.n_absorb, cfg.d
    lam0 = cfg.lam if lam_policy == "absolute" else 1e-4
    W0 = np.stack([inputs.weight(cfg, l) for l in range(L)])
    fit_chunks = range(cfg.n_chunks - 1) if selection == "heldout" else range(cfg.n_chunks)

    # oracle side: the policy's error per layer, its selection, and the chosen layers' dW
    eps_ref, dW_ref = [], []
    for l in range(L):
        al = np.concatenate([stack_rows[(l, c)][0].f64 for c in fit_chunks])
        af = np.concatenate([stack_rows[(l, c)][1].f64 for c in fit_chunks])
        G, C = oracle.gram(al, af)
        lam = lam0 if lam_policy == "absolute" else oracle.trace_scaled_lambda(G, lam0)
        dW = oracle.ridge_solve(G, C, W0[l].astype(np.float64), lam)
        dW_ref.append(dW)
        if selection == "prefit":
            eps_ref.append(oracle.reconstruction_error(al, af, W0[l], np.zeros_like(dW))[1])
        elif selection == "heldout":
            hl, hf = stack_rows[(l, cfg.n_chunks - 1)]
            eps_ref.append(oracle.reconstruction_error(hl.f64, hf.f64, W0[l], dW)[1])
        else:
            eps_ref.append(oracle.reconstruction_error(al, af, W0[l], dW)[1])
    eps_ref = np.array(eps_ref)
    tau = None if threshold is None else float(np.median(eps_ref))
    want = oracle.select_layers(eps_ref, K) if tau is None else oracle.select_below(eps_ref, tau, K)

    # GPU side
    st = LayerStack(torch.from_numpy(W0.copy()).cuda(), cfg.heads, cfg.head_dim, cfg.n_q, lam0, K,
                    selection=selection, lam_policy=lam_policy, threshold=tau)
    for c in range(cfg.n_chunks):
        for l in range(L):
            al, af = stack_rows[(l, c)]
            st.accumulate_rows(l, dev(al), dev(af), heldout=selection == "heldout" and c == cfg.n_chunks - 1)
    conv = st.transition()
    torch.cuda.synchronize()
    eps_gpu = st.eps_rel.cpu().numpy()
    say(selection, lam_policy, threshold, "eps max rel diff", np.max(np.abs(eps_gpu - eps_ref) / eps_ref),
        "converted", conv, "oracle", want)
    assert np.all(np.abs(eps_gpu - eps_ref) <= 1e-3 * eps_ref)
    # the selection: the oracle's, up to near-ties at the boundary (and at the threshold)
    assert len(conv) == len(want) or tau is not None
    for i in conv:
        for j in set(range(L)) - set(conv):
            if tau is None or eps_ref[j] <= tau * (1 - 1e-3):
                assert eps_ref[i] <= eps_ref[j] * (1 + 1e-3), (i, j)
        if tau is not None:
            assert eps_ref[i] <= tau * (1 + 1e-3)
    # the chosen layers' updates (the solve ran on the compact batch under prefit)
    Wn = st.W.cpu().numpy()
    for l in range(L):
        if l in conv:
            assert relfro(Wn[l].astype(np.float64) - W0[l], dW_ref[l]) <= TOL_DW, l
        else:
            assert np.array_equal(Wn[l], W0[l]), l
    if selection == "prefit" and conv:
        assert st.info_compact.cpu().tolist() == [0] * len(conv)
    else:
        assert st.info.cpu().tolist() == [0] * L
