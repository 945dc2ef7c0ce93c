"""Benchmark of the ISPA hot path on one MI355X.

One step = the whole warmup-and-absorb path of one attention layer (by
default the Wan-14B-shaped layer, the largest single layer; --config picks
another): for each of the 4 warmup chunks, ispa_decomp_attn (local branch,
history branch, fused LSE merge) then ispa_gram_accum on (A_loc, A_full);
then ispa_absorb_solve_ex (dW for the layer).  Inputs are seeded synthetic
data already resident in HBM when timing starts.

Prints ONE JSON line.  `value` is decomposable-attention TFLOP/s over the
whole step (attention matmul FLOPs of the 4 chunks / step time); the per-kernel
numbers, the absorb ms/layer, the roofline of the dominant kernel and the
oracle's CPU rate are reported beside it.

    python bench.py [--steps K] [--warmup W] [--config 3] [--also 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decomposable-attn TFLOP/s (% bf16 MFMA peak) + absorb ms/layer, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 (vector and MFMA)
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
# fp8-key attention: half its FLOPs (S = K Q^T) at the fp8 rate, half (P V) at the bf16 rate
PEAK_FP8K_TFLOPS = round(1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS), 1)
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=3,
                    help="1: Wan-1.3B layer, 2: long history, 3: Wan-14B layer (the largest single layer, default), "
                         "4: 30-layer 1.3B stack")
    ap.add_argument("--also", type=lambda v: [int(x) for x in v.split(",") if x], default=[1],
                    help="other single-layer configurations whose core figures are reported beside (comma list)")
    ap.add_argument("--gen-workers", type=int, default=min(16, os.cpu_count() or 1),
                    help="processes drawing the 30-layer stack's inputs (config 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm", type=float, default=1.0, metavar="SECONDS",
                    help="untimed steps for this long before the warmup steps (GPU clocks settle)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU seconds for the oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (calibrates HBM byte counters)")
    ap.add_argument("--traffic", type=str, default=None,
                    help="measured HBM traffic of the attention kernel (from rocprofv3 counters); default "
                         "profiles/attn_bf16_kernel_<workload>_hbm_traffic.json")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the hot path is one layer on one device, "
                                   "with no sharding or collectives; --gpus must be 1"}), flush=True)
        sys.exit(2)

    if args.config == 4:
        # the stack's inputs are drawn by worker processes before this process touches the GPU
        stack_inputs = generate_stack_inputs(args.gen_workers)
    import torch

    from kv_cache_absorption_ispa_amd import inputs, ispa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "launches": 3}), flush=True)
        return
    ispa.load_library()
    ispa.ispa_device_check(0)
    if args.config == 4:
        return bench_stack(args, stack_inputs)
    cfg = inputs.CONFIGS[args.config]
    main_run = time_layer_step(cfg, args.steps, args.warmup, args.prewarm)
    result = layer_result(args, cfg, main_run)
    # the comparison, streaming, split-KV, fp8 and no-refinement figures on the headline layer's chunk 0
    result.update(layer_extras(cfg, main_run))
    main_run.release()
    # the other single-layer shapes' core figures, timed the same way (fewer steps)
    also = {}
    for other in args.also:
        if other == args.config or other not in (1, 2, 3):
            continue
        ocfg = inputs.CONFIGS[other]
        run = time_layer_step(ocfg, max(3, args.steps // 2), 1, min(args.prewarm, 0.5))
        also[ocfg.name] = core_figures(ocfg, run)
        run.release()
    if also:
        result["also"] = also
    result["reference_bf16_gemm_tflops"] = reference_gemm_tflops()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


class LayerRun:
    """Device inputs and buffers of one layer shape, with the timed steps' measurements."""

    def release(self):
        import torch

        self.__dict__.clear()
        torch.cuda.empty_cache()


def time_layer_step(cfg, steps: int, warmup: int, prewarm_s: float) -> LayerRun:
    """One step = for each warmup chunk: ispa_decomp_attn (both branches and the fused merge) then
    ispa_gram_accum on its rows; then ispa_absorb_solve_ex (R = C W on a caller-owned side stream).
    Inputs resident in HBM; `steps` timed steps after `warmup` untimed ones, per-kernel durations from
    HIP events recorded on the launch stream inside the timed steps."""
    import torch

    from kv_cache_absorption_ispa_amd import inputs, ispa

    H, D, d = cfg.heads, cfg.head_dim, cfg.d
    r = LayerRun()

    def dev(t):
        return torch.from_numpy(t.raw.view(np.int16)).view(torch.bfloat16).cuda()

    log(f"[bench] generating inputs for {cfg.name}")
    r.chunks = []
    for c in range(cfg.n_chunks):
        x = inputs.chunk_inputs(cfg, 0, c)
        r.chunks.append(dict(q=dev(x.q), kl=dev(x.k_loc), vl=dev(x.v_loc), kh=dev(x.k_hist), vh=dev(x.v_hist)))
    r.W = torch.from_numpy(inputs.weight(cfg, 0)).cuda()
    nq = cfg.n_q
    r.o_loc = torch.empty(nq, H, D, dtype=torch.bfloat16, device="cuda")
    r.o_hist = torch.empty_like(r.o_loc)
    r.o_full = torch.empty_like(r.o_loc)
    r.lse = [torch.empty(H, nq, device="cuda") for _ in range(3)]
    r.G = torch.empty(d, d, device="cuda")
    r.C = torch.empty(d, d, device="cuda")
    r.dW = torch.empty(d, d, device="cuda")
    r.info = torch.empty(1, dtype=torch.int32, device="cuda")
    r.gws = ispa.workspace(ispa.ispa_gram_workspace_size(nq, d, torch.bfloat16))
    r.atws = ispa.workspace(ispa.ispa_decomp_attn_workspace_size(r.chunks[0]["q"], cfg.n_loc, cfg.n_hist))
    r.aws = ispa.workspace(ispa.ispa_absorb_workspace_size(d, d, 1))
    r.side = ispa.SideStream()  # caller-owned stream for R = C W beside the factorisation
    torch.cuda.synchronize()
    n_ev = 2 * cfg.n_chunks + 1

    def step(events=None):
        for c, ch in enumerate(r.chunks):
            if events is not None:
                events[2 * c][0].record()
            ispa.ispa_decomp_attn(ch["q"], ch["kl"], ch["vl"], ch["kh"], ch["vh"], o_loc=r.o_loc, lse_loc=r.lse[0],
                                  o_hist=r.o_hist, lse_hist=r.lse[1], o_full=r.o_full, lse_full=r.lse[2],
                                  workspace=r.atws)
            if events is not None:
                events[2 * c][1].record()
                events[2 * c + 1][0].record()
            ispa.ispa_gram_accum(r.o_loc, r.o_full, r.G, r.C, accumulate=c > 0, workspace=r.gws)
            if events is not None:
                events[2 * c + 1][1].record()
        if events is not None:
            events[-1][0].record()
        ispa.ispa_absorb_solve_ex(r.G, r.C, r.W, cfg.lam, r.dW, r.info, workspace=r.aws, side=r.side)
        if events is not None:
            events[-1][1].record()

    r.prewarm_steps = prewarm(step, prewarm_s)
    log(f"[bench] {cfg.name}: prewarm {r.prewarm_steps} steps, warmup {warmup} steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if r.info.item() != 0:
        raise RuntimeError(f"absorb failed, info = {r.info.item()}")
    log(f"[bench] {cfg.name}: timing {steps} steps")
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    r.steps = steps
    r.ms_per_step = wall * 1e3 / steps
    r.attn_ms, r.gram_ms, r.solve_ms = [], [], []
    for ev in evs:
        for c in range(cfg.n_chunks):
            r.attn_ms.append(ev[2 * c][0].elapsed_time(ev[2 * c][1]))
            r.gram_ms.append(ev[2 * c + 1][0].elapsed_time(ev[2 * c + 1][1]))
        r.solve_ms.append(ev[-1][0].elapsed_time(ev[-1][1]))
    return r


def core_figures(cfg, r: LayerRun) -> dict:
    """Whole-step and per-kernel figures of a timed layer run."""
    d, nq = cfg.d, cfg.n_q
    attn_flops = cfg.attn_flops()
    attn_avg = float(np.mean(r.attn_ms))
    achieved = attn_flops / (attn_avg * 1e-3) / 1e12
    gram_flops = 3.0 * nq * d * d
    solve_flops = 13.0 / 3.0 * float(d) ** 3
    solve_bytes = 16.0 * d * d
    solve_ms = float(np.mean(r.solve_ms))
    gram_ms = float(np.mean(r.gram_ms))
    return {
        "workload": workload_name(cfg),
        "ms_per_step": round(r.ms_per_step, 4),
        "value_tflops": round(attn_flops * cfg.n_chunks / (r.ms_per_step * 1e-3) / 1e12, 2),
        "attn_tflops_kernel": round(achieved, 2),
        "attn_pct_bf16_peak": round(100 * achieved / PEAK_BF16_TFLOPS, 2),
        "attn_ms_per_chunk": round(attn_avg, 4),
        "gram_ms_per_chunk": round(gram_ms, 4),
        # algorithmic Gram work: 2 d^2 per row for C plus d^2 per row for the symmetric G
        "gram_tflops": round(gram_flops / (gram_ms * 1e-3) / 1e12, 2),
        "gram_pct_bf16_peak": round(100 * gram_flops / (gram_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "absorb_ms_per_layer": round(solve_ms, 4),
        # algorithmic solve work 13/3 d^3 (factor d^3/3, R = C W 2 d^3, two triangular solves 2 d^3) and its
        # compulsory bytes (read G, C, W, write dW: 16 d^2), against the measured absorb time
        "absorb_tflops": round(solve_flops / (solve_ms * 1e-3) / 1e12, 3),
        "absorb_pct_fp32_peak": round(100 * solve_flops / (solve_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 2),
        "absorb_gbps": round(solve_bytes / (solve_ms * 1e-3) / 1e9, 1),
    }


def workload_name(cfg) -> str:
    return (f"{cfg.name}: {cfg.heads} heads x {cfg.head_dim}, {cfg.n_q} queries/chunk, {cfg.n_sink} sink + "
            f"{cfg.n_chunk} chunk local keys, {cfg.n_hist} history keys, {cfg.n_chunks} warmup chunks, "
            f"absorb d={cfg.d}")


def layer_result(args, cfg, r: LayerRun) -> dict:
    """The JSON line's fixed keys, the roofline of the dominant kernel and the core figures."""
    core = core_figures(cfg, r)
    attn_flops = cfg.attn_flops()
    achieved = core["attn_tflops_kernel"]
    traffic = None
    tpath = args.traffic or os.path.join(ROOT, "profiles", f"attn_bf16_kernel_{cfg.name}_hbm_traffic.json")
    if os.path.exists(tpath):
        try:
            with open(tpath) as f:
                t = json.load(f)
            if t.get("kernel_source_sha") == kernel_source_sha():
                traffic = t.get("bytes_per_launch")
        except Exception:
            traffic = None
    out = {
        "metric": METRIC,
        "value": core["value_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": core["ms_per_step"],
        "prewarm_steps": r.prewarm_steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, 8 sink keys at 4x norm; random-init W)",
        "config": {
            "workload": core["workload"],
            "global_batch": cfg.n_chunks * cfg.n_q,
            "seq_len": cfg.n_loc + cfg.n_hist,
            "parallelism": "single GPU",
        },
    }
    out.update({k: v for k, v in core.items() if k not in ("workload", "ms_per_step", "value_tflops")})
    out["roofline"] = {
        "bound": "mfma",
        "kernel": "attn_bf16_kernel<128, 8, 1, 128, false, false> (ispa_decomp_attn)",
        "achieved": achieved,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "algorithmic_flops_per_launch": attn_flops,
    }
    return out


def layer_extras(cfg, r: LayerRun) -> dict:
    """Comparison and variant figures on chunk 0 of the timed layer (each timed back to back)."""
    import torch

    from kv_cache_absorption_ispa_amd import ispa

    H, D, d, nq = cfg.heads, cfg.head_dim, cfg.d, cfg.n_q
    attn_flops = cfg.attn_flops()
    ch = r.chunks[0]
    o_loc, o_hist, o_full, lse = r.o_loc, r.o_hist, r.o_full, r.lse
    tf = lambda ms, fl=attn_flops: round(fl / (ms * 1e-3) / 1e12, 2)

    # ---- the ratio to one softmax pass over the concatenated keys: the decomposable call on its two
    # buffers, the single pass, and the decomposable call on two views of the single pass's buffer, timed
    # with the same protocol on the same chunk (rounds interleaved, so clock drift hits all three alike)
    kcat = torch.cat([ch["kl"], ch["kh"]])
    vcat = torch.cat([ch["vl"], ch["vh"]])
    o_single = torch.empty_like(o_loc)
    lse_single = torch.empty(H, nq, device="cuda")
    nl = cfg.n_loc
    two = lambda: ispa.ispa_decomp_attn(ch["q"], ch["kl"], ch["vl"], ch["kh"], ch["vh"], o_loc=o_loc, lse_loc=lse[0],
                                        o_hist=o_hist, lse_hist=lse[1], o_full=o_full, lse_full=lse[2],
                                        workspace=r.atws)
    single = lambda: ispa.ispa_full_attn(ch["q"], kcat, vcat, o=o_single, lse=lse_single)
    views = lambda: ispa.ispa_decomp_attn(ch["q"], kcat[:nl], vcat[:nl], kcat[nl:], vcat[nl:], o_loc=o_loc,
                                          lse_loc=lse[0], o_hist=o_hist, lse_hist=lse[1], o_full=o_full,
                                          lse_full=lse[2], workspace=r.atws)
    two_ms, single_ms, views_ms = interleaved_ms([two, single, views])
    del kcat, vcat

    # ---- the same chunk with its keys as a streaming cache holds them: sink and chunk in their own
    # buffers, the history as the two runs of a wrapped ring (two chunks, then one), attended in place
    ns, nc = cfg.n_sink, cfg.n_chunk
    loc_segs = [(ch["kl"][:ns].clone(), ch["vl"][:ns].clone()), (ch["kl"][ns:].clone(), ch["vl"][ns:].clone())]
    cut = (cfg.n_hist // nc - 1) * nc if cfg.n_hist % nc == 0 and cfg.n_hist > nc else cfg.n_hist // 2
    hist_segs = [(ch["kh"][:cut].clone(), ch["vh"][:cut].clone()), (ch["kh"][cut:].clone(), ch["vh"][cut:].clone())]
    seg_ms = back_to_back_ms(lambda: ispa.ispa_decomp_attn_segments(
        ch["q"], loc_segs, hist_segs, o_loc=o_loc, lse_loc=lse[0], o_hist=o_hist, lse_hist=lse[1], o_full=o_full,
        lse_full=lse[2], workspace=r.atws))
    del loc_segs, hist_segs

    # ---- split-KV form (ispa_decomp_attn_splitkv, one workgroup per CU): at the full chunk every XCD
    # already has more units than spare workgroups (P = 1, the unsplit launch); a short query chunk of
    # 512 queries is where the key split pays
    skws = ispa.workspace(ispa.ispa_decomp_attn_splitkv_workspace_size(ch["q"], cfg.n_loc, cfg.n_hist, 0))
    sk_ms = back_to_back_ms(lambda: ispa.ispa_decomp_attn_splitkv(
        ch["q"], [(ch["kl"], ch["vl"])], [(ch["kh"], ch["vh"])], o_loc=o_loc, lse_loc=lse[0], o_hist=o_hist,
        lse_hist=lse[1], o_full=o_full, lse_full=lse[2], workspace=skws))
    nq_s = 512
    q_s = ch["q"][:nq_s].contiguous()
    o_s = [torch.empty(nq_s, H, D, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    l_s = [torch.empty(H, nq_s, device="cuda") for _ in range(3)]
    short_unsplit = back_to_back_ms(lambda: ispa.ispa_decomp_attn(
        q_s, ch["kl"], ch["vl"], ch["kh"], ch["vh"], o_loc=o_s[0], lse_loc=l_s[0], o_hist=o_s[1], lse_hist=l_s[1],
        o_full=o_s[2], lse_full=l_s[2], workspace=skws))
    short_split = back_to_back_ms(lambda: ispa.ispa_decomp_attn_splitkv(
        q_s, [(ch["kl"], ch["vl"])], [(ch["kh"], ch["vh"])], o_loc=o_s[0], lse_loc=l_s[0], o_hist=o_s[1],
        lse_hist=l_s[1], o_full=o_s[2], lse_full=l_s[2], workspace=skws))
    short_flops = attn_flops * nq_s / nq
    del skws, q_s, o_s, l_s

    # ---- the standalone N-way merge (ispa_lse_merge) of the chunk's two branch results into O_full and
    # LSE_full: reads both (O, LSE) pairs once and writes one, so HBM-bound
    two()
    merge_ms = back_to_back_ms(lambda: ispa.ispa_lse_merge([o_loc, o_hist], [lse[0], lse[1]], o_full, lse[2]))
    merge_bytes = 3 * (o_loc.numel() * o_loc.element_size() + lse[0].numel() * 4)

    # ---- the absorb without its refinement step (ispa_absorb_solve_ex, ISPA_ABSORB_NO_REFINE)
    dW2 = torch.empty_like(r.dW)
    norefine_ms = back_to_back_ms(lambda: ispa.ispa_absorb_solve_ex(r.G, r.C, r.W, cfg.lam, dW2, r.info, refine=False,
                                                                    workspace=r.aws, side=r.side), n=3)
    del dW2

    # ---- fp8 keys (ispa_decomp_attn_fp8k): Q and K as E4M3 codes with per-head scales (quantised on the
    # GPU, timed apart), S = K Q^T on the fp8 matrix cores; and the W8A8 projection of the chunk's rows
    q8 = torch.empty(nq, H, D, dtype=torch.uint8, device="cuda")
    kl8 = torch.empty(cfg.n_loc, H, D, dtype=torch.uint8, device="cuda")
    kh8 = torch.empty(cfg.n_hist, H, D, dtype=torch.uint8, device="cuda")
    qsc, klsc, khsc = (torch.empty(H, device="cuda") for _ in range(3))
    qws = ispa.workspace(ispa.ispa_quantize_fp8_heads_workspace_size(max(nq, cfg.n_hist, cfg.n_loc), H))

    def quant_qk():
        ispa.ispa_quantize_fp8_heads(ch["q"], q8, qsc, workspace=qws)
        ispa.ispa_quantize_fp8_heads(ch["kl"], kl8, klsc, workspace=qws)
        ispa.ispa_quantize_fp8_heads(ch["kh"], kh8, khsc, workspace=qws)

    quant_ms = back_to_back_ms(quant_qk)
    f8_ms = back_to_back_ms(lambda: ispa.ispa_decomp_attn_fp8k(
        q8, qsc, [(kl8, klsc, ch["vl"])], [(kh8, khsc, ch["vh"])], o_loc=o_loc, lse_loc=lse[0], o_hist=o_hist,
        lse_hist=lse[1], o_full=o_full, lse_full=lse[2], workspace=r.atws))
    a8 = torch.empty(nq, d, dtype=torch.uint8, device="cuda")
    asc = torch.empty(nq, device="cuda")
    w8t = torch.empty(d, d, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(d, device="cuda")
    a_rows = o_loc.reshape(nq, d)
    ispa.ispa_quantize_fp8_cols(r.W, w8t, wsc)
    y8 = torch.empty(nq, d, dtype=torch.bfloat16, device="cuda")
    rowq_ms = back_to_back_ms(lambda: ispa.ispa_quantize_fp8_rows(a_rows, a8, asc))
    w8a8_ms = back_to_back_ms(lambda: ispa.ispa_w8a8_gemm(a8, asc, w8t, wsc, y8))
    del q8, kl8, kh8, qws, a8, w8t, y8

    med = lambda v: float(np.median(v))
    return {
        "ratio": {
            "protocol": "back to back, 10 launches per round, 5 rounds interleaved, median, chunk 0",
            "decomp_two_buffers_ms": round(med(two_ms), 4),
            "single_pass_ms": round(med(single_ms), 4),
            "single_pass_tflops": tf(med(single_ms)),
            "single_pass_pct_bf16_peak": round(100 * attn_flops / (med(single_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "decomp_on_single_pass_buffer_ms": round(med(views_ms), 4),
            "decomp_vs_single_pass": round(med(two_ms) / med(single_ms), 4),
        },
        "ratio_decomp_vs_single_pass": round(med(two_ms) / med(single_ms), 4),
        "splitkv": {
            "workers": "one per compute unit",
            "ms": round(med(sk_ms), 4),
            "ratio_vs_two_buffer": round(med(sk_ms) / med(two_ms), 4),
            "short_chunk_queries": nq_s,
            "short_chunk_unsplit_ms": round(med(short_unsplit), 4),
            "short_chunk_split_ms": round(med(short_split), 4),
            "short_chunk_speedup": round(med(short_unsplit) / med(short_split), 3),
            "short_chunk_split_tflops": tf(med(short_split), short_flops),
        },
        "fp8": {
            "attn_ms": round(med(f8_ms), 4),
            "attn_tflops": tf(med(f8_ms)),
            "attn_speedup_vs_bf16": round(med(two_ms) / med(f8_ms), 3),
            "attn_peak_tflops": PEAK_FP8K_TFLOPS,
            "quantize_q_k_ms": round(med(quant_ms), 4),
            "w8a8_rows": nq, "w8a8_d": d,
            "quantize_rows_ms": round(med(rowq_ms), 4),
            "w8a8_gemm_ms": round(med(w8a8_ms), 4),
            "w8a8_tflops": tf(med(w8a8_ms), 2.0 * nq * d * d),
            "w8a8_frac_of_fp8_peak": round(2.0 * nq * d * d / (med(w8a8_ms) * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        },
        "segments": {
            "layout": f"local [{ns} sink | {nc} chunk], history [{cut} | {cfg.n_hist - cut}] (wrapped ring)",
            "ms": round(med(seg_ms), 4),
            "two_buffer_ms": round(med(two_ms), 4),
            "ratio_vs_two_buffer": round(med(seg_ms) / med(two_ms), 4),
            "tflops": tf(med(seg_ms)),
        },
        "absorb_ms_per_layer_no_refine": round(med(norefine_ms), 4),
        "lse_merge": {
            "parts": 2,
            "ms": round(med(merge_ms), 4),
            "algorithmic_bytes": merge_bytes,
            "gbps": round(merge_bytes / (med(merge_ms) * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(merge_bytes / (med(merge_ms) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        },
    }


# --------------------------------------------------------------------------- #
# 30-layer stack (config 4): warmup of every layer, transition, post-absorb chunk
# --------------------------------------------------------------------------- #
def _draw_chunk(job):
    from kv_cache_absorption_ispa_amd import inputs

    layer, chunk = job
    x = inputs.chunk_inputs(inputs.WAN13B_STACK30, layer, chunk)
    return layer, chunk, [t.raw for t in (x.q, x.k_loc, x.v_loc, x.k_hist, x.v_hist)]


def generate_stack_inputs(workers: int):
    """Host draws of every (layer, chunk) of the stack: 4 warmup chunks and the post-absorb chunk."""
    import multiprocessing as mp

    from kv_cache_absorption_ispa_amd import inputs

    cfg = inputs.WAN13B_STACK30
    jobs = [(l, c) for c in range(cfg.n_chunks + 1) for l in range(cfg.n_layers)]
    log(f"[bench] drawing {len(jobs)} chunk inputs of {cfg.name} with {workers} processes")
    t0 = time.perf_counter()
    out = {}
    with mp.get_context("spawn").Pool(workers) as pool:
        for i, (l, c, raws) in enumerate(pool.imap(_draw_chunk, jobs, chunksize=1)):
            out[(l, c)] = raws
            if (i + 1) % 30 == 0:
                log(f"[bench]   {i + 1}/{len(jobs)} drawn ({time.perf_counter() - t0:.0f} s)")
    return out


def bench_stack(args, host_inputs):
    """Config 4: 30 Wan-1.3B-shaped layers x 4 warmup chunks (decomposable attention + Gram), the
    transition (batched absorb of all 30, eps, ranking, W += dW on the 15 lowest) and one post-absorb
    chunk where those 15 attend locally.  One step = all of it; inputs resident in HBM."""
    import torch

    from kv_cache_absorption_ispa_amd import inputs, ispa
    from kv_cache_absorption_ispa_amd.stack import LayerStack

    cfg = inputs.WAN13B_STACK30
    L, H, D, d, nq = cfg.n_layers, cfg.heads, cfg.head_dim, cfg.d, cfg.n_q

    def dev(raw):
        return torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).cuda()

    log("[bench] uploading stack inputs")
    X = {}
    for key in sorted(host_inputs):
        X[key] = [dev(r) for r in host_inputs.pop(key)]
    W0 = torch.from_numpy(np.stack([inputs.weight(cfg, l) for l in range(L)])).cuda()
    W = W0.clone()
    st = LayerStack(W, H, D, nq, cfg.lam, cfg.n_absorb)
    o_loc = torch.empty(nq, H, D, dtype=torch.bfloat16, device="cuda")
    o_full = torch.empty_like(o_loc)
    torch.cuda.synchronize()

    def run(ev=None):
        """One pass of the stack; ev: dict of event lists for per-phase timing."""
        W.copy_(W0)  # fresh weights (restored before the phase markers)
        st.reset()
        def mark(k):
            if ev is not None:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                ev[k].append(e)

        mark("t0")
        for c in range(cfg.n_chunks):
            for l in range(L):
                q, kl, vl, kh, vh = X[(l, c)]
                st.warmup_chunk(l, q, kl, vl, kh, vh, o_loc, o_full)
        mark("t1")
        st.solve_and_rank()
        mark("t2")
        conv = st.convert()
        mark("t3")
        for l in range(L):
            q, kl, vl, kh, vh = X[(l, cfg.n_chunks)]
            st.post_chunk(l, q, kl, vl, kh, vh, o_full)
        mark("t4")
        return conv

    pw = prewarm(run, args.prewarm)
    log(f"[bench] stack prewarm {pw} passes, warmup {args.warmup} passes")
    for _ in range(args.warmup):
        conv = run()
    torch.cuda.synchronize()
    if st.info.cpu().tolist() != [0] * L:
        raise RuntimeError(f"absorb failed: info = {st.info.cpu().tolist()}")

    log(f"[bench] timing {args.steps} stack passes")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        conv = run()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-phase times (separate pass, same work)
    ev = {k: [] for k in ("t0", "t1", "t2", "t3", "t4")}
    for _ in range(args.steps):
        run(ev)
        torch.cuda.synchronize()
    ph = lambda a, b: float(np.median([x.elapsed_time(y) for x, y in zip(ev[a], ev[b])]))
    warm_ms, solve_ms, conv_ms, post_ms = ph("t0", "t1"), ph("t1", "t2"), ph("t2", "t3"), ph("t3", "t4")

    # the same post-absorb chunk with no layer converted (every layer keeps its history)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ws = ispa.workspace(ispa.ispa_decomp_attn_workspace_size(X[(0, 0)][0], cfg.n_loc, cfg.n_hist))
    full_post = []
    for _ in range(max(args.steps, 2)):
        e0.record()
        for l in range(L):
            q, kl, vl, kh, vh = X[(l, cfg.n_chunks)]
            ispa.ispa_decomp_attn(q, kl, vl, kh, vh, o_full=o_full, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        full_post.append(e0.elapsed_time(e1))
    full_post_ms = float(np.median(full_post))

    # the transition under the other selection / lambda policies, on the same warmup statistics
    policies = {}
    for name, kw in (("prefit", dict(selection="prefit")), ("heldout", dict(selection="heldout")),
                     ("trace_lambda", dict(lam_policy="trace")), ("threshold", dict(threshold=0.5))):
        times, n_c = [], 0
        for _ in range(max(args.steps, 2)):
            st2 = LayerStack(W0.clone(), H, D, nq, cfg.lam if "lam_policy" not in kw else 1e-4, cfg.n_absorb, **kw)
            st2.G.copy_(st.G)
            st2.C.copy_(st.C)
            st2.E.copy_(st.E)
            st2.chunks_seen = [cfg.n_chunks] * L
            if kw.get("selection") == "heldout":  # timing stand-in: the fitted rows as held-out rows
                st2.G_h.copy_(st.G)
                st2.C_h.copy_(st.C)
                st2.E_h.copy_(st.E)
                st2.heldout_seen = [1] * L
            torch.cuda.synchronize()
            t_a = time.perf_counter()
            n_c = len(st2.transition())
            torch.cuda.synchronize()
            times.append((time.perf_counter() - t_a) * 1e3)
            del st2
        policies[name] = {"transition_ms": round(float(np.median(times)), 3), "converted": n_c}

    n_conv = len(conv)
    f_full, f_loc = cfg.attn_flops(), cfg.attn_flops(n_hist=0)
    warm_flops = L * cfg.n_chunks * f_full
    post_flops = (L - n_conv) * f_full + n_conv * f_loc
    value = (warm_flops + post_flops) / (ms_per_step * 1e-3) / 1e12
    warm_tf = warm_flops / (warm_ms * 1e-3) / 1e12
    kv_total = L * 2 * (cfg.n_loc + cfg.n_hist) * d * 2
    evicted = st.evicted_kv_bytes(cfg.n_hist)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V per layer and chunk, 8 sink keys at 4x norm; random-init W)",
        "config": {
            "workload": f"{cfg.name}: {L} layers of {H} heads x {D}, {nq} queries/chunk, {cfg.n_sink} sink + "
                        f"{cfg.n_chunk} chunk local keys, {cfg.n_hist} history keys, {cfg.n_chunks} warmup chunks, "
                        f"batched absorb of all {L} (d={d}), {cfg.n_absorb} converted, 1 post-absorb chunk",
            "global_batch": L * (cfg.n_chunks + 1) * nq,
            "seq_len": cfg.n_loc + cfg.n_hist,
            "parallelism": "single GPU",
        },
        "warmup_ms": round(warm_ms, 3),
        "warmup_attn_gram_tflops": round(warm_tf, 2),
        "transition_ms": round(solve_ms + conv_ms, 3),
        "transition_policies": policies,
        "absorb_ms_per_layer": round(solve_ms / L, 4),
        "post_chunk_ms": round(post_ms, 3),
        "post_chunk_ms_no_eviction": round(full_post_ms, 3),
        "post_chunk_speedup": round(full_post_ms / post_ms, 3),
        "converted_layers": sorted(conv),
        "kv_bytes_total": kv_total,
        "kv_bytes_evicted": evicted,
        "kv_evicted_frac_of_history": round(evicted / (L * 2 * cfg.n_hist * d * 2), 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inputs.WAN13B_LAYER, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def reference_gemm_tflops(n: int = 8192, reps: int = 20) -> float:
    """A vendor-library bf16 GEMM (torch.matmul, n x n x n) timed in the same run: what a tuned dense MFMA
    kernel reaches at the clock the GPU holds under load, for reading the attention kernel's efficiency
    beside the spec peak.  Measurement only; not part of the hot path."""
    import torch

    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    return round(2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)


def interleaved_ms(fns, n: int = 10, rounds: int = 5, warm: int = 3):
    """Per-launch ms of each of `fns`, launched n times back to back per round, the functions taking turns
    round by round."""
    import torch
    for fn in fns:
        for _ in range(warm):
            fn()
    out = [[] for _ in fns]
    for _ in range(rounds):
        for i, fn in enumerate(fns):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            out[i].append(e0.elapsed_time(e1) / n)
    return out


def back_to_back_ms(fn, n: int = 10, rounds: int = 3, warm: int = 3):
    """Per-launch ms of `fn`, launched n times back to back, for each of `rounds` rounds."""
    import torch
    for _ in range(warm):
        fn()
    out = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / n)
    return out


def prewarm(step, seconds: float) -> int:
    """Untimed steps for `seconds` so the GPU clocks settle before the warmup steps."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def kernel_source_sha() -> str:
    import hashlib

    p = os.path.join(ROOT, "kv_cache_absorption_ispa_amd", "csrc", "attn_kernels.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(cfg, target_s: float):
    """The oracle (float64 numpy, as it stands) on a bounded sample of the same workload: decomposable
    attention (both branches and the merge) of whole warmup chunks, the last one possibly cut to a query
    prefix, over all local and history keys, stopping after about target_s seconds."""
    import oracle
    from kv_cache_absorption_ispa_amd import inputs

    threads, blas = os.cpu_count() or 1, "unknown"
    try:
        from threadpoolctl import threadpool_info

        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if pools:
            threads = max(int(i.get("num_threads", 1)) for i in pools)
            i = pools[0]
            blas = f"{i.get('internal_api', '?')} {i.get('version', '?')} ({i.get('architecture', '?')} kernels)"
    except Exception:
        pass
    def decomposed(x, qs):
        kl, vl, kh, vh = x.k_loc.f64, x.v_loc.f64, x.k_hist.f64, x.v_hist.f64
        o_l, l_l = oracle.attention(qs, kl, vl, cfg.scale)
        o_h, l_h = oracle.attention(qs, kh, vh, cfg.scale)
        return oracle.merge(o_l, l_l, o_h, l_h)

    # grow the query sample of chunk 0 until one run takes a measurable time
    x0 = inputs.chunk_inputs(cfg, 0, 0)
    q0 = x0.q.f64
    n = 32
    while True:
        t0 = time.perf_counter()
        decomposed(x0, q0[:n])
        t = time.perf_counter() - t0
        if t > 0.5 or n >= cfg.n_q:
            break
        n = min(cfg.n_q, n * 4)
    # then whole warmup chunks (or a query prefix of one) up to about target_s of CPU time
    per_q = t / n
    done_q, elapsed, chunks = 0, 0.0, 0
    for c in range(cfg.n_chunks):
        want = int(min(cfg.n_q, max(32, (target_s - elapsed) / per_q)))
        x = x0 if c == 0 else inputs.chunk_inputs(cfg, 0, c)
        t0 = time.perf_counter()
        decomposed(x, x.q.f64[:want])
        elapsed += time.perf_counter() - t0
        done_q += want
        chunks += 1
        if want < cfg.n_q or elapsed >= target_s:
            break
    flops = 4.0 * done_q * (cfg.n_loc + cfg.n_hist) * cfg.head_dim * cfg.heads
    return {
        "value": round(flops / elapsed / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "blas": blas,
        "kind": "oracle",
        "sample": f"{done_q} queries ({chunks} of {cfg.n_chunks} warmup chunks, {cfg.n_q} queries each), all "
                  f"{cfg.heads} heads, {cfg.n_loc}+{cfg.n_hist} keys, decomposed attention and merge; {elapsed:.1f} s",
    }


if __name__ == "__main__":
    main()
