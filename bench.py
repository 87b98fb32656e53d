"""Benchmark of the gfx950 NVFP4 block-scaled GEMM.

One step = one pass of the attention-projection sweep of the pages (M in
{16, 32, 64, 128, 256, 512, 1024} x N = 768 x K = 6144, bf16 out): seven
``nvfp4_gemm`` calls on inputs already quantised and resident in HBM.  Each
step uses the next of several rotating buffer sets (together more than twice
the 256 MB Infinity Cache), so weights stream from HBM as in a real decode
pass over many layers.  ``value`` is the step's total TFLOPS (2*M*N*K summed
over the sweep / step time).

Printed as one JSON line, with per-shape results, the roofline of the
dominant call (timed with HIP events on the stream it runs on), the other
workloads of the pages (MoE expert sweep, large compute-bound shapes, the
grouped 256-expert MoE GEMM, the quantiser), and the CPU oracle timed on a
bounded sample of the same sweep.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOPS & % roofline (MFMA peak or HBM GB/s), M=16..8192"
PEAK_F16_TFLOPS = 2500.0      # dense f16 MFMA, MI355X
PEAK_FP4_TFLOPS = 10100.0     # dense fp4 MFMA, MI355X (context: not the issued instruction)
PEAK_HBM_GBPS = 8000.0
ROTATE_BYTES = 600 << 20      # > 2 x 256 MB Infinity Cache


def algo_bytes(M, N, K):
    """Bytes the method must move: packed codes + scales of A and B, bf16 D, alpha."""
    return (M + N) * K * 9 // 16 + 2 * M * N + 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads and the CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is a design note, "
                                   "not implemented", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import nvfp4_block_scaled_07_amd as nv
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def quantise(x_np, with_gs=True):
        xt = torch.from_numpy(x_np).to(dev)
        R, K = xt.shape
        gs = None
        if with_gs:
            gs = torch.empty(1, dtype=torch.float32, device=dev)
            nv.nvfp4_global_scale(xt, xt.numel(), gs)
        q = torch.empty((R, K // 2), dtype=torch.uint8, device=dev)
        sf = torch.empty((R, K // 16), dtype=torch.uint8, device=dev)
        nv.nvfp4_quantize(xt, R, K, gs, q, sf)
        return q, sf, gs

    def sweep_inputs(name, rotate=True):
        w = synth.WORKLOADS[name]
        a, b = synth.single_operands(name)
        qa, sfa, gsa = quantise(a)
        qb, sfb, gsb = quantise(b)
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
        nv.nvfp4_alpha_from_scales(gsa, gsb, alpha, 1)
        per_set = sum(t.numel() for t in (qa, sfa, qb, sfb))
        nsets = max(1, -(-ROTATE_BYTES // per_set)) if rotate else 1
        sets = [(qa, sfa, qb, sfb)] + [tuple(t.clone() for t in (qa, sfa, qb, sfb)) for _ in range(nsets - 1)]
        outs, wss = {}, {}
        for m in w["ms"]:
            outs[m] = torch.empty((m, w["n"]), dtype=torch.int16, device=dev)
            wss[m] = nv.gemm_workspace(m, w["n"], w["k"])
        return w, sets, alpha, outs, wss

    def call(w, s, alpha, outs, wss, m):
        qa, sfa, qb, sfb = s
        nv.nvfp4_gemm(qa[:m], sfa[:m], qb, sfb, alpha, outs[m], m, w["n"], w["k"], wss[m])

    # ---------------- headline: attention-projection sweep -----------------
    # Each step replays one captured HIP graph holding the seven GEMM calls on
    # one buffer set; graphs rotate over the sets, so the host enqueues one
    # replay per step and the GPU never waits on Python.
    name = "attn_proj_n768_k6144"
    w, sets, alpha, outs, wss = sweep_inputs(name)
    ms = list(w["ms"])
    N, K = w["n"], w["k"]
    graphs = [capture(torch, lambda s=s: [call(w, s, alpha, outs, wss, m) for m in ms]) for s in sets]

    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        graphs[(args.warmup + i) % len(graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = wall * 1e3 / args.steps
    flops_step = sum(2.0 * m * N * K for m in ms)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # per-call durations: a graph of back-to-back calls of one shape over the
    # rotating sets, timed with HIP events on the launch stream
    shapes = []
    for m in ms:
        reps = min(len(sets), 64)
        g = capture(torch, lambda: [call(w, sets[i], alpha, outs, wss, m) for i in range(reps)])
        t_us = replay_us(torch, stream, g, reps)
        fl = 2.0 * m * N * K
        by = algo_bytes(m, N, K)
        shapes.append(dict(M=m, N=N, K=K, plan=nv.nvfp4_gemm_plan(m, N, K), us=round(t_us, 3),
                           tflops=round(fl / t_us / 1e6, 2), gbps=round(by / t_us / 1e3, 1),
                           frac_f16_mfma=round(fl / t_us / 1e6 / PEAK_F16_TFLOPS, 4),
                           frac_fp4_peak=round(fl / t_us / 1e6 / PEAK_FP4_TFLOPS, 4),
                           frac_hbm=round(by / t_us / 1e3 / PEAK_HBM_GBPS, 4)))
        del g
    dom = max(shapes, key=lambda r: r["us"])
    fl = 2.0 * dom["M"] * N * K
    by = algo_bytes(dom["M"], N, K)
    mfma_bound = fl / by > PEAK_F16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if mfma_bound:
        roofline = dict(bound="mfma", achieved=dom["tflops"], peak=PEAK_F16_TFLOPS, unit="TFLOP/s",
                        frac=round(dom["tflops"] / PEAK_F16_TFLOPS, 4), traffic=None,
                        kernel_call=f"nvfp4_gemm M={dom['M']} N={N} K={K} ({dom['plan']})")
    else:
        roofline = dict(bound="hbm", achieved=dom["gbps"], peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(dom["gbps"] / PEAK_HBM_GBPS, 4), traffic=None,
                        kernel_call=f"nvfp4_gemm M={dom['M']} N={N} K={K} ({dom['plan']})")
    del graphs
    del sets, outs, wss
    torch.cuda.empty_cache()

    out = dict(metric=METRIC, value=round(value, 3), unit="TFLOPS", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms_per_step, 5), gpu_ms_per_step=round(gpu_ms / args.steps, 5),
               higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="f16", data="synthetic",
               config=dict(workload=f"{name}: nvfp4_gemm M in {ms} x N={N} x K={K}, bf16 out, "
                                    f"rotating HBM-resident buffer sets (cold cache)",
                           M=ms, N=N, K=K, block_size=16),
               roofline=roofline, shapes=shapes)

    if not args.no_extra:
        out["other_workloads"] = other_workloads(nv, torch, dev, stream, synth, quantise, sweep_inputs, call)
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


def capture(torch, fn):
    """Capture fn's launches (on torch's current stream) into a HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                  # eager run first (same work, no capture)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_us(torch, stream, g, calls, repeats=5):
    """Median over `repeats` replays of the per-call time (us) of a graph holding `calls` calls."""
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / calls)
    return float(np.median(ts))


def timed(torch, stream, fn, reps):
    g = capture(torch, lambda: [fn(i) for i in range(reps)])
    t = replay_us(torch, stream, g, reps)
    del g
    return t


def other_workloads(nv, torch, dev, stream, synth, quantise, sweep_inputs, call):
    res = {}
    # MoE expert-shape sweep (cold, rotating) and large compute-bound shapes (warm)
    for name, rotate, reps in (("moe_expert_n2048_k6144", True, 50), ("large_n6144_k6144", False, 10)):
        w, sets, alpha, outs, wss = sweep_inputs(name, rotate)
        rows = []
        for m in w["ms"]:
            us = timed(torch, stream, lambda i: call(w, sets[i % len(sets)], alpha, outs, wss, m), reps)
            fl = 2.0 * m * w["n"] * w["k"]
            by = algo_bytes(m, w["n"], w["k"])
            rows.append(dict(M=m, N=w["n"], K=w["k"], plan=nv.nvfp4_gemm_plan(m, w["n"], w["k"]), us=round(us, 2),
                             tflops=round(fl / us / 1e6, 2), gbps=round(by / us / 1e3, 1),
                             frac_f16_mfma=round(fl / us / 1e6 / PEAK_F16_TFLOPS, 4),
                             frac_fp4_peak=round(fl / us / 1e6 / PEAK_FP4_TFLOPS, 4)))
        res[name] = dict(cache="cold (rotating sets)" if rotate else "warm", shapes=rows)
        del sets, outs, wss
        torch.cuda.empty_cache()

    # grouped MoE: 512 tokens, top-8 of 256 experts, [rows_e, 6144] x [6144, 2048] per expert
    g = synth.GROUPED
    T, E, N, K = g["tokens"], g["experts"], g["n"], g["k"]
    tok, off = synth.routing(g["seed_router"], T, E, g["top_k"])
    rows = int(off[-1])
    qa_tok, sfa_tok, gsa = quantise(synth.token_activations(T, K))
    tok_t = torch.from_numpy(tok).to(dev)
    qa, sfa = qa_tok[tok_t].contiguous(), sfa_tok[tok_t].contiguous()
    b = torch.from_numpy(synth.random_codes(g["seed_expert_base"], E * N, K)).to(dev)
    bsf = torch.from_numpy(synth.random_scale_bytes(g["seed_expert_base"] + 1, E * N, K, 0x20, 0x38)).to(dev)
    off_t = torch.from_numpy(off).to(dev)
    alpha = torch.full((E,), 1.0, dtype=torch.float32, device=dev) / gsa
    d = torch.empty((rows, N), dtype=torch.int16, device=dev)
    need = nv.nvfp4_grouped_workspace_size(rows, N, K, E)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    us = timed(torch, stream, lambda i: nv.nvfp4_grouped_gemm(qa, sfa, b, bsf, off_t, alpha, d, rows, N, K, E, ws),
               10)
    active = int((np.diff(off) > 0).sum())
    by = active * N * K * 9 // 16 + rows * K * 9 // 16 + 2 * rows * N + 4 * (E + 1) + 4 * E
    fl = 2.0 * rows * N * K
    res["grouped_moe_512tok_256exp_top8"] = dict(rows=rows, active_experts=active, N=N, K=K, us=round(us, 2),
                                                 gbps=round(by / us / 1e3, 1),
                                                 frac_hbm=round(by / us / 1e3 / PEAK_HBM_GBPS, 4),
                                                 tflops=round(fl / us / 1e6, 2),
                                                 rows_per_expert_max=int(np.diff(off).max()))
    del b, bsf, qa, sfa, d
    torch.cuda.empty_cache()

    # quantiser (prologue): 16384 x 6144 fp32 -> NVFP4
    x = torch.from_numpy(synth.normal_f32(4001, (16384, 6144))).to(dev)
    q = torch.empty((16384, 3072), dtype=torch.uint8, device=dev)
    sf = torch.empty((16384, 384), dtype=torch.uint8, device=dev)
    gs = torch.ones(1, dtype=torch.float32, device=dev)
    us = timed(torch, stream, lambda i: nv.nvfp4_quantize(x, 16384, 6144, gs, q, sf), 10)
    by = 16384 * 6144 * (4 + 0.5 + 1 / 16)
    res["quantize_16384x6144"] = dict(us=round(us, 2), gbps=round(by / us / 1e3, 1),
                                      frac_hbm=round(by / us / 1e3 / PEAK_HBM_GBPS, 4))
    return res


def cpu_baseline(seconds):
    """The oracle (numpy: LUT dequant to fp64, BLAS dgemm, RNE to bf16) on the
    same sweep, repeated for about `seconds` of wall time."""
    import synth
    from oracle import nvfp4_ref as o
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    name = "attn_proj_n768_k6144"
    w = synth.WORKLOADS[name]
    a, b = synth.single_operands(name)
    gsa, gsb = o.global_encode_scale(a), o.global_encode_scale(b)
    qa, sfa = o.quantize(a, gsa)
    qb, sfb = o.quantize(b, gsb)
    alpha = o.alpha_from_scales(gsa, gsb)
    flops = 0.0
    passes = 0
    t0 = time.perf_counter()
    while True:
        for m in w["ms"]:
            o.gemm(qa[:m], sfa[:m], qb, sfb, alpha)
            flops += 2.0 * m * w["n"] * w["k"]
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    t = time.perf_counter() - t0
    return dict(value=round(flops / t / 1e12, 5), unit="TFLOPS", cores=cores, kind="oracle",
                sample=f"{passes} passes of the {name} sweep (M={list(w['ms'])}, N={w['n']}, K={w['k']}) "
                       f"in {t:.1f} s: LUT dequant to fp64, dgemm, RNE to bf16")


if __name__ == "__main__":
    main()
