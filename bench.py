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
GRAPH_STEPS = 8               # steps captured per HIP graph


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
    ap.add_argument("--profile-call", type=int, default=0, metavar="M",
                    help="for hardware-counter runs: one 256 MiB device copy (counter calibration), then 8 "
                         "cold calls of the headline GEMM at this M; prints nothing else")
    ap.add_argument("--graph", action="store_true",
                    help="with --profile-call: time the call as the headline does (graphs of 64 calls over "
                         "the rotating sets, replayed 8 times) instead of 8 eager calls")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs of a --profile-call run (FETCH_SIZE, "
                         "WRITE_SIZE) into the HBM traffic record read by the roofline (no GPU needed)")
    args = ap.parse_args()
    if args.traffic:
        if not args.profile_call:
            raise SystemExit("--traffic needs the --profile-call M the counters were taken with")
        write_traffic_record(*args.traffic, m=args.profile_call)
        return
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

    if args.profile_call:
        profile_call(torch, nv, sweep_inputs, call, args.profile_call, args.graph)
        return

    # ---------------- headline: attention-projection sweep -----------------
    # Steps are captured into HIP graphs, GRAPH_STEPS consecutive steps (each
    # on the next buffer set) per graph, as a serving loop would capture a
    # whole pass; single-step graphs cover a remainder.  The host enqueues one
    # replay per GRAPH_STEPS steps and the GPU never waits on Python.
    name = "attn_proj_n768_k6144"
    w, sets, alpha, outs, wss = sweep_inputs(name)
    ms = list(w["ms"])
    N, K = w["n"], w["k"]
    G = min(GRAPH_STEPS, len(sets))
    multi = [capture(torch, lambda j=j: [call(w, sets[(j * G + t) % len(sets)], alpha, outs, wss, m)
                                         for t in range(G) for m in ms])
             for j in range((len(sets) + G - 1) // G)]
    single = [capture(torch, lambda t=t: [call(w, sets[t], alpha, outs, wss, m) for m in ms]) for t in range(G)]

    def run_steps(n, first):
        i = 0
        while n - i >= G:
            multi[((first + i) // G) % len(multi)].replay()
            i += G
        while i < n:
            single[(first + i) % G].replay()
            i += 1

    run_steps(args.warmup, 0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    run_steps(args.steps, args.warmup)
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
    call_name = f"nvfp4_gemm M={dom['M']} N={N} K={K}"
    traffic = read_traffic_record(call_name, dom["plan"])
    if mfma_bound:
        roofline = dict(bound="mfma", achieved=dom["tflops"], peak=PEAK_F16_TFLOPS, unit="TFLOP/s",
                        frac=round(dom["tflops"] / PEAK_F16_TFLOPS, 4), traffic=traffic,
                        kernel_call=f"{call_name} ({dom['plan']})", algorithmic_bytes=by,
                        algorithmic_flops=fl)
    else:
        roofline = dict(bound="hbm", achieved=dom["gbps"], peak=PEAK_HBM_GBPS, unit="GB/s",
                        frac=round(dom["gbps"] / PEAK_HBM_GBPS, 4), traffic=traffic,
                        kernel_call=f"{call_name} ({dom['plan']})", algorithmic_bytes=by,
                        algorithmic_flops=fl)
    del multi, single
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


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_headline_dominant_call.json")
COPY_BYTES = 256 << 20


def kernel_sources_digest():
    """sha256 over the library's kernel sources: a traffic record only holds
    for the kernels it was measured on."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "nvfp4_block_scaled_07_amd", "csrc")
    for f in sorted(os.listdir(src)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(src, f), "rb").read())
    return h.hexdigest()[:16]


def profile_call(torch, nv, sweep_inputs, call, m, graph=False):
    """Workload of the profiler runs: a plain 256 MiB copy (its FETCH_SIZE and
    WRITE_SIZE calibrate the counters), then 8 cold calls of one headline GEMM,
    or (graph=True) the per-call timing of the headline: a graph of 64 calls
    over the rotating sets, replayed 8 times, with its HIP-event time printed."""
    x = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    del x, y
    name = "attn_proj_n768_k6144"
    w, sets, alpha, outs, wss = sweep_inputs(name)
    if m not in outs:
        raise SystemExit(f"M={m} is not a shape of {name}: {list(outs)}")
    if graph:
        reps = min(len(sets), 64)
        g = capture(torch, lambda: [call(w, sets[i], alpha, outs, wss, m) for i in range(reps)])
        us = replay_us(torch, torch.cuda.current_stream(), g, reps, repeats=8)
        print(json.dumps({"call": f"nvfp4_gemm M={m} N={w['n']} K={w['k']} "
                                  f"({nv.nvfp4_gemm_plan(m, w['n'], w['k'])})", "us_per_call": round(us, 3)}))
        return
    for i in range(8):
        call(w, sets[i % len(sets)], alpha, outs, wss, m)
    torch.cuda.synchronize()


def _counter_rows(path, counter):
    import csv
    rows = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            rows.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return rows


def write_traffic_record(fetch_csv, write_csv, m):
    """FETCH_SIZE / WRITE_SIZE are in KiB per dispatch.  Each is scaled by
    what the same counter reads for the plain copy of COPY_BYTES (which must
    fetch and write exactly COPY_BYTES), then averaged over the GEMM dispatches."""
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, counter)
        copies = [v for n, g, v in rows if "copy" in n.lower() or "elementwise" in n.lower()]
        gemm = [(n, g, v) for n, g, v in rows if "k_gemm" in n]
        if not copies or not gemm:
            raise SystemExit(f"{path}: no copy or no GEMM dispatch with {counter}")
        calib = max(copies) * 1024.0 / COPY_BYTES
        out[counter] = dict(copy_kib=max(copies), factor=round(1.0 / calib, 6),
                            gemm_kib_mean=sum(v for _, _, v in gemm) / len(gemm),
                            bytes_per_launch=sum(v for _, _, v in gemm) / len(gemm) * 1024.0 / calib,
                            dispatches=len(gemm), kernel=gemm[0][0][:160], grid=gemm[0][1])
    rec = dict(sources_sha256_16=kernel_sources_digest(), copy_bytes=COPY_BYTES, counters=out,
               traffic_bytes_per_launch=round(out["FETCH_SIZE"]["bytes_per_launch"] +
                                              out["WRITE_SIZE"]["bytes_per_launch"]))
    import nvfp4_block_scaled_07_amd as nv
    import synth
    w = synth.WORKLOADS["attn_proj_n768_k6144"]
    rec["call"] = f"nvfp4_gemm M={m} N={w['n']} K={w['k']} ({nv.nvfp4_gemm_plan(m, w['n'], w['k'])})"
    os.makedirs(os.path.dirname(TRAFFIC_RECORD), exist_ok=True)
    json.dump(rec, open(TRAFFIC_RECORD, "w"), indent=1)
    print(json.dumps(rec))


def read_traffic_record(call_name, plan):
    """HBM bytes per launch of the dominant call from the committed counter
    record, or None when it was taken for another call or other kernels."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256_16") != kernel_sources_digest() or rec.get("call") != f"{call_name} ({plan})":
        return None
    return rec["traffic_bytes_per_launch"]


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
    # the same call on weights packed once into the stage-contiguous layout
    # (packing is a one-time weight transform, outside the timed region)
    pb, psf = nv.grouped_pack(b, bsf, N, K, E)
    del b, bsf
    torch.cuda.empty_cache()
    us_p = timed(torch, stream, lambda i: nv.nvfp4_grouped_gemm_packed(qa, sfa, pb, psf, off_t, alpha, d, rows, N, K,
                                                                       E), 10)
    res["grouped_moe_512tok_256exp_top8"]["packed_weights"] = dict(
        us=round(us_p, 2), gbps=round(by / us_p / 1e3, 1), frac_hbm=round(by / us_p / 1e3 / PEAK_HBM_GBPS, 4),
        tflops=round(fl / us_p / 1e6, 2))
    del pb, psf, qa, sfa, d
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
