"""Benchmark of the gfx950 NVFP4 block-scaled GEMM.

One step = one pass over the pages' single-GEMM workloads across the metric's
range M = 16..8192: the attention projections (M in {16, 32, 64, 128, 256,
512, 1024} x N = 768 x K = 6144), the MoE expert shapes (M in {16, 32, 64,
256, 1024} x N = 2048 x K = 6144) and the compute-bound shapes (M in {4096,
8192} x N = 6144 x K = 6144): fourteen ``nvfp4_gemm`` calls on inputs already
quantised and resident in HBM.  Each call of a step reads the next of several
rotating buffer sets of its workload (each workload's sets together more than
twice the 256 MB Infinity Cache), so operands stream from HBM as in a real
pass over many layers.  ``value`` is the step's TFLOPS (2*M*N*K summed over
the fourteen calls / step time).

Printed as one JSON line, with per-shape results, the roofline of the
dominant call (timed with HIP events on the stream it runs on), the other
workloads of the pages (M = 16384, the grouped 256-expert MoE GEMM, the MoE
expert FFN, MXFP4, the vendor bf16 GEMM at every shape, the quantiser), and
the CPU oracle timed on one or more passes of the same step.
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
PEAK_FP4_TFLOPS = 10100.0     # dense FP4 MFMA, MI355X: the roofline's compute peak
PEAK_F16_TFLOPS = 2500.0      # dense f16 MFMA, MI355X: the instruction the exact path issues
PEAK_HBM_GBPS = 8000.0
ROTATE_BYTES = 600 << 20      # > 2 x 256 MB Infinity Cache
GRAPH_STEPS = 8               # steps captured per HIP graph
RAMP_S = 0.25                 # untimed clock ramp before the warmup steps (seconds)

# the step: (workload, the M values it contributes)
STEP = (("attn_proj_n768_k6144", (16, 32, 64, 128, 256, 512, 1024)),
        ("moe_expert_n2048_k6144", (16, 32, 64, 256, 1024)),
        ("large_n6144_k6144", (4096, 8192)))


def algo_bytes(M, N, K):
    """Bytes the method must move: packed codes + scales of A and B, bf16 D, alpha."""
    return (M + N) * K * 9 // 16 + 2 * M * N + 4


def roofline_frac(flops, nbytes, us):
    """max(flops / dense FP4 peak, bytes / HBM bandwidth) / measured time."""
    return max(flops / (PEAK_FP4_TFLOPS * 1e6), nbytes / (PEAK_HBM_GBPS * 1e3)) / us


def shape_row(nv, m, n, k, us, **extra):
    fl, by = 2.0 * m * n * k, algo_bytes(m, n, k)
    return dict(M=m, N=n, K=k, plan=nv.nvfp4_gemm_plan(m, n, k), us=round(us, 3),
                tflops=round(fl / us / 1e6, 2), gbps=round(by / us / 1e3, 1),
                frac_roofline=round(roofline_frac(fl, by, us), 4),
                frac_f16_mfma=round(fl / us / 1e6 / PEAK_F16_TFLOPS, 4),
                frac_hbm=round(by / us / 1e3 / PEAK_HBM_GBPS, 4), **extra)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads and the CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--ramp-seconds", type=float, default=RAMP_S,
                    help="untimed step replays before the warmup steps: the GPU clocks ramp up under sustained load")
    ap.add_argument("--workload", default="attn_proj_n768_k6144", help="workload of --profile-call")
    ap.add_argument("--profile-call", type=int, default=0, metavar="M",
                    help="for hardware-counter runs: one 256 MiB device copy (counter calibration), then 8 "
                         "cold calls of the --workload GEMM at this M; prints nothing else")
    ap.add_argument("--profile-grouped", action="store_true",
                    help="for profiler runs: one 256 MiB device copy (counter calibration), then the grouped "
                         "MoE GEMM on packed weights (graph of 10 calls, replayed 4 times); prints its time")
    ap.add_argument("--profile-grouped-plain", action="store_true",
                    help="for profiler runs: the grouped MoE GEMM on plain [E][N][K/2] weights with linear scales "
                         "(nvfp4_grouped_gemm; graph of 10 calls, replayed 6 times); prints its time")
    ap.add_argument("--profile-mx", type=int, default=0, metavar="M",
                    help="for profiler runs: the MXFP4 GEMM M x 6144 x 6144 (graph of 10 calls, replayed 6 times); "
                         "prints its time")
    ap.add_argument("--profile-quantize", action="store_true",
                    help="run only the quantiser workload (16384 x 6144 fp32) as the bench times it, for a profiler")
    ap.add_argument("--profile-fused", action="store_true",
                    help="run only the fused-quantisation grouped call (512 tokens, packed weights), for a profiler")
    ap.add_argument("--profile-moe", action="store_true",
                    help="run only the MoE expert FFN layer (512 tokens, top-8 of 256 experts) as the bench times "
                         "it, for a profiler")
    ap.add_argument("--graph", action="store_true",
                    help="with --profile-call: time the call as the bench does (graphs of back-to-back calls over "
                         "the rotating sets, replayed 8 times) instead of 8 eager calls")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a --profile-call or "
                         "--profile-grouped run into the HBM traffic record the bench reads (no GPU needed)")
    ap.add_argument("--requests", metavar="REQ_CSV",
                    help="with --traffic: a third counter CSV of the same run with TCC_EA0_RDREQ_32B_sum, "
                         "TCC_EA0_RDREQ_64B_sum, TCC_EA0_RDREQ_128B_sum, as a cross-check of the copy scaling")
    args = ap.parse_args()
    if args.traffic:
        if not args.profile_call and not args.profile_grouped and not args.profile_grouped_plain:
            raise SystemExit("--traffic needs the --profile-call M, --profile-grouped or --profile-grouped-plain the "
                             "counters were taken with")
        write_traffic_record(*args.traffic, args.requests,
                             "grouped" if args.profile_grouped else
                             "grouped_plain" if args.profile_grouped_plain else (args.workload, args.profile_call))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; multi-GPU sharding is a design note, "
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

    def sweep_inputs(name, ms=None, rotate=True):
        """Quantised operands of a workload (A at the largest M used), copied
        into rotating buffer sets of more than ROTATE_BYTES together, plus
        the alpha, outputs and workspaces of its M values."""
        w = dict(synth.WORKLOADS[name])
        w["ms"] = tuple(ms or w["ms"])
        a, b = synth.single_operands(name, max(w["ms"]))
        qa, sfa, gsa = quantise(a)
        qb, sfb, gsb = quantise(b)
        del a, b
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
        profile_call(torch, nv, sweep_inputs, call, args.workload, args.profile_call, args.graph)
        return
    if args.profile_grouped or args.profile_grouped_plain:
        profile_grouped(torch, nv, synth, quantise, stream, packed=args.profile_grouped)
        return
    if args.profile_mx:
        profile_mx(torch, nv, synth, stream, args.profile_mx)
        return
    if args.profile_quantize:
        us, by = quantize_workload(nv, torch, dev, stream, synth)
        print(json.dumps({"call": "nvfp4_quantize 16384 x 6144", "us_per_call": round(us, 2),
                          "gbps": round(by / us / 1e3, 1)}), flush=True)
        return
    if args.profile_fused:
        print(json.dumps(fused_grouped_workload(nv, torch, dev, stream, synth, quantise)), flush=True)
        return
    if args.profile_moe:
        print(json.dumps(moe_ffn_workload(nv, torch, dev, stream, synth)), flush=True)
        return

    # ------------------------------- the step -------------------------------
    # Steps are captured into HIP graphs, GRAPH_STEPS consecutive steps per
    # graph, as a serving loop would capture a whole pass; step j reads buffer
    # set j of each workload (modulo its count).  The host enqueues one replay
    # per GRAPH_STEPS steps and the GPU never waits on Python.
    inputs = [(name, ms) + sweep_inputs(name, ms) for name, ms in STEP]
    period = int(np.lcm.reduce([len(inp[3]) for inp in inputs]))   # steps until the set pattern repeats
    G = GRAPH_STEPS

    def step(j):
        for name, ms, w, sets, alpha, outs, wss in inputs:
            for m in ms:
                call(w, sets[j % len(sets)], alpha, outs, wss, m)

    ngraphs = min(max(1, -(-period // G)), 16)
    multi = [capture(torch, lambda j=j: [step(j * G + t) for t in range(G)]) for j in range(ngraphs)]
    single = [capture(torch, lambda t=t: step(t)) for t in range(G)]

    def run_steps(n, first):
        i = 0
        while n - i >= G:
            multi[((first + i) // G) % len(multi)].replay()
            i += G
        while i < n:
            single[(first + i) % G].replay()
            i += 1

    # clock ramp: untimed replays of the step graphs for ramp_seconds (as the
    # per-shape timings below replay for at least 50 ms before timing), then
    # the warmup steps, then exactly `steps` timed steps
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < args.ramp_seconds:
        run_steps(G, 0)
        torch.cuda.synchronize()
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
    flops_step = sum(2.0 * m * inp[2]["n"] * inp[2]["k"] for inp in inputs for m in inp[1])
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    del multi, single

    # per-call durations: a graph of back-to-back calls of one shape over the
    # rotating sets, timed with HIP events on the launch stream
    shapes = []
    for name, ms, w, sets, alpha, outs, wss in inputs:
        for m in ms:
            reps = min(len(sets), 64)
            g = capture(torch, lambda: [call(w, sets[i], alpha, outs, wss, m) for i in range(reps)])
            t_us = replay_us(torch, stream, g, reps)
            del g
            # the same calls on one buffer set (operands L2 / Infinity Cache resident)
            g = capture(torch, lambda: [call(w, sets[0], alpha, outs, wss, m) for _ in range(reps)])
            t_warm = replay_us(torch, stream, g, reps)
            del g
            shapes.append(shape_row(nv, m, w["n"], w["k"], t_us, workload=name, us_warm=round(t_warm, 3)))
    dom = max(shapes, key=lambda r: r["us"])
    fl = 2.0 * dom["M"] * dom["N"] * dom["K"]
    by = algo_bytes(dom["M"], dom["N"], dom["K"])
    call_name = f"nvfp4_gemm M={dom['M']} N={dom['N']} K={dom['K']} ({dom['plan']})"
    traffic = read_traffic_record(traffic_record_path(dom["workload"], dom["M"]), call_name)
    mfma_bound = fl / (PEAK_FP4_TFLOPS * 1e6) >= by / (PEAK_HBM_GBPS * 1e3)
    roofline = dict(bound="mfma" if mfma_bound else "hbm",
                    achieved=dom["tflops"] if mfma_bound else dom["gbps"],
                    peak=PEAK_FP4_TFLOPS if mfma_bound else PEAK_HBM_GBPS,
                    unit="TFLOP/s" if mfma_bound else "GB/s",
                    frac=round(roofline_frac(fl, by, dom["us"]), 4), traffic=traffic,
                    kernel_call=call_name, us=dom["us"], algorithmic_bytes=by, algorithmic_flops=fl,
                    frac_f16_mfma_issued=round(dom["tflops"] / PEAK_F16_TFLOPS, 4),
                    note="frac = max(flops / dense FP4 peak, bytes / 8 TB/s) / time of the dominant call; the exact "
                         "NVFP4 path issues f16 MFMAs (e4m3 scales per 16 elements are not powers of two), whose "
                         "dense peak is 2.5 PFLOP/s: frac_f16_mfma_issued")
    # launch floor: a graph of 64 one-element fills (the smallest kernel)
    tiny = torch.zeros(1, dtype=torch.float32, device=dev)
    g = capture(torch, lambda: [tiny.fill_(float(i)) for i in range(64)])
    launch_floor = replay_us(torch, stream, g, 64)
    del g, tiny
    del inputs
    torch.cuda.empty_cache()

    out = dict(metric=METRIC, value=round(value, 3), unit="TFLOPS", n_gpus=1, steps=args.steps,
               warmup=args.warmup, clock_ramp_s=args.ramp_seconds, ms_per_step=round(ms_per_step, 5),
               gpu_ms_per_step=round(gpu_ms / args.steps, 5),
               higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="f16", data="synthetic",
               config=dict(workload="nvfp4_gemm over M=16..8192: attn_proj_n768_k6144 (M 16..1024 x 768 x 6144) + "
                                    "moe_expert_n2048_k6144 (M 16..1024 x 2048 x 6144) + large_n6144_k6144 (M 4096, "
                                    "8192 x 6144 x 6144), bf16 out; every call cold: rotating HBM-resident buffer "
                                    "sets of more than 512 MB per workload",
                           calls={name: list(ms) for name, ms in STEP}, K=6144, block_size=16,
                           inputs="A ~ N(0,1), B ~ N(0,0.02), quantised on the GPU with per-tensor encode scales "
                                  "2688/amax, alpha = 1/(gsA*gsB)"),
               roofline=roofline, shapes=shapes,
               launch_floor_us=dict(us=round(launch_floor, 3),
                                    note="per kernel in a graph of 64 one-element fills: the floor under every call"))

    if not args.no_extra:
        out["other_workloads"] = other_workloads(nv, torch, dev, stream, synth, quantise, sweep_inputs, call)
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


GROUPED_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_grouped_moe_packed.json")
COPY_BYTES = 256 << 20


def _strip_c_comments(text):
    """C/C++ source without // and /* */ comments (string and character
    literals kept) and without trailing blanks, so that a comment edit does not
    change the digest."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(l.rstrip() for l in "".join(out).splitlines() if l.strip())


def kernel_sources_digest():
    """sha256 over the library's kernel sources (comments stripped) and the
    build's source list and compiler flags: a traffic record only holds for the
    kernels it was measured on."""
    import hashlib
    from nvfp4_block_scaled_07_amd import build as b
    h = hashlib.sha256()
    src = os.path.join(ROOT, "nvfp4_block_scaled_07_amd", "csrc")
    for f in sorted(os.listdir(src)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(_strip_c_comments(open(os.path.join(src, f)).read()).encode())
    h.update(repr((b.SOURCES, b.SCHED_SOURCES, [x for x in b.FLAGS if not os.path.isabs(x)])).encode())
    return h.hexdigest()[:16]


def traffic_record_path(workload, m):
    """Counter record of one nvfp4_gemm call of a workload."""
    return os.path.join(ROOT, "profiles", f"traffic_{workload}_m{m}.json")


def calibration_copy(torch):
    """A plain device copy of COPY_BYTES: it must fetch and write exactly
    COPY_BYTES, which calibrates the traffic counters."""
    x = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    del x, y


def profile_call(torch, nv, sweep_inputs, call, name, m, graph=False):
    """Workload of the profiler runs: a plain 256 MiB copy (its FETCH_SIZE and
    WRITE_SIZE calibrate the counters), then 8 cold calls of one GEMM of the
    step, or (graph=True) its per-call timing as the bench takes it: a graph
    of back-to-back calls over the rotating sets, replayed 8 times, with its
    HIP-event time printed."""
    calibration_copy(torch)
    w, sets, alpha, outs, wss = sweep_inputs(name, (m,))
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


def grouped_inputs(torch, nv, synth, quantise, dev):
    """The grouped MoE workload as stated: 512 tokens of N(0, 1) activations
    routed top-8 over 256 experts, quantised on the GPU with their encode
    scale and gathered per expert; each expert's [2048][6144] weights drawn
    N(0, 0.02) (the same seeded draws as the parity test) and quantised on the
    GPU with the expert's own encode scale; alpha[e] = 1 / (gs_a * gs_e)."""
    from concurrent.futures import ThreadPoolExecutor
    g = synth.GROUPED
    T, E, N, K = g["tokens"], g["experts"], g["n"], g["k"]
    tok, off = synth.routing(g["seed_router"], T, E, g["top_k"])
    rows = int(off[-1])
    x32 = synth.token_activations(T, K)
    qa_tok, sfa_tok, gsa = quantise(x32)
    tok_t = torch.from_numpy(tok).to(dev)
    qa, sfa = qa_tok[tok_t].contiguous(), sfa_tok[tok_t].contiguous()
    # the same tokens as bf16 activations, for the fused-quantisation call
    x_bf16 = torch.from_numpy(x32).to(dev).to(torch.bfloat16)
    b = torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev)
    bsf = torch.empty((E, N, K // 16), dtype=torch.uint8, device=dev)
    gs_e = torch.empty(E, dtype=torch.float32, device=dev)
    ahead = 16
    with ThreadPoolExecutor(8) as threads:
        futs = {e: threads.submit(synth.expert_weights, e, N, K) for e in range(min(ahead, E))}
        for e in range(E):
            w = torch.from_numpy(futs.pop(e).result()).to(dev)
            if e + ahead < E:
                futs[e + ahead] = threads.submit(synth.expert_weights, e + ahead, N, K)
            nv.nvfp4_global_scale(w, w.numel(), gs_e[e:e + 1])
            nv.nvfp4_quantize(w, N, K, gs_e[e:e + 1], b[e], bsf[e])
            del w
    alpha = torch.empty(E, dtype=torch.float32, device=dev)
    nv.nvfp4_alpha_from_scales(gsa, gs_e, alpha, E)
    active = int((np.diff(off) > 0).sum())
    return dict(rows=rows, N=N, K=K, E=E, T=T, qa=qa, sfa=sfa, b=b, bsf=bsf, off=torch.from_numpy(off).to(dev),
                x_bf16=x_bf16, tok=tok_t.to(torch.int32), gsa=gsa, alpha=alpha,
                d=torch.empty((rows, N), dtype=torch.int16, device=dev), active=active,
                rows_per_expert_max=int(np.diff(off).max()),
                # expert weights of the active experts, activations, bf16 out, offsets, alphas
                bytes=active * N * K * 9 // 16 + rows * K * 9 // 16 + 2 * rows * N + 4 * (E + 1) + 4 * E,
                flops=2.0 * rows * N * K)


def profile_mx(torch, nv, synth, stream, m):
    """Workload of the MXFP4 profiler runs: one M x 6144 x 6144 call, random
    codes and E8M0 scales in [120, 134], timed as the bench's large shapes."""
    N = K = 6144
    dev = torch.device("cuda")
    a = torch.from_numpy(synth.random_codes(9100, m, K)).to(dev)
    asf = torch.from_numpy(synth.random_scale_bytes(9101, m, 2 * K, 120, 134)[:, : K // 32].copy()).to(dev)
    b = torch.from_numpy(synth.random_codes(9102, N, K)).to(dev)
    bsf = torch.from_numpy(synth.random_scale_bytes(9103, N, 2 * K, 120, 134)[:, : K // 32].copy()).to(dev)
    d = torch.empty((m, N), dtype=torch.int16, device=dev)
    ws = nv.mx_gemm_workspace(m, N, K)
    us = timed(torch, stream, lambda i: nv.nvfp4_mx_gemm(a, asf, b, bsf, None, d, m, N, K, ws), 10)
    fl = 2.0 * m * N * K
    print(json.dumps({"call": f"nvfp4_mx_gemm M={m} N={N} K={K} ({nv.nvfp4_mx_gemm_plan(m, N, K)})",
                      "us_per_call": round(us, 2), "tflops": round(fl / us / 1e6, 1)}))


def grouped_call_name(rows, N, K, E):
    return f"nvfp4_grouped_gemm_packed rows={rows} N={N} K={K} E={E}"


def profile_grouped(torch, nv, synth, quantise, stream, packed=True):
    """Workload of the grouped profiler runs: the 256 MiB calibration copy,
    then the grouped MoE GEMM on packed expert weights (packed) or on the
    plain [E][N][K/2] weights with linear scales (nvfp4_grouped_gemm), timed
    as the bench times it (a graph of 10 calls); prints the call and its time."""
    calibration_copy(torch)
    gi = grouped_inputs(torch, nv, synth, quantise, torch.device("cuda"))
    rows, N, K, E = gi["rows"], gi["N"], gi["K"], gi["E"]
    if packed:
        pb, psf = nv.grouped_pack(gi["b"], gi["bsf"], N, K, E)
        del gi["b"], gi["bsf"]
        fn = lambda i: nv.nvfp4_grouped_gemm_packed(gi["qa"], gi["sfa"], pb, psf, gi["off"], gi["alpha"], gi["d"],
                                                     rows, N, K, E)
        name = grouped_call_name(rows, N, K, E)
    else:
        fn = lambda i: nv.nvfp4_grouped_gemm(gi["qa"], gi["sfa"], gi["b"], gi["bsf"], gi["off"], gi["alpha"], gi["d"],
                                              rows, N, K, E)
        name = f"nvfp4_grouped_gemm rows={rows} N={N} K={K} E={E}"
    us = timed(torch, stream, fn, 10)
    print(json.dumps({"call": name, "us_per_call": round(us, 2),
                      "algorithmic_bytes": gi["bytes"], "gbps": round(gi["bytes"] / us / 1e3, 1)}))


def _counter_rows(path, counter):
    import csv
    rows = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            rows.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return rows


def _is_copy(name):
    return "copybuffer" in name.lower()


def write_traffic_record(fetch_csv, write_csv, requests_csv, target):
    """FETCH_SIZE / WRITE_SIZE are in KiB per dispatch.  Each is scaled by
    what the same counter reads for the plain copy of COPY_BYTES (which must
    fetch and write exactly COPY_BYTES), then averaged over the dispatches of
    the profiled kernel.  With a third CSV of read requests by size
    (TCC_EA0_RDREQ_{32B,64B,128B}_sum), the fetched bytes are also summed
    request by request, for the copy and for the kernel, as a cross-check of
    the copy scaling (which assumes the kernel's request sizes match the copy's)."""
    import nvfp4_block_scaled_07_amd as nv
    import synth
    if target in ("grouped", "grouped_plain"):
        g = synth.GROUPED
        _, off = synth.routing(g["seed_router"], g["tokens"], g["experts"], g["top_k"])
        if target == "grouped":
            call = grouped_call_name(int(off[-1]), g["n"], g["k"], g["experts"])
            path_out = GROUPED_TRAFFIC_RECORD
        else:
            call = f"nvfp4_grouped_gemm rows={int(off[-1])} N={g['n']} K={g['k']} E={g['experts']}"
            path_out = os.path.join(os.path.dirname(GROUPED_TRAFFIC_RECORD), "traffic_grouped_moe_plain.json")
        match = "k_grouped"
    else:
        name, m = target
        w = synth.WORKLOADS[name]
        call = f"nvfp4_gemm M={m} N={w['n']} K={w['k']} ({nv.nvfp4_gemm_plan(m, w['n'], w['k'])})"
        match, path_out = "k_gemm", traffic_record_path(name, m)
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, counter)
        copies = [v for n, g_, v in rows if _is_copy(n)]
        kern = [(n, g_, v) for n, g_, v in rows if match in n]
        if not copies or not kern:
            raise SystemExit(f"{path}: no copy or no {match} dispatch with {counter}")
        calib = max(copies) * 1024.0 / COPY_BYTES
        out[counter] = dict(copy_kib=max(copies), factor=round(1.0 / calib, 6),
                            kernel_kib_mean=sum(v for _, _, v in kern) / len(kern),
                            bytes_per_launch=sum(v for _, _, v in kern) / len(kern) * 1024.0 / calib,
                            dispatches=len(kern), kernel=kern[0][0][:160], grid=kern[0][1])
    rec = dict(sources_sha256_16=kernel_sources_digest(), call=call, copy_bytes=COPY_BYTES, counters=out,
               traffic_bytes_per_launch=round(out["FETCH_SIZE"]["bytes_per_launch"] +
                                              out["WRITE_SIZE"]["bytes_per_launch"]))
    if requests_csv:
        import csv
        per = {}
        for r in csv.DictReader(open(requests_csv)):
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])

        def read_bytes(c):
            return (32 * c.get("TCC_EA0_RDREQ_32B_sum", 0) + 64 * c.get("TCC_EA0_RDREQ_64B_sum", 0) +
                    128 * c.get("TCC_EA0_RDREQ_128B_sum", 0))
        copy = max((read_bytes(c), c) for (i, n), c in per.items() if _is_copy(n))
        kern = [c for (i, n), c in per.items() if match in n]
        rec["read_requests"] = dict(
            copy_read_bytes=copy[0], copy_requests=copy[1],
            kernel_read_bytes_mean=sum(read_bytes(c) for c in kern) / len(kern),
            kernel_requests_mean={k: sum(c.get(k, 0) for c in kern) / len(kern) for k in sorted(kern[0])},
            dispatches=len(kern))
    os.makedirs(os.path.dirname(path_out), exist_ok=True)
    json.dump(rec, open(path_out, "w"), indent=1)
    print(json.dumps(rec))


def read_traffic_record(path, call):
    """HBM bytes per launch of `call` from a committed counter record, or None
    when the record was taken for another call or for other kernel sources."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256_16") != kernel_sources_digest() or rec.get("call") != call:
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


def replay_us(torch, stream, g, calls, repeats=5, warm_s=0.05):
    """Median over `repeats` replays of the per-call time (us) of a graph holding `calls` calls,
    after untimed replays for at least `warm_s` seconds (at least 3): the clocks ramp up under
    sustained load, and the inputs of several workloads are built on the host just before."""
    t0 = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t0 < warm_s:
        g.replay()
        torch.cuda.synchronize()
        n += 1
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
    # the largest compute-bound shape, beyond the metric's range (cold, rotating sets)
    w, sets, alpha, outs, wss = sweep_inputs("large_n6144_k6144", (16384,))
    us = timed(torch, stream, lambda i: call(w, sets[i % len(sets)], alpha, outs, wss, 16384), 2 * len(sets))
    res["large_n6144_k6144_m16384"] = dict(cache="cold (rotating sets)",
                                           shapes=[shape_row(nv, 16384, w["n"], w["k"], us)])
    del sets, outs, wss
    torch.cuda.empty_cache()

    # decode rows against a 16384 x 6144 weight (56.6 MB: the weight stream
    # at M <= 64 without the launch floor dominating; cold, rotating sets)
    w, sets, alpha, outs, wss = sweep_inputs("decode_wide_n16384_k6144")
    rows = []
    for m in w["ms"]:
        us = timed(torch, stream, lambda i: call(w, sets[i % len(sets)], alpha, outs, wss, m), 2 * len(sets))
        rows.append(shape_row(nv, m, w["n"], w["k"], us))
    res["decode_wide_n16384_k6144"] = dict(cache="cold (rotating sets)", shapes=rows)
    del sets, outs, wss
    torch.cuda.empty_cache()

    # grouped MoE: 512 tokens, top-8 of 256 experts, [rows_e, 6144] x [6144, 2048] per expert
    gi = grouped_inputs(torch, nv, synth, quantise, dev)
    rows, N, K, E = gi["rows"], gi["N"], gi["K"], gi["E"]
    qa, sfa, b, bsf, off_t, alpha, d = (gi[k] for k in ("qa", "sfa", "b", "bsf", "off", "alpha", "d"))
    need = nv.nvfp4_grouped_workspace_size(rows, N, K, E)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    us = timed(torch, stream, lambda i: nv.nvfp4_grouped_gemm(qa, sfa, b, bsf, off_t, alpha, d, rows, N, K, E, ws),
               10)
    by, fl = gi["bytes"], gi["flops"]
    res["grouped_moe_512tok_256exp_top8"] = dict(rows=rows, active_experts=gi["active"], N=N, K=K, us=round(us, 2),
                                                 gbps=round(by / us / 1e3, 1),
                                                 frac_hbm=round(by / us / 1e3 / PEAK_HBM_GBPS, 4),
                                                 tflops=round(fl / us / 1e6, 2),
                                                 rows_per_expert_max=gi["rows_per_expert_max"],
                                                 algorithmic_bytes=by)
    # the plain-weight call with both scale tensors in the 8 x 4 tiled layout,
    # read in place (nvfp4_grouped_gemm_sf; the weights' scales as one
    # [E * N][K/16] matrix), converted outside the timed region
    tsa = torch.empty(nv.nvfp4_scales_8x4_size(rows, K), dtype=torch.uint8, device=dev)
    tsb = torch.empty(nv.nvfp4_scales_8x4_size(E * N, K), dtype=torch.uint8, device=dev)
    nv.nvfp4_scales_to_8x4(sfa, tsa, rows, K)
    nv.nvfp4_scales_to_8x4(bsf.view(E * N, K // 16), tsb, E * N, K)
    us_t = timed(torch, stream, lambda i: nv.nvfp4_grouped_gemm_sf(qa, tsa, b, tsb, off_t, alpha, d, rows, N, K, E,
                                                                   nv.SF_8x4), 10)
    res["grouped_moe_512tok_256exp_top8"]["tiled_8x4_scales"] = dict(
        us=round(us_t, 2), gbps=round(by / us_t / 1e3, 1), frac_hbm=round(by / us_t / 1e3 / PEAK_HBM_GBPS, 4))
    del tsa, tsb
    # the same call on weights packed once into the stage-contiguous layout
    # (packing is a one-time weight transform, outside the timed region)
    pb, psf = nv.grouped_pack(b, bsf, N, K, E)
    T, x_bf16, tok_i32, gsa = gi["T"], gi["x_bf16"], gi["tok"], gi["gsa"]
    del b, bsf, gi
    torch.cuda.empty_cache()
    us_p = timed(torch, stream, lambda i: nv.nvfp4_grouped_gemm_packed(qa, sfa, pb, psf, off_t, alpha, d, rows, N, K,
                                                                       E), 10)
    res["grouped_moe_512tok_256exp_top8"]["packed_weights"] = dict(
        us=round(us_p, 2), gbps=round(by / us_p / 1e3, 1), frac_hbm=round(by / us_p / 1e3 / PEAK_HBM_GBPS, 4),
        tflops=round(fl / us_p / 1e6, 2),
        traffic=read_traffic_record(GROUPED_TRAFFIC_RECORD, grouped_call_name(rows, N, K, E)))
    # the MoE step from bf16 token activations: gather + quantise fused into
    # the GEMM's A load, against the unfused sequence (quantise kernel on the
    # tokens, row gather, grouped GEMM) on the same packed weights
    us_f = timed(torch, stream, lambda i: nv.nvfp4_grouped_gemm_packed_fused(
        x_bf16, tok_i32, gsa, pb, psf, off_t, alpha, d, rows, T, N, K, E), 10)
    x32 = x_bf16.float()
    q_tok = torch.empty((T, K // 2), dtype=torch.uint8, device=dev)
    sf_tok = torch.empty((T, K // 16), dtype=torch.uint8, device=dev)
    tok64 = tok_i32.long()

    def unfused(i):
        nv.nvfp4_quantize(x32, T, K, gsa, q_tok, sf_tok)
        torch.index_select(q_tok, 0, tok64, out=qa)
        torch.index_select(sf_tok, 0, tok64, out=sfa)
        nv.nvfp4_grouped_gemm_packed(qa, sfa, pb, psf, off_t, alpha, d, rows, N, K, E)
    us_u = timed(torch, stream, unfused, 10)
    # weights, bf16 tokens, row tokens, bf16 out, offsets, alphas
    by_f = by - rows * K * 9 // 16 + T * K * 2 + 4 * rows
    res["grouped_moe_512tok_256exp_top8"]["fused_quant_packed"] = dict(
        note="nvfp4_grouped_gemm_packed_fused: bf16 tokens gathered and quantised inside the GEMM",
        us=round(us_f, 2), gbps=round(by_f / us_f / 1e3, 1), frac_hbm=round(by_f / us_f / 1e3 / PEAK_HBM_GBPS, 4),
        algorithmic_bytes=by_f, unfused_pipeline_us=round(us_u, 2))
    del pb, psf, qa, sfa, d, x32, q_tok, sf_tok
    torch.cuda.empty_cache()

    # one MoE layer's experts (nvfp4_moe_ffn): 512 tokens, top-8 of 256
    # experts, H = 6144, I = 2048; gate/up grouped GEMM with the activation
    # gather and quantisation fused, SwiGLU + NVFP4, down grouped GEMM, combine
    res["moe_ffn_512tok_256exp_top8"] = moe_ffn_workload(nv, torch, dev, stream, synth)
    torch.cuda.empty_cache()

    # grouped calls with the same rows in every expert, weights >= 512 MB
    uni = []
    for u in synth.GROUPED_UNIFORM:
        N, K, E, me = u["n"], u["k"], u["experts"], u["rows_per_expert"]
        rows = E * me
        off = synth.uniform_offsets(me, E)
        qa = torch.from_numpy(synth.random_codes(u["seed"], rows, K)).to(dev)
        sfa = torch.from_numpy(synth.random_scale_bytes(u["seed"] + 1, rows, K, 0x20, 0x38)).to(dev)
        b = torch.from_numpy(synth.random_codes(u["seed"] + 2, E * N, K)).to(dev)
        bsf = torch.from_numpy(synth.random_scale_bytes(u["seed"] + 3, E * N, K, 0x20, 0x38)).to(dev)
        off_t = torch.from_numpy(off).to(dev)
        d = torch.empty((rows, N), dtype=torch.int16, device=dev)
        by = E * N * K * 9 // 16 + rows * K * 9 // 16 + 2 * rows * N + 4 * (E + 1)
        fl = 2.0 * rows * N * K
        need = nv.nvfp4_grouped_workspace_size(rows, N, K, E)
        ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        us = timed(torch, stream, lambda i: nv.nvfp4_grouped_gemm(qa, sfa, b, bsf, off_t, None, d, rows, N, K, E, ws),
                   10)
        pb, psf = nv.grouped_pack(b, bsf, N, K, E)
        del b, bsf
        us_p = timed(torch, stream, lambda i: nv.nvfp4_grouped_gemm_packed(qa, sfa, pb, psf, off_t, None, d, rows, N,
                                                                           K, E), 10)
        uni.append(dict(E=E, rows_per_expert=me, N=N, K=K, algorithmic_bytes=by,
                        us=round(us, 2), frac_hbm=round(by / us / 1e3 / PEAK_HBM_GBPS, 4),
                        packed_us=round(us_p, 2), packed_gbps=round(by / us_p / 1e3, 1),
                        packed_frac_hbm=round(by / us_p / 1e3 / PEAK_HBM_GBPS, 4),
                        packed_tflops=round(fl / us_p / 1e6, 2)))
        del pb, psf, qa, sfa, d, ws
        torch.cuda.empty_cache()
    res["grouped_uniform_experts"] = dict(cache="cold (weights >= 512 MB)", shapes=uni)

    # MXFP4 (E8M0 scale per 32 elements, the scaled FP4 MFMA): the attention
    # sweep (cold, rotating sets) and the large shapes, random codes and scales
    mxr = {}
    for name, rotate, reps in (("attn_proj_n768_k6144", True, 64), ("large_n6144_k6144", True, 16)):
        w = synth.WORKLOADS[name]
        N, K = w["n"], w["k"]
        rows = []
        for m in w["ms"]:
            per = (m + N) * K * 17 // 32
            nsets = max(1, -(-ROTATE_BYTES // per)) if rotate else 1
            sets = []
            for i in range(nsets):
                sd = 9000 + 10 * i if i < 2 else None
                if sd is None:
                    sets.append(tuple(t.clone() for t in sets[i % 2]))
                    continue
                sets.append((torch.from_numpy(synth.random_codes(sd, m, K)).to(dev),
                             torch.from_numpy(synth.random_scale_bytes(sd + 1, m, 2 * K, 120, 134)[:, : K // 32]
                                              .copy()).to(dev),
                             torch.from_numpy(synth.random_codes(sd + 2, N, K)).to(dev),
                             torch.from_numpy(synth.random_scale_bytes(sd + 3, N, 2 * K, 120, 134)[:, : K // 32]
                                              .copy()).to(dev)))
            d = torch.empty((m, N), dtype=torch.int16, device=dev)
            ws = nv.mx_gemm_workspace(m, N, K)
            r = min(reps, max(len(sets), 8)) if rotate else reps
            us = timed(torch, stream, lambda i: nv.nvfp4_mx_gemm(*sets[i % len(sets)], None, d, m, N, K, ws), r)
            fl = 2.0 * m * N * K
            rows.append(dict(M=m, N=N, K=K, plan=nv.nvfp4_mx_gemm_plan(m, N, K), us=round(us, 2),
                             tflops=round(fl / us / 1e6, 2), frac_fp4_peak=round(fl / us / 1e6 / PEAK_FP4_TFLOPS, 4)))
            del sets, d, ws
            torch.cuda.empty_cache()
        mxr[name] = dict(cache="cold (rotating sets)" if rotate else "warm", shapes=rows)
    res["mxfp4"] = mxr

    # context: the vendor bf16 GEMM (torch.matmul -> hipBLASLt) on already
    # dequantised operands at the same shapes, cold as above (the MI355X
    # counterpart of the pages' FP4-vs-BF16 throughput comparison)
    ref = []
    step_shapes = [(m, synth.WORKLOADS[name]["n"], synth.WORKLOADS[name]["k"]) for name, ms in STEP for m in ms]
    for (m, n, k) in step_shapes + [(16384, 6144, 6144)]:
        per = (m * k + k * n) * 2
        nsets = max(1, min(64, (ROTATE_BYTES + per - 1) // per))
        gen = torch.Generator(device=dev).manual_seed(m * 7 + n)
        xa = [torch.randn(m, k, device=dev, dtype=torch.bfloat16, generator=gen) for _ in range(nsets)]
        xb = [torch.randn(k, n, device=dev, dtype=torch.bfloat16, generator=gen)
              for _ in range(nsets)]  # [K][N], contiguous
        reps = max(nsets, 8) if m <= 1024 else 2 * nsets
        us = timed(torch, stream, lambda i: torch.matmul(xa[i % nsets], xb[i % nsets]), reps)
        ref.append(dict(M=m, N=n, K=k, us=round(us, 2), tflops=round(2.0 * m * n * k / us / 1e6, 1)))
        del xa, xb
        torch.cuda.empty_cache()
    res["bf16_matmul_reference"] = dict(note="torch.matmul bf16 x bf16 -> bf16 (hipBLASLt) at every shape of "
                                             "the step and M = 16384, operands already dequantised (N(0,1) "
                                             "draws), rotating sets of more than 512 MB; context only",
                                        shapes=ref)

    # decode calls on scales in the tiled layouts (nvfp4_gemm_sf; the register
    # tiles read them in place) against the same calls on linear scales, cold
    tiled = []
    for name, m in (("attn_proj_n768_k6144", 16), ("attn_proj_n768_k6144", 64), ("moe_expert_n2048_k6144", 64)):
        w, sets, alpha, outs, wss = sweep_inputs(name, (m,))
        n, k = w["n"], w["k"]
        layouts = ((nv.SF_128x4, "sf128x4_us", nv.nvfp4_scales_128x4_size, nv.nvfp4_scales_to_128x4),
                   (nv.SF_8x4, "sf8x4_us", nv.nvfp4_scales_8x4_size, nv.nvfp4_scales_to_8x4))
        tsets = []
        for qa, sfa, qb, sfb in sets:
            t = {}
            for lay, _, size, to in layouts:
                ta = torch.empty(size(m, k), dtype=torch.uint8, device=dev)
                tb = torch.empty(size(n, k), dtype=torch.uint8, device=dev)
                to(sfa[:m], ta, m, k)
                to(sfb, tb, n, k)
                t[lay] = (ta, tb)
            tsets.append(t)
        reps, ns = 2 * len(sets), len(sets)
        row = dict(M=m, N=n, K=k, plan=nv.nvfp4_gemm_plan(m, n, k),
                   linear_us=round(timed(torch, stream, lambda i: call(w, sets[i % ns], alpha, outs, wss, m), reps), 2))
        for lay, key, _, _ in layouts:
            need = nv.nvfp4_gemm_sf_workspace_size(m, n, k, lay)
            ws = nv.nvfp4_workspace_init(torch.empty(need, dtype=torch.uint8, device=dev)) if need else None
            row[key] = round(timed(torch, stream, lambda i: nv.nvfp4_gemm_sf(
                sets[i % ns][0][:m], tsets[i % ns][lay][0], sets[i % ns][2], tsets[i % ns][lay][1], alpha, outs[m],
                m, n, k, lay, ws), reps), 2)
        tiled.append(row)
        del sets, tsets, outs, wss
        torch.cuda.empty_cache()
    res["tiled_scales"] = dict(note="nvfp4_gemm_sf with both scale tensors in the 128 x 4 or 8 x 4 tiled layout, "
                                    "read in place by the register tiles, against nvfp4_gemm on linear scales; "
                                    "cold (rotating sets)", shapes=tiled)

    # quantiser (prologue): 16384 x 6144 fp32 -> NVFP4
    us, by = quantize_workload(nv, torch, dev, stream, synth)
    res["quantize_16384x6144"] = dict(us=round(us, 2), gbps=round(by / us / 1e3, 1),
                                      frac_hbm=round(by / us / 1e3 / PEAK_HBM_GBPS, 4))
    return res


def quantize_workload(nv, torch, dev, stream, synth):
    """nvfp4_quantize on 16384 x 6144 fp32 activations (gs = 1), timed as a
    graph of 10 calls; returns (us per call, bytes moved per call)."""
    x = torch.from_numpy(synth.normal_f32(4001, (16384, 6144))).to(dev)
    q = torch.empty((16384, 3072), dtype=torch.uint8, device=dev)
    sf = torch.empty((16384, 384), dtype=torch.uint8, device=dev)
    gs = torch.ones(1, dtype=torch.float32, device=dev)
    us = timed(torch, stream, lambda i: nv.nvfp4_quantize(x, 16384, 6144, gs, q, sf), 10)
    return us, 16384 * 6144 * (4 + 0.5 + 1 / 16)


def fused_grouped_workload(nv, torch, dev, stream, synth, quantise):
    """The 512-token grouped call from bf16 token activations with the gather
    and quantisation fused into the A load (packed weights), timed as a graph
    of 10 calls."""
    gi = grouped_inputs(torch, nv, synth, quantise, dev)
    rows, N, K, E, T = gi["rows"], gi["N"], gi["K"], gi["E"], gi["T"]
    pb, psf = nv.grouped_pack(gi["b"], gi["bsf"], N, K, E)
    del gi["b"], gi["bsf"]
    torch.cuda.empty_cache()
    us = timed(torch, stream, lambda i: nv.nvfp4_grouped_gemm_packed_fused(
        gi["x_bf16"], gi["tok"], gi["gsa"], pb, psf, gi["off"], gi["alpha"], gi["d"], rows, T, N, K, E), 10)
    return dict(call=f"nvfp4_grouped_gemm_packed_fused rows={rows} T={T} N={N} K={K} E={E}", us_per_call=round(us, 2))


def moe_ffn_workload(nv, torch, dev, stream, synth):
    g = synth.GROUPED
    T, E, H, k = g["tokens"], g["experts"], g["k"], g["top_k"]
    I = g["n"]
    tok, off = synth.routing(g["seed_router"], T, E, k)
    rows = int(off[-1])
    tr = synth.token_rows(tok, T, k)
    tw = synth.routing_weights(g["seed_router"] + 1, T, k)
    x32 = torch.from_numpy(synth.token_activations(T, H)).to(dev)
    x = x32.to(torch.bfloat16)
    gs_x = torch.empty(1, dtype=torch.float32, device=dev)
    nv.nvfp4_global_scale(x32, x32.numel(), gs_x)
    del x32

    def packed(seed, N, K):
        b = torch.from_numpy(synth.random_codes(seed, E * N, K)).to(dev)
        bsf = torch.from_numpy(synth.random_scale_bytes(seed + 1, E * N, K, 0x20, 0x38)).to(dev)
        pb, psf = nv.grouped_pack(b, bsf, N, K, E)
        del b, bsf
        torch.cuda.empty_cache()
        return pb, psf
    pgu, pgusf = packed(g["seed_expert_base"] + 100, 2 * I, H)
    pd, pdsf = packed(g["seed_expert_base"] + 200, H, I)
    a_gu = torch.full((E,), 1e-4, dtype=torch.float32, device=dev)
    a_d = torch.full((E,), 1e-3, dtype=torch.float32, device=dev)
    gs_h = torch.ones(1, dtype=torch.float32, device=dev)
    tok_t = torch.from_numpy(tok.astype(np.int32)).to(dev)
    off_t = torch.from_numpy(off).to(dev)
    tr_t, tw_t = torch.from_numpy(tr).to(dev), torch.from_numpy(tw).to(dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(nv.nvfp4_moe_ffn_workspace_size(T, H, I, k), dtype=torch.uint8, device=dev)
    us = timed(torch, stream, lambda i: nv.nvfp4_moe_ffn(x, gs_x, tok_t, off_t, pgu, pgusf, a_gu, gs_h, pd, pdsf,
                                                         a_d, tr_t, tw_t, out, T, H, I, E, k, ws), 10)
    active = int((np.diff(off) > 0).sum())
    # expert weights, bf16 tokens in and out, routing indices and weights
    by = active * 3 * I * H * 9 // 16 + 2 * T * H * 2 + rows * 4 + T * k * 8 + 4 * (E + 1) + 8 * E
    fl = 2.0 * rows * 3 * I * H
    del pgu, pgusf, pd, pdsf, ws
    return dict(note="nvfp4_moe_ffn: gather+quantise of the routed tokens, gate/up grouped GEMM, SwiGLU+NVFP4, "
                     "down grouped GEMM, combine; packed expert weights", T=T, H=H, I=I, E=E, top_k=k, us=round(us, 2),
                gbps=round(by / us / 1e3, 1), frac_hbm=round(by / us / 1e3 / PEAK_HBM_GBPS, 4),
                tflops=round(fl / us / 1e6, 2), algorithmic_bytes=by)


def blas_info():
    """(BLAS library name and version, its thread count) as numpy reports them."""
    name = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {})
        name = f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"]
                      or [0]) or None
    except Exception:
        pass
    return name, threads


def cpu_baseline(seconds):
    """The oracle (numpy: LUT dequant to fp64, BLAS dgemm, RNE to bf16) on the
    step's fourteen shapes, whole passes repeated for at least `seconds` of
    wall time.  The oracle's time does not depend on the values, so its
    inputs are seeded random codes and scale bytes of the same shapes."""
    import synth
    from oracle import nvfp4_ref as o
    blas, blas_threads = blas_info()
    per_config = {}
    data = {}
    for name, ms in STEP:
        w = synth.WORKLOADS[name]
        mmax, n, k = max(ms), w["n"], w["k"]
        data[name] = (synth.random_codes(8001, mmax, k), synth.random_scale_bytes(8002, mmax, k, 0x30, 0x40),
                      synth.random_codes(8003, n, k), synth.random_scale_bytes(8004, n, k, 0x30, 0x40))
        per_config[name] = dict(seconds=0.0, flops=0.0)
    passes = 0
    t0 = time.perf_counter()
    while True:
        for name, ms in STEP:
            qa, sfa, qb, sfb = data[name]
            w = synth.WORKLOADS[name]
            for m in ms:
                t = time.perf_counter()
                o.gemm(qa[:m], sfa[:m], qb, sfb, np.float32(1.0))
                per_config[name]["seconds"] += time.perf_counter() - t
                per_config[name]["flops"] += 2.0 * m * w["n"] * w["k"]
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    total = time.perf_counter() - t0
    flops = sum(v["flops"] for v in per_config.values())
    return dict(value=round(flops / total / 1e12, 5), unit="TFLOPS", cores=len(os.sched_getaffinity(0)),
                kind="oracle", blas=blas, blas_threads=blas_threads,
                per_config={name: dict(tflops=round(v["flops"] / v["seconds"] / 1e12, 5),
                                       seconds_per_pass=round(v["seconds"] / passes, 3))
                            for name, v in per_config.items()},
                sample=f"{passes} whole passes of the step's 14 shapes (M 16..1024 x 768, M 16..1024 x 2048, "
                       f"M 4096 and 8192 x 6144; K = 6144) in {total:.1f} s on {len(os.sched_getaffinity(0))} "
                       f"cores: LUT dequant to fp64, dgemm, RNE to bf16")


if __name__ == "__main__":
    main()
