"""Seeded synthetic inputs shared by the tests, the bench and the smoke run.

This module holds no arithmetic of the method: it only draws random numbers
(numpy PCG64 via ``default_rng``) and routes tokens to experts.  Quantisation,
scales and alpha are computed independently by the oracle (numpy) and by the
HIP library.

Workloads are the shapes of the pages (P3 = "When a Benchmark Crashes: The
Elusive FP4 GEMM Comparison on Blackwell SM120", sections "Why This Message
Was Written" and "Assumptions Made" item 3: M x 768 x 6144 attention
projections and M x 2048 x 6144 MoE experts for M from 16 to 1024; GLM-5 with
hidden size 6144, MoE intermediate size 2048, 256 experts, 8 active per
token).  The model's weights and activations are not available, so N(0, 1)
activations and N(0, 0.02) weights stand in for them.
"""
from __future__ import annotations

import numpy as np

K_HIDDEN = 6144
N_ATTN = 768
N_EXPERT = 2048
NUM_EXPERTS = 256
TOP_K = 8

# name -> description of a single-GEMM workload (M sweep, N, K, seeds, sigmas)
WORKLOADS = {
    # p1 smoke shape: M=128, N=256, K=256, both operands N(0,1), unit global scale
    "smoke_128x256x256": dict(ms=(128,), n=256, k=256, seed_a=1001, seed_b=1002,
                              sigma_a=1.0, sigma_b=1.0, unit_global_scale=True),
    "attn_proj_n768_k6144": dict(ms=(16, 32, 64, 128, 256, 512, 1024), n=N_ATTN, k=K_HIDDEN,
                                 seed_a=2001, seed_b=2002, sigma_a=1.0, sigma_b=0.02,
                                 unit_global_scale=False),
    "moe_expert_n2048_k6144": dict(ms=(16, 32, 64, 256, 1024), n=N_EXPERT, k=K_HIDDEN,
                                   seed_a=3001, seed_b=3002, sigma_a=1.0, sigma_b=0.02,
                                   unit_global_scale=False),
    "large_n6144_k6144": dict(ms=(4096, 8192, 16384), n=K_HIDDEN, k=K_HIDDEN,
                              seed_a=4001, seed_b=4002, sigma_a=1.0, sigma_b=0.02,
                              unit_global_scale=False),
    # decode rows against a weight large enough to stream from HBM (56.6 MB of
    # codes and scales): not one of the pages' shapes; it shows the weight
    # stream of the single GEMM at M <= 64 without the launch floor dominating
    "decode_wide_n16384_k6144": dict(ms=(16, 32, 64), n=16384, k=K_HIDDEN,
                                     seed_a=6001, seed_b=6002, sigma_a=1.0, sigma_b=0.02,
                                     unit_global_scale=False),
}

GROUPED = dict(tokens=512, experts=NUM_EXPERTS, top_k=TOP_K, n=N_EXPERT, k=K_HIDDEN,
               seed_a=5001, seed_router=5003, seed_expert_base=5000 + 10000, sigma_b=0.02)


# Grouped calls of E experts with the same row count each: per-expert rows
# 16, 32, 64 at both expert widths, with weights totalling >= 512 MB so that
# they stream from HBM (256 experts x 768 x 6144 -> 679 MB; 80 x 2048 x 6144
# -> 566 MB).  Random code bytes and scale bytes 0x20..0x38 on both sides.
GROUPED_UNIFORM = [dict(n=n, rows_per_expert=m, experts=e, k=K_HIDDEN, seed=7000 + 10 * i)
                   for i, (n, e, m) in enumerate([(768, 256, 16), (768, 256, 32), (768, 256, 64),
                                                  (2048, 80, 16), (2048, 80, 32), (2048, 80, 64)])]


def uniform_offsets(rows_per_expert: int, experts: int) -> np.ndarray:
    """offsets int32[experts+1] with rows_per_expert rows in every expert."""
    return (np.arange(experts + 1, dtype=np.int64) * rows_per_expert).astype(np.int32)


def normal_f32(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma^2) float32 draws from PCG64(seed)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def single_operands(name: str, m: int | None = None):
    """(A fp32 [M][K], B fp32 [N][K]) for a single-GEMM workload.  A is drawn
    at the largest M of the sweep and sliced, so sweeps are nested."""
    w = WORKLOADS[name]
    mmax = max(w["ms"])
    m = mmax if m is None else m
    if m > mmax:
        a = normal_f32(w["seed_a"], (m, w["k"]), w["sigma_a"])
    else:
        a = normal_f32(w["seed_a"], (mmax, w["k"]), w["sigma_a"])[:m]
    b = normal_f32(w["seed_b"], (w["n"], w["k"]), w["sigma_b"])
    return np.ascontiguousarray(a), b


def expert_weights(e: int, n: int = N_EXPERT, k: int = K_HIDDEN) -> np.ndarray:
    """fp32 [N][K] weights of expert e, N(0, 0.02)."""
    return normal_f32(GROUPED["seed_expert_base"] + e, (n, k), GROUPED["sigma_b"])


def token_activations(tokens: int = 512, k: int = K_HIDDEN) -> np.ndarray:
    return normal_f32(GROUPED["seed_a"], (tokens, k), 1.0)


def routing(seed: int, tokens: int, experts: int, top_k: int):
    """Top-k routing from N(0,1) logits [tokens][experts].

    Softmax is monotone, so ranking the logits ranks the probabilities; ties
    break towards the lower expert id (stable sort on -logit).  Rows are
    ordered by expert, then token.  Returns (token_of_row int64[tokens*top_k],
    offsets int32[experts+1])."""
    logits = normal_f32(seed, (tokens, experts), 1.0)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]   # [T][top_k]
    tok = np.repeat(np.arange(tokens, dtype=np.int64), top_k)
    exp = order.reshape(-1).astype(np.int64)
    perm = np.lexsort((tok, exp))                                    # expert, then token
    token_of_row = tok[perm]
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return token_of_row, offsets


def token_rows(token_of_row: np.ndarray, tokens: int, top_k: int) -> np.ndarray:
    """Inverse of the routing's row order: int32[tokens][top_k], the rows of
    each token in ascending row order."""
    order = np.argsort(token_of_row, kind="stable")
    return order.reshape(tokens, top_k).astype(np.int32)


def routing_weights(seed: int, tokens: int, top_k: int) -> np.ndarray:
    """Seeded positive combine weights float32[tokens][top_k] summing to about 1."""
    w = np.random.default_rng(seed).uniform(0.05, 1.0, size=(tokens, top_k))
    return (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def random_codes(seed: int, rows: int, k: int) -> np.ndarray:
    """Uniform random packed bytes uint8[rows][k/2] (every e2m1 code pair)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)


def random_scale_bytes(seed: int, rows: int, k: int, lo: int = 0x00, hi: int = 0x7E,
                       signed: bool = False) -> np.ndarray:
    """Random e4m3 scale bytes uint8[rows][k/16] with codes in [lo, hi]
    (0x7F, the NaN code, is excluded by the default range); optionally a
    random sign bit."""
    rng = np.random.default_rng(seed)
    s = rng.integers(lo, hi + 1, size=(rows, k // 16), dtype=np.int64)
    if signed:
        s |= rng.integers(0, 2, size=s.shape) << 7
    return s.astype(np.uint8)


def adversarial_offsets(kind: str, rows: int, experts: int) -> np.ndarray:
    """Row-count distributions for grouped tests: 'one' (all rows in one
    expert), 'alternate' (64, 0, 64, 0, ...), 'ones' (one row each, then 0),
    'empty' (no rows at all)."""
    counts = np.zeros(experts, dtype=np.int64)
    if kind == "one":
        counts[experts // 2] = rows
    elif kind == "alternate":
        left = rows
        for e in range(0, experts, 2):
            c = min(64, left)
            counts[e] = c
            left -= c
        counts[-1] += left
    elif kind == "ones":
        c = min(rows, experts)
        counts[:c] = 1
        counts[-1] += rows - c
    elif kind == "empty":
        pass
    else:
        raise ValueError(kind)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return offsets


def fp32_bit_patterns(lo: int, hi: int, negative: bool = False) -> np.ndarray:
    """The fp32 values whose bit patterns are lo, lo + 1, ..., hi - 1 (all
    below 2^31), with the sign bit set when ``negative``: the inputs of the
    exhaustive rounding sweep."""
    if not 0 <= lo <= hi <= 1 << 31:
        raise ValueError("pattern range must lie in [0, 2^31]")
    bits = np.arange(lo, hi, dtype=np.uint32)
    if negative:
        bits |= np.uint32(0x80000000)
    return bits.view(np.float32)
