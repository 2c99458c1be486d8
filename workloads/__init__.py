"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and lays them out; it contains none of
the operators' arithmetic (no GEMM, gather, scatter or reduction).  Both the
CPU oracle and the GPU library are fed from here, so neither needs to import
the other.

Recipe (all draws are numpy ``default_rng(seed)`` float32 normals, scaled in
float32, then rounded to the 16-bit format with round-to-nearest-even):
  * activations ~ N(0, 1); weights ~ N(0, 1) / sqrt(K) (K = reduction length),
    so every GEMM output entry is ~N(0, 1);
  * ReduceScatter destination slices (the peer partial sums already there)
    ~ N(0, 1) in float32;
  * MoE router: logits = N(0,1) + bias_e with bias_e = -s * ln(e + 1), the log
    of a Zipf(s) pmf up to a constant; softmax over all experts in float32; the
    top-k experts by probability (ties to the lower id); gate weights are the
    raw softmax probabilities (not renormalised).

The workload shapes follow the Flux README's quick-start commands (M N K =
4096 12288 6144 for the plain GEMM; 4096 49152 12288 and 4096 12288 49152 for
the AllGather and ReduceScatter MLP layers, here taken per rank at TP=8).
"""
from __future__ import annotations

import numpy as np

F16, BF16 = 0, 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's RNE cast); return bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, dt: int) -> np.ndarray:
    return f32_to_f16_bits(x) if dt == F16 else f32_to_bf16_bits(x)


def normal_f32(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def normal_bits(shape, seed: int, dt: int, scale: float = 1.0) -> np.ndarray:
    """16-bit patterns of N(0, scale^2) values in format ``dt``."""
    return to_bits(normal_f32(shape, seed, scale), dt)


def permutation(n: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).permutation(n).astype(np.int32)


# ---------------------------------------------------------------------------
# Dense GEMM / AllGather-GEMM / GEMM-ReduceScatter workloads
# ---------------------------------------------------------------------------

def gemm_inputs(M: int, N: int, K: int, dt: int = F16, seed: int = 201):
    """A [M,K] ~ N(0,1), B [K,N] ~ N(0,1)/sqrt(K)."""
    A = normal_bits((M, K), seed, dt)
    B = normal_bits((K, N), seed + 1, dt, 1.0 / np.sqrt(K))
    return A, B


def ag_inputs(n_chunks: int, Mc: int, N: int, K: int, dt: int = F16, seed: int = 301,
              arrival: str = "ring"):
    """Row chunks X_c [Mc,K] ~ N(0,1) (one per emulated rank), W [K,N] ~ N(0,1)/sqrt(K).

    ``arrival``: "ring" = chunk 0 is local (already present) and chunks 1..n-1
    arrive in that order; "random" = all chunks arrive in a seeded permutation.
    """
    chunks = normal_bits((n_chunks, Mc, K), seed, dt)
    W = normal_bits((K, N), seed + 1, dt, 1.0 / np.sqrt(K))
    if arrival == "random":
        order = permutation(n_chunks, seed + 2)
    else:
        order = np.arange(n_chunks, dtype=np.int32)
    return chunks, W, order


def rs_inputs(M: int, N: int, K: int, n_ranks: int, dt: int = F16, seed: int = 401):
    """A [M,K] ~ N(0,1), W [K,N] ~ N(0,1)/sqrt(K), n_ranks fp32 slices [M/n,N] ~ N(0,1)."""
    A = normal_bits((M, K), seed, dt)
    W = normal_bits((K, N), seed + 1, dt, 1.0 / np.sqrt(K))
    seeds = normal_f32((n_ranks, M // n_ranks, N), seed + 2)
    return A, W, seeds


# ---------------------------------------------------------------------------
# MoE workload
# ---------------------------------------------------------------------------

def moe_routing(T: int, n_experts: int, topk: int, seed: int, zipf_s: float = 1.2):
    """Router draws: logits N(0,1) + log-Zipf bias, softmax, top-k (ties -> lower id).

    Returns (topk_ids int32 [T,topk], topk_weights float32 [T,topk]).
    """
    logits = normal_f32((T, n_experts), seed)
    bias = (-zipf_s * np.log(np.arange(1, n_experts + 1, dtype=np.float64))).astype(np.float32)
    logits = logits + bias[None, :]
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m, dtype=np.float32)
    probs = ex / ex.sum(axis=1, keepdims=True, dtype=np.float32)
    ids = np.argsort(-probs, axis=1, kind="stable")[:, :topk].astype(np.int32)
    wts = np.take_along_axis(probs, ids, axis=1).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(wts)


def moe_inputs(T: int, hidden: int, ffn: int, n_experts: int, n_local: int, topk: int = 2,
               dt: int = BF16, seed: int = 501, zipf_s: float = 1.2):
    """Full MoE-layer inputs for one expert-parallel rank (local experts given separately)."""
    ids, wts = moe_routing(T, n_experts, topk, seed, zipf_s)
    X = normal_bits((T, hidden), seed + 1, dt)
    W1 = normal_bits((n_local, hidden, ffn), seed + 2, dt, 1.0 / np.sqrt(hidden))
    W2 = normal_bits((n_local, ffn, hidden), seed + 3, dt, 1.0 / np.sqrt(ffn))
    out_seed = normal_f32((T, hidden), seed + 4)
    return dict(topk_ids=ids, topk_weights=wts, X=X, W1=W1, W2=W2, out_seed=out_seed)


# ---------------------------------------------------------------------------
# Named workloads (tiny parity case and the full-size TP=8 / EP=8 rank-0 shares)
# ---------------------------------------------------------------------------

TINY_AG = dict(n_chunks=4, Mc=64, N=512, K=512, dt=F16, seed=101, arrival="random")
DENSE_GEMM = dict(M=4096, N=12288, K=6144, dt=F16, seed=201)
AG_TP8 = dict(n_chunks=8, Mc=512, N=6144, K=12288, dt=F16, seed=301, arrival="ring")
RS_TP8 = dict(M=4096, N=12288, K=6144, n_ranks=8, dt=F16, seed=401)
MOE_EP8 = dict(T=16384, hidden=4096, ffn=2816, n_experts=64, n_local=8, topk=2, dt=BF16,
               seed=501, zipf_s=1.2, rank=0)
