"""Every-element forms of the oracle's dense and MoE operators, for the
full-size workloads.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/`` may
import it; the product path never does, and it shares no code with the HIP
library.

The C oracle (``fm_oracle.c``) computes each output with explicit fp64 loops.
That is too slow for every element of the full-size workloads (3e11 to 4e11
multiply-adds each), so its full-size checks sample outputs.  The functions
here compute the same definitions for every element: the 16-bit inputs are
decoded exactly to float64, rows are gathered, numpy's float64 matrix product
is the one library step, and results are scattered or added in float64.
There is no blocking or reordering beyond what the definitions state.

Sources, by page and section:
  * FLUX paper review, section 三, "MLP 前向传播": Output1 = GEMM(AllGather(X),
    W1); Output2 = ReduceScatter(GEMM(Output1, W2)), each rank keeping the sum
    of its row slice.
  * COMET article, "COMET 的技术原理": layer 0 gathers each local expert's
    token rows and multiplies them by that expert's weights; the combine adds
    every local (token, k) result row, times its gate weight, into the token's
    output row.

Pins: ``tests/oracle_pins.py`` (``pin_full_*``) ties each function to the C
oracle's loops, to brute force on tiny inputs and to the hand-worked fixtures
in ``tests/golden/``.
"""
from __future__ import annotations

import numpy as np

F16, BF16 = 0, 1


def decode(dt: int, bits: np.ndarray) -> np.ndarray:
    """16-bit storage bits -> float64, exactly (IEEE binary16, or bfloat16 as
    the top half of an IEEE binary32)."""
    b = np.ascontiguousarray(bits)
    if b.dtype == np.float16:
        b = b.view(np.uint16)
    assert b.dtype == np.uint16, b.dtype
    if dt == F16:
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm(dt: int, A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C = A B for A [M,K] and B [K,N] (16-bit bits), in float64."""
    assert A.ndim == 2 and B.ndim == 2 and A.shape[1] == B.shape[0], (A.shape, B.shape)
    return decode(dt, A) @ decode(dt, B)


def ag_gemm(dt: int, chunks, W: np.ndarray) -> np.ndarray:
    """GEMM(AllGather(X), W): chunk c holds rows [c*Mc, (c+1)*Mc) of X, whatever
    order the chunks arrive in."""
    return gemm(dt, np.concatenate([np.asarray(c) for c in chunks], axis=0), W)


def gemm_rs(dt: int, A: np.ndarray, W: np.ndarray, seeds) -> list:
    """Rank-local share of GEMM-ReduceScatter: slice p of A W (rows
    [p*M/P, (p+1)*M/P)) added onto the fp32 destination seeds[p]."""
    P = len(seeds)
    M = A.shape[0]
    assert M % P == 0
    C = gemm(dt, A, W)
    Ms = M // P
    return [np.asarray(s, dtype=np.float64) + C[p * Ms:(p + 1) * Ms] for p, s in enumerate(seeds)]


def moe_layer0(dt: int, X: np.ndarray, W1: np.ndarray, sorted_pairs, offsets,
               topk: int) -> np.ndarray:
    """H row r = X[token of pair sorted_pairs[r]] W1[e] for the local expert e
    whose row range [offsets[e], offsets[e+1]) holds r.  A pair id p is token
    p // topk, choice p % topk."""
    off = np.asarray(offsets, dtype=np.int64)
    sp = np.asarray(sorted_pairs, dtype=np.int64)
    n_local, hidden, ffn = W1.shape
    assert X.shape[1] == hidden and off.shape[0] == n_local + 1
    x = decode(dt, X)
    H = np.empty((int(off[-1]), ffn), dtype=np.float64)
    for e in range(n_local):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            H[r0:r1] = x[sp[r0:r1] // topk] @ decode(dt, W1[e])
    return H


def moe_layer1(dt: int, H: np.ndarray, W2: np.ndarray, topk_ids, topk_weights, sorted_pairs,
               offsets, seed, e0: int) -> np.ndarray:
    """out[t] = seed[t] + sum over k with a local expert e = topk_ids[t,k] - e0
    of topk_weights[t,k] * (H[row of pair t*topk+k] W2[e]), in float64.

    The terms are added expert by expert, and within an expert by k; for one
    (expert, k) every token has at most one pair, so each step adds into
    distinct rows."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    wts = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, topk = ids.shape
    n_local, ffn, hidden = W2.shape
    sp = np.asarray(sorted_pairs, dtype=np.int64)
    rows = int(np.asarray(offsets)[-1])
    row_of_pair = np.full(T * topk, -1, dtype=np.int64)
    row_of_pair[sp[:rows]] = np.arange(rows)
    h = decode(dt, H)
    out = np.array(seed, dtype=np.float64, copy=True)
    assert out.shape == (T, hidden)
    for e in range(n_local):
        w2 = decode(dt, W2[e])
        for k in range(topk):
            toks = np.nonzero(ids[:, k] == e0 + e)[0]
            if toks.size == 0:
                continue
            r = row_of_pair[toks * topk + k]
            assert (r >= 0).all(), "a local pair has no row"
            out[toks] += wts[toks, k][:, None] * (h[r] @ w2)
    return out
