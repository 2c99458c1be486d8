"""Pins for the CPU oracle: each check ties one oracle function to something
other than itself -- a textbook routine (numpy float64 matmul, bincount,
cumsum, stable argsort), a closed form, an invariant, a hand-worked example
from tests/golden/, or brute force on tiny inputs.

Every check takes an ``oracle.Oracle`` and raises AssertionError on failure,
so the same checks can be run against builds with a planted mistake (see
test_oracle_mutants.py) to show that they would catch it.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F16, BF16 = 0, 1


# -- independent decoders (numpy's own float16 / float32 reinterpretation) --

def np_decode(bits: np.ndarray, dt: int) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if dt == F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(vals, dt):
    v = np.asarray(vals, dtype=np.float32)
    return wl.to_bits(v, dt)


# ---------------------------------------------------------------------------
# element formats
# ---------------------------------------------------------------------------

def pin_decode_exhaustive(o):
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt in (F16, BF16):
        mine = o.decode(dt, allbits)
        ref = np_decode(allbits, dt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(mine), nan)
        assert np.array_equal(mine[~nan], ref[~nan]), f"decode mismatch dt={dt}"


def pin_round_f16(o):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.integers(-30, 18, 20000)),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0**-24, 2.0**-25,
                  2.0**-25 * 1.5, 1.0 + 2.0**-11, 1.0 + 3 * 2.0**-11]),
    ])
    mine = o.round_f16(x)
    ref = x.astype(np.float16).view(np.uint16)  # numpy rounds double -> half directly
    assert np.array_equal(mine, ref), "f16 rounding differs from numpy's RNE cast"


def pin_round_bf16(o):
    # exact ties and a case where going through float32 first would double-round
    one = 1.0
    cases = {
        one + 2.0**-8: 0x3F80,                 # halfway 1 .. 1+2^-7 -> even (1.0)
        one + 3 * 2.0**-8: 0x3F82,             # halfway 1+2^-7 .. 1+2^-6 -> even
        one + 2.0**-8 + 2.0**-40: 0x3F81,      # just above halfway -> up
        -(one + 2.0**-8 + 2.0**-40): 0xBF81,
        0.0: 0x0000,
        3.0e38: 0x7F62,                        # 3e38 = 1.7634 * 2^127 -> 0x7F62
        3.4e38: 0x7F80,                        # rounds past the largest finite -> inf
    }
    for x, want in cases.items():
        got = o._L.or_double_to_bf16(x)
        assert got == want, f"bf16({x!r}) = {got:#06x}, want {want:#06x}"
    # property: result is the nearest bf16, ties to even, on random doubles
    rng = np.random.default_rng(11)
    x = rng.standard_normal(5000) * np.exp2(rng.integers(-20, 20, 5000))
    b = o.round_bf16(x)
    v = np_decode(b, BF16)
    up = np_decode((b.astype(np.int64) + 1).astype(np.uint16), BF16)
    dn = np_decode((b.astype(np.int64) - 1).astype(np.uint16), BF16)
    err = np.abs(v - x)
    assert np.all(err <= np.abs(up - x)) and np.all(err <= np.abs(dn - x))
    tie = (err == np.abs(up - x)) | (err == np.abs(dn - x))
    assert np.all((b[tie] & 1) == 0)


# ---------------------------------------------------------------------------
# O1 GEMM
# ---------------------------------------------------------------------------

def pin_gemm_numpy(o):
    for (M, N, K), dt in itertools.product([(1, 1, 1), (3, 5, 7), (33, 17, 129), (64, 40, 48)],
                                           (F16, BF16)):
        A, B = wl.gemm_inputs(M, N, K, dt, seed=M * 1000 + N * 10 + K)
        C = o.gemm(dt, A, B)
        ref = np_decode(A, dt) @ np_decode(B, dt)
        assert _rel(C, ref) <= 1e-12, (M, N, K, dt)


def pin_gemm_identity(o):
    A = wl.normal_bits((24, 16), 5, F16)
    eye = _bits(np.eye(16), F16)
    C = o.gemm(F16, A, eye)
    assert np.array_equal(C, np_decode(A, F16))


def pin_gemm_bruteforce(o):
    A = wl.normal_bits((3, 4), 21, BF16)
    B = wl.normal_bits((4, 5), 22, BF16)
    a = np_decode(A, BF16).tolist()
    b = np_decode(B, BF16).tolist()
    C = o.gemm(BF16, A, B)
    for i in range(3):
        for j in range(5):
            s = 0.0
            for k in range(4):
                s += a[i][k] * b[k][j]
            assert abs(C[i, j] - s) <= 1e-14 * max(1.0, abs(s))


def pin_gemm_entries(o):
    A, B = wl.gemm_inputs(40, 24, 72, F16, seed=3)
    full = o.gemm(F16, A, B)
    rows = np.array([0, 39, 17, 5])
    cols = np.array([0, 23, 11, 7])
    got = o.gemm_entries(F16, A, B, rows, cols)
    assert np.allclose(got, full[rows, cols], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# O2 AllGather-GEMM
# ---------------------------------------------------------------------------

def pin_ag_concat(o):
    chunks, W, order = wl.ag_inputs(4, 8, 24, 32, F16, seed=31, arrival="random")
    C = o.ag_gemm(F16, list(chunks), W, arrival=order)
    X = np.concatenate([np_decode(c, F16) for c in chunks], axis=0)
    assert _rel(C, X @ np_decode(W, F16)) <= 1e-12


def pin_ag_arrival_invariance(o):
    chunks, W, _ = wl.ag_inputs(4, 4, 16, 16, BF16, seed=32)
    base = o.ag_gemm(BF16, list(chunks), W, arrival=[0, 1, 2, 3])
    for perm in itertools.permutations(range(4)):
        got = o.ag_gemm(BF16, list(chunks), W, arrival=list(perm))
        assert np.array_equal(got, base), perm


# ---------------------------------------------------------------------------
# O3 GEMM-ReduceScatter
# ---------------------------------------------------------------------------

def pin_rs_sum_of_slices(o):
    A, W, seeds = wl.rs_inputs(32, 24, 40, 4, F16, seed=41)
    dst = o.gemm_rs(F16, A, W, list(seeds))
    delta = np.concatenate([d - s.astype(np.float64) for d, s in zip(dst, seeds)], axis=0)
    full = np_decode(A, F16) @ np_decode(W, F16)
    assert np.abs(delta - full).max() <= 1e-12


def pin_rs_split_k_bruteforce(o):
    P = 4
    A, W, seeds = wl.rs_inputs(8, 6, 12, P, BF16, seed=42)
    dst = o.gemm_rs(BF16, A, W, list(seeds))
    a = np_decode(A, BF16)
    w = np_decode(W, BF16)
    Ks = 12 // P
    # P emulated ranks, each holding a contiguous K shard; slice r gets the sum of
    # every rank's partial for its rows.
    for r in range(P):
        rows = slice(r * 2, (r + 1) * 2)
        total = np.zeros((2, 6))
        for p in range(P):
            ks = slice(p * Ks, (p + 1) * Ks)
            total += a[rows, ks] @ w[ks, :]
        assert np.abs(dst[r] - seeds[r] - total).max() <= 1e-12, r


def pin_rs_single_rank_is_gemm(o):
    A, W, seeds = wl.rs_inputs(16, 8, 24, 1, F16, seed=43)
    zero = np.zeros_like(seeds)
    dst = o.gemm_rs(F16, A, W, list(zero))
    assert np.array_equal(dst[0], o.gemm(F16, A, W))


# ---------------------------------------------------------------------------
# O4 routing index
# ---------------------------------------------------------------------------

def _np_route(ids, e0, n_local):
    flat = ids.reshape(-1).astype(np.int64)
    local = (flat >= e0) & (flat < e0 + n_local)
    le = flat - e0
    counts = np.bincount(le[local], minlength=n_local)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pids = np.nonzero(local)[0]
    order = np.argsort(le[pids], kind="stable")
    return offsets, pids[order].astype(np.int32)


def pin_route_numpy(o):
    rng = np.random.default_rng(51)
    for T, E, k, e0, nl in [(100, 16, 2, 4, 4), (257, 64, 2, 0, 8), (64, 8, 1, 0, 8),
                            (33, 64, 4, 56, 8), (50, 16, 2, 12, 4)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        off, sp = o.moe_route(ids, e0, nl)
        roff, rsp = _np_route(ids, e0, nl)
        assert np.array_equal(off, roff) and np.array_equal(sp, rsp), (T, E, k, e0, nl)


def pin_route_edges(o):
    ids = np.full((10, 2), 3, dtype=np.int32)
    ids[:, 1] = 5
    off, sp = o.moe_route(ids, 8, 8)                 # nothing local
    assert np.array_equal(off, np.zeros(9, np.int32)) and sp.size == 0
    off, sp = o.moe_route(ids, 0, 8)                 # everything local
    assert off[-1] == 20 and np.array_equal(sp[:10], np.arange(0, 20, 2))


def pin_route_routing_workload(o):
    ids, _ = wl.moe_routing(2048, 64, 2, seed=52)
    for r in range(8):
        off, sp = o.moe_route(ids, 8 * r, 8)
        roff, rsp = _np_route(ids, 8 * r, 8)
        assert np.array_equal(off, roff) and np.array_equal(sp, rsp)


# ---------------------------------------------------------------------------
# O5 / O6 MoE layers
# ---------------------------------------------------------------------------

def _tiny_moe(seed=61, T=40, hidden=16, ffn=8, E=8, nl=4, e0=2, topk=2, dt=BF16):
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, topk, dt, seed=seed, zipf_s=0.5)
    return inp, e0, nl, topk, dt


def pin_moe_layer0_bruteforce(o):
    inp, e0, nl, topk, dt = _tiny_moe()
    off, sp = o.moe_route(inp["topk_ids"], e0, nl)
    H = o.moe_layer0(dt, inp["X"], inp["W1"], sp, off, topk)
    x = np_decode(inp["X"], dt)
    w1 = np_decode(inp["W1"], dt)
    assert H.shape[0] == off[-1] > 0
    for e in range(nl):
        for r in range(off[e], off[e + 1]):
            t = sp[r] // topk
            assert np.abs(H[r] - x[t] @ w1[e]).max() <= 1e-12
    rows = np.array([0, H.shape[0] - 1, H.shape[0] // 2])
    part = o.moe_layer0_rows(dt, inp["X"], inp["W1"], sp, off, topk, rows)
    assert np.array_equal(part, H[rows])


def pin_moe_ag_layer0_gather(o):
    """Layer 0 behind a token AllGather: 4 chunks of 6 tokens arriving in
    every order.  Brute force on the concatenated tokens (numpy decode and
    fp64 dot products) fixes the placement by chunk index and the gather."""
    inp, e0, nl, topk, dt = _tiny_moe(seed=71)
    T = inp["X"].shape[0]
    n = 4
    assert T % n == 0
    chunks = [inp["X"][c * (T // n):(c + 1) * (T // n)] for c in range(n)]
    off, sp = o.moe_route(inp["topk_ids"], e0, nl)
    x = np_decode(inp["X"], dt)
    w1 = np_decode(inp["W1"], dt)
    ref = np.zeros((int(off[-1]), w1.shape[2]))
    for e in range(nl):
        for r in range(off[e], off[e + 1]):
            ref[r] = x[sp[r] // topk] @ w1[e]
    for perm in itertools.permutations(range(n)):
        H = o.moe_ag_layer0(dt, chunks, inp["W1"], sp, off, topk, arrival=list(perm))
        assert np.abs(H - ref).max() <= 1e-12, perm


def pin_moe_layer0_onehot_is_gemm(o):
    T, hidden, ffn = 24, 16, 8
    X = wl.normal_bits((T, hidden), 62, BF16)
    W1 = wl.normal_bits((1, hidden, ffn), 63, BF16)
    ids = np.zeros((T, 1), dtype=np.int32)
    off, sp = o.moe_route(ids, 0, 1)
    H = o.moe_layer0(BF16, X, W1, sp, off, 1)
    assert np.array_equal(H, o.gemm(BF16, X, W1[0]))


# -- O5a activation (closed forms and identities) ---------------------------

_ACT_X = np.concatenate([np.linspace(-8.0, 8.0, 3201), [0.0, -0.0, 1e-300, -1e-300, 40.0, -40.0]])


def pin_act_none(o):
    assert np.array_equal(o.activation(0, _ACT_X), _ACT_X)


def pin_act_relu(o):
    y, yn = o.activation(1, _ACT_X), o.activation(1, -_ACT_X)
    assert (y >= 0).all()
    assert np.array_equal(y - yn, _ACT_X)          # relu(x) - relu(-x) = x
    assert (y * yn == 0).all()                     # one of the two is zero


def pin_act_gelu(o):
    import math
    y, yn = o.activation(2, _ACT_X), o.activation(2, -_ACT_X)
    # odd part: g(x) - g(-x) = x, since tanh is odd (checks the 1/2 factor)
    assert np.abs((y - yn) - _ACT_X).max() <= 1e-12
    # the tanh form approximates the exact GELU x * Phi(x) (Phi the normal CDF,
    # through math.erf) to within a few 1e-4: a wrong constant breaks this
    exact = np.array([x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) for x in _ACT_X])
    assert np.abs(y - exact).max() <= 1e-3
    assert o.activation(2, np.array([0.0]))[0] == 0.0


def pin_act_silu(o):
    import math
    ln3 = math.log(3.0)
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 exactly
    y = o.activation(3, np.array([ln3, -ln3, 0.0]))
    assert abs(y[0] - 0.75 * ln3) <= 1e-15 and abs(y[1] + 0.25 * ln3) <= 1e-15 and y[2] == 0.0
    d = o.activation(3, _ACT_X) - o.activation(3, -_ACT_X)
    assert np.abs(d - _ACT_X).max() <= 1e-12      # x*s(x) + x*s(-x) = x


def pin_moe_layer1_token_loop(o):
    inp, e0, nl, topk, dt = _tiny_moe(seed=64)
    off, sp = o.moe_route(inp["topk_ids"], e0, nl)
    Hb = o.round_bf16(o.moe_layer0(dt, inp["X"], inp["W1"], sp, off, topk))
    out = o.moe_layer1(dt, Hb, inp["W2"], inp["topk_ids"], inp["topk_weights"], sp, off,
                       inp["out_seed"], e0)
    h = np_decode(Hb, dt)
    w2 = np_decode(inp["W2"], dt)
    ids, wts = inp["topk_ids"], inp["topk_weights"]
    T = ids.shape[0]
    pos = {int(p): r for r, p in enumerate(sp)}
    ref = inp["out_seed"].astype(np.float64).copy()
    for t in range(T):
        for k in range(topk):
            e = int(ids[t, k]) - e0
            if 0 <= e < nl:
                ref[t] += float(wts[t, k]) * (h[pos[t * topk + k]] @ w2[e])
    assert np.abs(out - ref).max() <= 1e-12
    toks = np.array([0, T - 1, 7])
    part = o.moe_layer1_tokens(dt, Hb, inp["W2"], ids, wts, sp, off, inp["out_seed"], e0, toks)
    assert np.array_equal(part, out[toks])


def pin_moe_identical_experts_chain(o):
    # all experts identical and local -> out = seed + (sum_k w) * (round(X W1) W2)
    T, hidden, ffn, E, topk = 32, 16, 8, 4, 2
    inp = wl.moe_inputs(T, hidden, ffn, E, E, topk, BF16, seed=65)
    W1 = np.repeat(inp["W1"][:1], E, axis=0)
    W2 = np.repeat(inp["W2"][:1], E, axis=0)
    off, sp = o.moe_route(inp["topk_ids"], 0, E)
    Hb = o.round_bf16(o.moe_layer0(BF16, inp["X"], W1, sp, off, topk))
    out = o.moe_layer1(BF16, Hb, W2, inp["topk_ids"], inp["topk_weights"], sp, off,
                       inp["out_seed"], 0)
    xw1 = o.round_bf16(np_decode(inp["X"], BF16) @ np_decode(W1[0], BF16))
    chain = np_decode(xw1, BF16) @ np_decode(W2[0], BF16)
    wsum = inp["topk_weights"].astype(np.float64).sum(axis=1, keepdims=True)
    ref = inp["out_seed"].astype(np.float64) + wsum * chain
    assert np.abs(out - ref).max() <= 1e-10


def pin_moe_ep_ranks_sum(o):
    # EP: the sum over ranks of each rank's local combine equals the all-expert combine
    T, hidden, ffn, E, topk = 48, 16, 8, 8, 2
    inp = wl.moe_inputs(T, hidden, ffn, E, E, topk, BF16, seed=66, zipf_s=1.2)
    zero = np.zeros_like(inp["out_seed"])
    off, sp = o.moe_route(inp["topk_ids"], 0, E)
    Hb = o.round_bf16(o.moe_layer0(BF16, inp["X"], inp["W1"], sp, off, topk))
    full = o.moe_layer1(BF16, Hb, inp["W2"], inp["topk_ids"], inp["topk_weights"], sp, off,
                        zero, 0)
    acc = np.zeros_like(full)
    for r in range(4):
        e0, nl = 2 * r, 2
        off_r, sp_r = o.moe_route(inp["topk_ids"], e0, nl)
        H_r = o.round_bf16(o.moe_layer0(BF16, inp["X"], inp["W1"][e0:e0 + nl], sp_r, off_r, topk))
        acc += o.moe_layer1(BF16, H_r, inp["W2"][e0:e0 + nl], inp["topk_ids"],
                            inp["topk_weights"], sp_r, off_r, zero, e0)
    assert np.abs(acc - full).max() <= 1e-10


# ---------------------------------------------------------------------------
# hand-worked fixtures (tests/golden)
# ---------------------------------------------------------------------------

def pin_golden_mlp(o):
    g = _load_golden("tiny_mlp_handworked.json")
    for dt in (F16, BF16):
        ag = g["ag_gemm"]
        chunks = [_bits(c, dt) for c in ag["chunks"]]
        C = o.ag_gemm(dt, chunks, _bits(ag["W"], dt), arrival=ag["arrival"])
        assert np.array_equal(C, np.asarray(ag["expected"], dtype=np.float64))
        rs = g["gemm_rs"]
        seeds = [np.asarray(s, dtype=np.float32) for s in rs["seeds"]]
        dst = o.gemm_rs(dt, _bits(rs["A"], dt), _bits(rs["W"], dt), seeds)
        for d, want in zip(dst, rs["expected"]):
            assert np.array_equal(d, np.asarray(want, dtype=np.float64))
    e = g["ect"]
    assert abs(o.ect(e["overall_time_us"], e["gemm_non_split_us"]) - e["expected_ect_us"]) < 1e-12


def pin_golden_moe(o):
    g = _load_golden("moe_handworked.json")
    ids = np.asarray(g["topk_ids"], dtype=np.int32)
    wts = np.asarray(g["topk_weights"], dtype=np.float32)
    off, sp = o.moe_route(ids, 2, 2)
    assert off.tolist() == g["expected_offsets"] and sp.tolist() == g["expected_sorted_pairs"]
    X = _bits(g["X"], BF16)
    W1 = _bits(g["W1"], BF16)
    W2 = _bits(g["W2"], BF16)
    H = o.moe_layer0(BF16, X, W1, sp, off, 2)
    assert np.array_equal(H, np.asarray(g["expected_H"], dtype=np.float64))
    out = o.moe_layer1(BF16, o.round_bf16(H), W2, ids, wts, sp, off,
                       np.asarray(g["seed"], dtype=np.float32), 2)
    assert np.array_equal(out, np.asarray(g["expected_out"], dtype=np.float64))



# ---------------------------------------------------------------------------
# every-element forms (oracle/full.py): C loops, brute force, fixtures
# ---------------------------------------------------------------------------

def pin_full_decode_exhaustive(o):
    from oracle import full
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt in (F16, BF16):
        mine = full.decode(dt, allbits)
        ref = o.decode(dt, allbits)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(mine), nan)
        assert np.array_equal(mine[~nan], ref[~nan])
        assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def pin_full_dense_vs_loops(o):
    from oracle import full
    for (M, N, K), dt in itertools.product([(1, 1, 1), (3, 5, 7), (33, 17, 129), (64, 40, 48)],
                                           (F16, BF16)):
        A, B = wl.gemm_inputs(M, N, K, dt, seed=M * 1000 + N * 10 + K + 7)
        assert _rel(full.gemm(dt, A, B), o.gemm(dt, A, B)) <= 1e-12, (M, N, K, dt)
    chunks, W, order = wl.ag_inputs(4, 8, 24, 32, BF16, seed=33, arrival="random")
    assert _rel(full.ag_gemm(BF16, list(chunks), W),
                o.ag_gemm(BF16, list(chunks), W, arrival=order)) <= 1e-12
    A, W, seeds = wl.rs_inputs(32, 24, 40, 4, F16, seed=44)
    for got, ref in zip(full.gemm_rs(F16, A, W, list(seeds)), o.gemm_rs(F16, A, W, list(seeds))):
        assert np.abs(got - ref).max() <= 1e-12


def pin_full_dense_bruteforce(o):
    from oracle import full
    A = wl.normal_bits((3, 4), 23, F16)
    B = wl.normal_bits((4, 5), 24, F16)
    a = np_decode(A, F16).tolist()
    b = np_decode(B, F16).tolist()
    C = full.gemm(F16, A, B)
    for i in range(3):
        for j in range(5):
            s = sum(a[i][k] * b[k][j] for k in range(4))
            assert abs(C[i, j] - s) <= 1e-14 * max(1.0, abs(s))
    # two ranks' slices, each seeded, on a K that does not divide evenly
    A2 = wl.normal_bits((4, 3), 25, BF16)
    W2 = wl.normal_bits((3, 2), 26, BF16)
    seeds = [np.full((2, 2), 1.5, np.float32), np.full((2, 2), -2.0, np.float32)]
    a2, w2 = np_decode(A2, BF16), np_decode(W2, BF16)
    dst = full.gemm_rs(BF16, A2, W2, seeds)
    for r in range(2):
        for i in range(2):
            for j in range(2):
                s = float(seeds[r][i, j]) + sum(a2[2 * r + i, k] * w2[k, j] for k in range(3))
                assert abs(dst[r][i, j] - s) <= 1e-14 * max(1.0, abs(s))


def pin_full_moe_bruteforce(o):
    from oracle import full
    for seed, topk, dt in [(67, 2, BF16), (68, 3, F16)]:
        inp, e0, nl, _, _ = _tiny_moe(seed=seed, topk=topk, dt=dt)
        off, sp = o.moe_route(inp["topk_ids"], e0, nl)
        H = full.moe_layer0(dt, inp["X"], inp["W1"], sp, off, topk)
        x = np_decode(inp["X"], dt)
        w1 = np_decode(inp["W1"], dt)
        assert H.shape == (int(off[-1]), w1.shape[2]) and H.shape[0] > 0
        for e in range(nl):
            for r in range(off[e], off[e + 1]):
                assert np.abs(H[r] - x[sp[r] // topk] @ w1[e]).max() <= 1e-12
        assert np.abs(H - o.moe_layer0(dt, inp["X"], inp["W1"], sp, off, topk)).max() <= 1e-12
        Hb = o.round_bf16(H) if dt == BF16 else o.round_f16(H)
        ids, wts = inp["topk_ids"], inp["topk_weights"]
        out = full.moe_layer1(dt, Hb, inp["W2"], ids, wts, sp, off, inp["out_seed"], e0)
        h = np_decode(Hb, dt)
        w2 = np_decode(inp["W2"], dt)
        pos = {int(p): r for r, p in enumerate(sp)}
        ref = inp["out_seed"].astype(np.float64).copy()
        for t in range(ids.shape[0]):
            for k in range(topk):
                e = int(ids[t, k]) - e0
                if 0 <= e < nl:
                    ref[t] += float(wts[t, k]) * (h[pos[t * topk + k]] @ w2[e])
        assert np.abs(out - ref).max() <= 1e-12
        assert np.abs(out - o.moe_layer1(dt, Hb, inp["W2"], ids, wts, sp, off, inp["out_seed"],
                                         e0)).max() <= 1e-12


def pin_full_moe_nothing_local(o):
    from oracle import full
    inp, _, nl, topk, dt = _tiny_moe(seed=69)
    e0 = 64                                   # no expert id reaches this range
    off, sp = o.moe_route(inp["topk_ids"], e0, nl)
    H = full.moe_layer0(dt, inp["X"], inp["W1"], sp, off, topk)
    assert H.shape == (0, inp["W1"].shape[2])
    out = full.moe_layer1(dt, np.zeros((0, H.shape[1]), np.uint16), inp["W2"], inp["topk_ids"],
                          inp["topk_weights"], sp, off, inp["out_seed"], e0)
    assert np.array_equal(out, inp["out_seed"].astype(np.float64))


def pin_full_golden(o):
    from oracle import full
    g = _load_golden("tiny_mlp_handworked.json")
    for dt in (F16, BF16):
        ag = g["ag_gemm"]
        C = full.ag_gemm(dt, [_bits(c, dt) for c in ag["chunks"]], _bits(ag["W"], dt))
        assert np.array_equal(C, np.asarray(ag["expected"], dtype=np.float64))
        rs = g["gemm_rs"]
        seeds = [np.asarray(s, dtype=np.float32) for s in rs["seeds"]]
        dst = full.gemm_rs(dt, _bits(rs["A"], dt), _bits(rs["W"], dt), seeds)
        for d, want in zip(dst, rs["expected"]):
            assert np.array_equal(d, np.asarray(want, dtype=np.float64))
    m = _load_golden("moe_handworked.json")
    ids = np.asarray(m["topk_ids"], dtype=np.int32)
    wts = np.asarray(m["topk_weights"], dtype=np.float32)
    off = np.asarray(m["expected_offsets"], dtype=np.int32)
    sp = np.asarray(m["expected_sorted_pairs"], dtype=np.int32)
    H = full.moe_layer0(BF16, _bits(m["X"], BF16), _bits(m["W1"], BF16), sp, off, 2)
    assert np.array_equal(H, np.asarray(m["expected_H"], dtype=np.float64))
    out = full.moe_layer1(BF16, _bits(m["expected_H"], BF16), _bits(m["W2"], BF16), ids, wts, sp,
                          off, np.asarray(m["seed"], dtype=np.float32), 2)
    assert np.array_equal(out, np.asarray(m["expected_out"], dtype=np.float64))

ALL_PINS = [
    pin_decode_exhaustive, pin_round_f16, pin_round_bf16,
    pin_gemm_numpy, pin_gemm_identity, pin_gemm_bruteforce, pin_gemm_entries,
    pin_ag_concat, pin_ag_arrival_invariance,
    pin_rs_sum_of_slices, pin_rs_split_k_bruteforce, pin_rs_single_rank_is_gemm,
    pin_route_numpy, pin_route_edges, pin_route_routing_workload,
    pin_moe_layer0_bruteforce, pin_moe_ag_layer0_gather, pin_moe_layer0_onehot_is_gemm,
    pin_act_none, pin_act_relu, pin_act_gelu, pin_act_silu,
    pin_moe_layer1_token_loop,
    pin_moe_identical_experts_chain, pin_moe_ep_ranks_sum,
    pin_golden_mlp, pin_golden_moe,
    pin_full_decode_exhaustive, pin_full_dense_vs_loops, pin_full_dense_bruteforce,
    pin_full_moe_bruteforce, pin_full_moe_nothing_local, pin_full_golden,
]
