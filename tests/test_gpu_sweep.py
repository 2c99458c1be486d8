"""Seeded random shapes, compared element by element with the oracle (on the
delta out - seed for the accumulating operators): the two read-modify-write
epilogues (the MoE combine and GEMM-ReduceScatter), whose DMA-fed forms count
their memory instructions, and the plain, AllGather and pull-mode GEMMs.
Ragged rows and columns, K tails, every tile form, both 16-bit types, chunk
counts and arrival orders.  The shapes are drawn once from fixed seeds, so
every run checks the same cases."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import BF16, F16, Arrival, assert_close, bits16, dev16, host64, say
from oracle import full
from test_gpu_dense import TILES, _ag_run, _gemm, _rs
from test_gpu_moe import _moe_run
from test_gpu_pull import Pull, _gemm_concat

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261202)


def _m8(lo, hi):
    return int(_rng.integers(lo // 8, hi // 8 + 1)) * 8


MOE_CASES = []
for _ in range(6):
    E = int(_rng.choice([8, 16, 64]))
    nl = int(_rng.integers(1, min(E, 16) + 1))
    MOE_CASES.append(dict(T=int(_rng.integers(64, 3000)), hidden=_m8(8, 1100), ffn=_m8(8, 700),
                          E=E, nl=nl, e0=int(_rng.integers(0, E - nl + 1)),
                          topk=int(_rng.choice([1, 2, 4])), dt=int(_rng.choice([F16, BF16])),
                          tile=str(_rng.choice(["256x256", "256x256w8", "256x128w8",
                                                "128x128"])),
                          seed=int(_rng.integers(1, 10_000))))

RS_CASES = []
for _ in range(6):
    P = int(_rng.choice([1, 2, 4, 8]))
    Ms = int(_rng.choice([256, 512, 100, 264]))
    RS_CASES.append(dict(M=P * Ms, N=_m8(8, 1100), K=_m8(8, 900), P=P,
                         dt=int(_rng.choice([F16, BF16])),
                         tile=str(_rng.choice(["256x256", "256x128", "128x128"])),
                         seed=int(_rng.integers(1, 10_000))))


# a second generator, so the cases above stay as they were
_rng2 = np.random.default_rng(20261203)


def _m8b(lo, hi):
    return int(_rng2.integers(lo // 8, hi // 8 + 1)) * 8


for _ in range(6):
    E = int(_rng2.choice([8, 16, 64]))
    nl = int(_rng2.integers(1, min(E, 16) + 1))
    MOE_CASES.append(dict(T=int(_rng2.integers(16, 4000)), hidden=_m8b(8, 1400),
                          ffn=_m8b(8, 900), E=E, nl=nl, e0=int(_rng2.integers(0, E - nl + 1)),
                          topk=int(_rng2.choice([1, 2, 3, 4])),
                          dt=int(_rng2.choice([F16, BF16])),
                          tile=str(_rng2.choice(["256x256", "256x256w4", "256x256w8",
                                                 "256x128w8", "128x128"])),
                          seed=int(_rng2.integers(1, 10_000))))

for _ in range(4):
    P = int(_rng2.choice([1, 2, 3, 4, 8]))
    Ms = int(_rng2.integers(1, 300))
    RS_CASES.append(dict(M=P * Ms, N=_m8b(8, 1400), K=_m8b(8, 1200), P=P,
                         dt=int(_rng2.choice([F16, BF16])),
                         tile=str(_rng2.choice(["256x256", "256x128", "128x128"])),
                         seed=int(_rng2.integers(1, 10_000))))

GEMM_CASES = [dict(M=int(_rng2.integers(1, 1600)), N=_m8b(8, 2000), K=_m8b(8, 1600),
                   dt=int(_rng2.choice([F16, BF16])), tile=str(_rng2.choice(TILES)),
                   out32=bool(_rng2.random() < 0.3), seed=int(_rng2.integers(1, 10_000)))
              for _ in range(10)]

AG_CASES = []
for _ in range(8):
    n = int(_rng2.integers(1, 9))
    AG_CASES.append(dict(n=n, Mc=int(_rng2.integers(1, 400)), N=_m8b(8, 1400),
                         K=_m8b(8, 1200), dt=int(_rng2.choice([F16, BF16])),
                         tile=str(_rng2.choice(TILES)),
                         order=[int(x) for x in _rng2.permutation(n)],
                         local=bool(_rng2.random() < 0.5), seed=int(_rng2.integers(1, 10_000))))


@pytest.mark.parametrize("c", MOE_CASES, ids=lambda c: "T{T}-h{hidden}-f{ffn}-E{E}-nl{nl}-k{topk}-{tile}".format(**c))
def test_moe_random_shapes(oracle, monkeypatch, c):
    monkeypatch.setenv("FM_MOE_TILE", c["tile"])
    say(f"moe sweep {c}")
    dt = c["dt"]
    inp = wl.moe_inputs(c["T"], c["hidden"], c["ffn"], c["E"], c["nl"], c["topk"], dt,
                        seed=c["seed"], zipf_s=1.2)
    roff, rsp = oracle.moe_route(inp["topk_ids"], c["e0"], c["nl"])
    Href = oracle.moe_layer0(dt, inp["X"], inp["W1"], rsp, roff, c["topk"])
    Hb = oracle.round_bf16(Href) if dt == BF16 else oracle.round_f16(Href)
    rows = int(roff[-1])
    # H at its full capacity of T * topk rows, as the API takes it (the
    # routing may leave no local rows at all)
    Hcap = np.zeros((c["T"] * c["topk"], c["ffn"]), dtype=np.uint16)
    Hcap[:rows] = Hb
    off, sp, H, out = _moe_run(inp, c["e0"], c["nl"], dt, H_in=Hcap)
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    assert_close(host64(H[:rows]), Href, "moe layer0 H")
    ref = oracle.moe_layer1(dt, Hb, inp["W2"], inp["topk_ids"], inp["topk_weights"], rsp, roff,
                            inp["out_seed"], c["e0"])
    assert_close(host64(out) - inp["out_seed"], ref - inp["out_seed"], "moe combine")


@pytest.mark.parametrize("c", RS_CASES, ids=lambda c: "M{M}-N{N}-K{K}-P{P}-{tile}".format(**c))
def test_rs_random_shapes(oracle, monkeypatch, c):
    monkeypatch.setenv("FM_TILE", c["tile"])
    say(f"rs sweep {c}")
    A, W, seeds = wl.rs_inputs(c["M"], c["N"], c["K"], c["P"], c["dt"], seed=c["seed"])
    got = _rs(A, W, seeds, c["dt"], rank=c["P"] - 1)
    ref = oracle.gemm_rs(c["dt"], A, W, list(seeds))
    for r in range(c["P"]):
        assert_close(got[r] - seeds[r], ref[r] - seeds[r], f"rs slice {r}")


@pytest.mark.parametrize("c", GEMM_CASES,
                         ids=lambda c: "M{M}-N{N}-K{K}-{tile}-out32{out32}".format(**c))
def test_gemm_random_shapes(monkeypatch, c):
    monkeypatch.setenv("FM_TILE", c["tile"])
    say(f"gemm sweep {c}")
    A, B = wl.gemm_inputs(c["M"], c["N"], c["K"], c["dt"], seed=c["seed"])
    C = _gemm(A, B, c["dt"], out32=c["out32"])
    assert_close(host64(C), full.gemm(c["dt"], A, B), "gemm")


@pytest.mark.parametrize("c", AG_CASES,
                         ids=lambda c: "n{n}-Mc{Mc}-N{N}-K{K}-{tile}-local{local}".format(**c))
def test_ag_and_pull_random_shapes(monkeypatch, c):
    """The AllGather-GEMM with pushed chunks (the first chunk of the order
    in place when `local`) and the pull form reading the same chunks in
    place, each against the oracle and bit-identical to fm_gemm on the
    concatenation."""
    import torch
    monkeypatch.setenv("FM_TILE", c["tile"])
    say(f"ag/pull sweep {c}")
    dt, n, Mc, N, K = c["dt"], c["n"], c["Mc"], c["N"], c["K"]
    chunks, W, _ = wl.ag_inputs(n, Mc, N, K, dt, seed=c["seed"])
    want = full.ag_gemm(dt, list(chunks), W)
    Wd = dev16(W, dt)
    ref = bits16(_gemm_concat(chunks, Wd, dt))
    arr = Arrival(chunks, dt, K)
    arr.poison()
    C = _ag_run(arr, Wd, N, c["order"], arr.next_epoch(),
                local=c["order"][0] if c["local"] else None)
    assert arr.err.item() == 0
    assert_close(host64(C), want, "ag")
    assert np.array_equal(bits16(C), ref)
    p = Pull(chunks, dt)
    Cp = p.run(Wd, N, c["order"], [20_000 * a for a in range(n)], hint=c["order"])
    assert p.err.item() == 0
    assert_close(host64(Cp), want, "pull")
    assert np.array_equal(bits16(Cp), ref)
    torch.cuda.synchronize()
