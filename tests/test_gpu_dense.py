"""GPU parity of the dense operators (fm_gemm, fm_ag_gemm, fm_gemm_rs) against
the CPU oracle, through the C ABI, on seeded inputs: small shapes spanning
several tiles with ragged tails and the edge cases, then the full-size TP=8
rank-0 workloads on every output element (the oracle's every-element forms)
and on sampled outputs of the oracle's loops."""
import numpy as np
import pytest

import workloads as wl
from oracle import full
from gpu_util import (BF16, F16, Arrival, assert_close, bits16, dev16, devf32, host64, say,
                      sample_coords)

pytestmark = pytest.mark.gpu

# FM_TILE forms: BMxBN[wNW] (4 or 8 waves; 4 when omitted).
TILES = ["256x128", "128x128", "256x256", "256x256w8", "256x128w8"]


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _at(C, rows, cols):
    import torch
    r = torch.from_numpy(rows).to(C.device)
    c = torch.from_numpy(cols).to(C.device)
    return C[r, c].float().cpu().numpy().astype(np.float64)


def _gemm(A_bits, B_bits, dt, out32=False):
    import torch
    import tile_gemm_communication_amd as fm
    M, K = A_bits.shape
    N = B_bits.shape[1]
    C = torch.empty((M, N), dtype=torch.float32 if out32 else
                    (torch.float16 if dt == F16 else torch.bfloat16), device="cuda:0")
    fm.fm_gemm(dev16(A_bits, dt), dev16(B_bits, dt), C)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("shape", [(256, 512, 512), (200, 136, 72), (1, 8, 8), (300, 264, 1000),
                                   (513, 392, 200), (64, 1024, 64)])
@pytest.mark.parametrize("dt", [F16, BF16])
def test_gemm_small(oracle, monkeypatch, tile, shape, dt):
    monkeypatch.setenv("FM_TILE", tile)
    monkeypatch.setenv("FM_SPLIT_TAIL", "0")
    M, N, K = shape
    say(f"fm_gemm {M}x{N}x{K} dt={dt} tile={tile}")
    A, B = wl.gemm_inputs(M, N, K, dt, seed=M + N + K)
    C = _gemm(A, B, dt)
    assert_close(host64(C), oracle.gemm(dt, A, B), f"gemm {shape}")


@pytest.mark.parametrize("dt", [F16, BF16])
def test_gemm_fp32_out(oracle, dt):
    A, B = wl.gemm_inputs(320, 264, 328, dt, seed=9)
    C = _gemm(A, B, dt, out32=True)
    ref = oracle.gemm(dt, A, B)
    # fp32 output: only accumulation error remains
    assert_close(host64(C), ref, "gemm fp32 out", max_abs=1e-4, rel_fro=1e-5)


def test_gemm_k_zero_and_m_zero():
    import torch
    import tile_gemm_communication_amd as fm
    A = torch.empty((64, 0), dtype=torch.float16, device="cuda:0")
    B = torch.empty((0, 128), dtype=torch.float16, device="cuda:0")
    C = torch.full((64, 128), 7.0, dtype=torch.float16, device="cuda:0")
    # a zero-length reduction: pass real (aligned) pointers
    A2 = torch.zeros(16, dtype=torch.float16, device="cuda:0")
    fm.lib().fm_gemm(0, 0, 64, 128, 0, A2.data_ptr(), A2.data_ptr(), C.data_ptr(), None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C).item() == 0
    C2 = torch.full((1, 8), 3.0, dtype=torch.float16, device="cuda:0")
    assert fm.lib().fm_gemm(0, 0, 0, 8, 8, A2.data_ptr(), A2.data_ptr(), C2.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert torch.all(C2 == 3.0)
    del A, B


# ---------------------------------------------------------------------------
# AllGather-GEMM
# ---------------------------------------------------------------------------

def _ag_run(arr, W, N, order, epoch, local=None, delay=0, spin_limit=0, skip=()):
    import torch
    import tile_gemm_communication_amd as fm
    C = torch.empty((arr.X.shape[0], N), dtype=arr.X.dtype, device="cuda:0")
    arr.err.zero_()
    arr.push(order, epoch, delay_cycles=delay, local=local, skip=skip)
    fm.fm_ag_gemm(arr.X, W, C, arr.flags, epoch, arr.n, order=list(order), err_word=arr.err,
                  spin_limit=spin_limit)
    arr.join()
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("tile", TILES)
def test_ag_tiny_random_arrival(oracle, monkeypatch, tile):
    """4 chunks of 64 x 512 fp16 arriving in a seeded random order; each
    256-row tile spans every chunk.  Equal to the oracle, and bit-identical to
    fm_gemm on the gathered buffer."""
    monkeypatch.setenv("FM_TILE", tile)
    monkeypatch.setenv("FM_SPLIT_TAIL", "0")
    c = wl.TINY_AG
    chunks, W, order = wl.ag_inputs(c["n_chunks"], c["Mc"], c["N"], c["K"], F16, seed=c["seed"],
                                    arrival="random")
    say(f"fm_ag_gemm tiny tile={tile} order={order.tolist()}")
    arr = Arrival(chunks, F16, c["K"])
    Wd = dev16(W, F16)
    arr.poison()
    C = _ag_run(arr, Wd, c["N"], order, arr.next_epoch())
    assert arr.err.item() == 0
    assert_close(host64(C), oracle.ag_gemm(F16, list(chunks), W, arrival=order), "ag tiny")
    ref = _gemm(bits16(arr.X), W, F16)
    assert np.array_equal(bits16(C), bits16(ref)), "fm_ag_gemm differs from fm_gemm bitwise"


def test_ag_arrival_order_invariance():
    """Results are bit-identical for every arrival order (and order hint)."""
    import itertools
    chunks, W, _ = wl.ag_inputs(4, 64, 256, 192, BF16, seed=111)
    arr = Arrival(chunks, BF16, 192)
    Wd = dev16(W, BF16)
    first = None
    for perm in list(itertools.permutations(range(4)))[::5]:
        arr.poison()
        C = _ag_run(arr, Wd, 256, perm, arr.next_epoch())
        assert arr.err.item() == 0
        b = bits16(C)
        if first is None:
            first = b
        assert np.array_equal(b, first), perm


@pytest.mark.parametrize("n_chunks,Mc", [(1, 300), (8, 64), (3, 512), (16, 32), (64, 16)])
def test_ag_chunk_layouts(oracle, n_chunks, Mc):
    """Chunks smaller, equal and larger than a tile; ragged M."""
    K, N = 136, 264
    chunks, W, order = wl.ag_inputs(n_chunks, Mc, N, K, F16, seed=n_chunks * 7 + Mc,
                                    arrival="random")
    arr = Arrival(chunks, F16, K)
    arr.poison()
    C = _ag_run(arr, dev16(W, F16), N, order, arr.next_epoch())
    assert arr.err.item() == 0
    assert_close(host64(C), oracle.ag_gemm(F16, list(chunks), W, arrival=order), "ag layouts")


# ---------------------------------------------------------------------------
# GEMM-ReduceScatter
# ---------------------------------------------------------------------------

def _rs(A, W, seeds, dt, rank=0, atomic=False):
    import torch
    import tile_gemm_communication_amd as fm
    dst = [devf32(s) for s in seeds]
    fm.fm_gemm_rs(dev16(A, dt), dev16(W, dt), dst, rank=rank, atomic=atomic)
    torch.cuda.synchronize()
    return [d.cpu().numpy().astype(np.float64) for d in dst]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("atomic", [False, True])
@pytest.mark.parametrize("dt", [F16, BF16])
def test_rs_small(oracle, monkeypatch, tile, atomic, dt):
    monkeypatch.setenv("FM_TILE", tile)
    monkeypatch.setenv("FM_SPLIT_TAIL", "0")
    A, W, seeds = wl.rs_inputs(256, 512, 512, 4, dt, seed=401)
    say(f"fm_gemm_rs 256x512x512 P=4 tile={tile} atomic={atomic} dt={dt}")
    got = _rs(A, W, seeds, dt, rank=0, atomic=atomic)
    ref = oracle.gemm_rs(dt, A, W, list(seeds))
    for r in range(4):
        assert_close(got[r] - seeds[r], ref[r] - seeds[r], f"rs slice {r}")


@pytest.mark.parametrize("M,P,rank", [(128, 4, 3), (520, 8, 5), (96, 1, 0), (264, 2, 1),
                                      (1024, 16, 15)])
def test_rs_slices_vs_tiles(oracle, M, P, rank):
    """Slices smaller than a tile (tiles straddle slices), ragged M, P = 1."""
    A, W, seeds = wl.rs_inputs(M, 200, 136, P, F16, seed=M + P)
    got = _rs(A, W, seeds, F16, rank=rank)
    ref = oracle.gemm_rs(F16, A, W, list(seeds))
    for r in range(P):
        assert_close(got[r] - seeds[r], ref[r] - seeds[r], f"rs slice {r}")


@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("M,N,K,P", [(1024, 512, 256, 2), (768, 520, 200, 3)])
def test_rs_full_tiles(oracle, monkeypatch, dt, M, N, K, P):
    """Slices a multiple of the tile height: full 256x256 tiles take the
    epilogue that fetches the slice rows by DMA, the column-edge tile of
    N = 520 the register form; K = 200 runs the K-tail kernel."""
    monkeypatch.setenv("FM_TILE", "256x256")
    monkeypatch.setenv("FM_SPLIT_TAIL", "0")
    say(f"fm_gemm_rs full tiles {M}x{N}x{K} P={P} dt={dt}")
    A, W, seeds = wl.rs_inputs(M, N, K, P, dt, seed=M + N + K)
    got = _rs(A, W, seeds, dt, rank=P - 1)
    ref = oracle.gemm_rs(dt, A, W, list(seeds))
    for r in range(P):
        assert_close(got[r] - seeds[r], ref[r] - seeds[r], f"rs slice {r}")


def test_rs_split_k_emulated_ranks(oracle):
    """P sequential calls with contiguous K shards (the other ranks' partials)
    accumulate into the same slices: seed + the full GEMM."""
    import torch
    import tile_gemm_communication_amd as fm
    P, M, N, K = 4, 256, 256, 512
    A, W, seeds = wl.rs_inputs(M, N, K, P, BF16, seed=77)
    dst = [devf32(s) for s in seeds]
    Ad, Wd = dev16(A, BF16), dev16(W, BF16)
    Ks = K // P
    for p in range(P):
        fm.fm_gemm_rs(Ad[:, p * Ks:(p + 1) * Ks].contiguous(), Wd[p * Ks:(p + 1) * Ks].contiguous(),
                      dst, rank=p)
    torch.cuda.synchronize()
    ref = oracle.gemm_rs(BF16, A, W, list(seeds))
    for r in range(P):
        assert_close(dst[r].cpu().numpy().astype(np.float64) - seeds[r], ref[r] - seeds[r],
                     f"split-K slice {r}")


# ---------------------------------------------------------------------------
# Full-size TP=8 rank-0 workloads (sampled outputs)
# ---------------------------------------------------------------------------

def test_full_dense_gemm(oracle):
    c = wl.DENSE_GEMM
    M, N, K = c["M"], c["N"], c["K"]
    say(f"full fm_gemm {M}x{N}x{K}")
    A, B = wl.gemm_inputs(M, N, K, F16, seed=c["seed"])
    C = _gemm(A, B, F16)
    rows, cols = sample_coords(M, N, 3000, seed=1)
    assert_close(_at(C, rows, cols), oracle.gemm_entries(F16, A, B, rows, cols),
                 "full gemm samples")
    assert_close(host64(C), full.gemm(F16, A, B), "full gemm, every element")



@pytest.mark.parametrize("out32", [False, True])
def test_full_dense_gemm_bf16(out32):
    """The full-size non-split GEMM (4096 x 12288 x 6144) with bf16 inputs,
    C in bf16 or fp32: every element against the oracle's every-element
    form."""
    c = wl.DENSE_GEMM
    M, N, K = c["M"], c["N"], c["K"]
    say(f"full fm_gemm bf16 {M}x{N}x{K} out32={out32}")
    A, B = wl.gemm_inputs(M, N, K, BF16, seed=c["seed"] + 7)
    C = _gemm(A, B, BF16, out32=out32)
    assert_close(host64(C), full.gemm(BF16, A, B), f"full bf16 gemm (fp32 C: {out32})")


@pytest.mark.parametrize("dt", [F16, BF16])
def test_full_ag_gemm(oracle, dt):
    import torch
    c = wl.AG_TP8
    n, Mc, N, K = c["n_chunks"], c["Mc"], c["N"], c["K"]
    say(f"full fm_ag_gemm {n}x{Mc} x {N} x {K} dt={dt}")
    chunks, W, order = wl.ag_inputs(n, Mc, N, K, dt, seed=c["seed"], arrival="ring")
    arr = Arrival(chunks, dt, K)
    Wd = dev16(W, dt)
    arr.poison()
    C = _ag_run(arr, Wd, N, order, arr.next_epoch(), local=0)
    assert arr.err.item() == 0
    X = np.concatenate(list(chunks), axis=0)
    rows, cols = sample_coords(n * Mc, N, 3000, seed=2, tile=(256, 128))
    assert_close(_at(C, rows, cols), oracle.gemm_entries(dt, X, W, rows, cols),
                 "full ag samples")
    assert_close(host64(C), full.ag_gemm(dt, list(chunks), W), "full ag, every element")
    ref = torch.empty_like(C)
    import tile_gemm_communication_amd as fm
    fm.fm_gemm(arr.X, Wd, ref)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), "AG != non-split GEMM bitwise"


@pytest.mark.parametrize("dt", [F16, BF16])
def test_full_gemm_rs(oracle, dt):
    c = wl.RS_TP8
    M, N, K, P = c["M"], c["N"], c["K"], c["n_ranks"]
    say(f"full fm_gemm_rs {M}x{N}x{K} P={P} dt={dt}")
    A, W, seeds = wl.rs_inputs(M, N, K, P, dt, seed=c["seed"])
    got = _rs(A, W, seeds, dt, rank=0)
    rows, cols = sample_coords(M, N, 3000, seed=3)
    ref = oracle.gemm_entries(dt, A, W, rows, cols)
    Ms = M // P
    delta = np.array([got[r // Ms][r % Ms, cc] - seeds[r // Ms][r % Ms, cc]
                      for r, cc in zip(rows, cols)])
    assert_close(delta, ref, "full rs samples")
    for p, want in enumerate(full.gemm_rs(dt, A, W, list(seeds))):
        assert_close(got[p] - seeds[p], want - seeds[p], f"full rs slice {p}, every element")


def _cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("extra_tiles,K", [(None, 128), (7, 200), (-1, 64)])
def test_split_tail_bit_identical(oracle, monkeypatch, extra_tiles, K):
    """A last wave of at most half the CUs runs as 256x128 halves in a second
    launch.  Per output element the K sum is unchanged, so the result equals
    the unsplit schedule bit for bit, and the oracle (every element, and
    sampled against its loops) within the parity bar.
    Shapes: one full wave plus half a wave; one full wave plus 7 tiles (and a
    ragged K); fewer tiles than half the CUs (halves only)."""
    import torch
    G = _cus()
    if extra_tiles is None:
        tiles_m, tiles_n = 6, (G + G // 2) // 6
    elif extra_tiles == -1:
        tiles_m, tiles_n = 2, max(1, G // 8)
    else:
        tiles_m, tiles_n = 1, G + extra_tiles
    # a ragged last column of tiles; with halves only, its right half lies
    # wholly past N
    M, N = 256 * tiles_m, 256 * tiles_n - (192 if extra_tiles == -1 else 8)
    say(f"split tail {M}x{N}x{K} tiles={tiles_m * tiles_n} cus={G}")
    monkeypatch.setenv("FM_TILE", "256x256")
    A, B = wl.gemm_inputs(M, N, K, F16, seed=M + N + K)
    monkeypatch.setenv("FM_SPLIT_TAIL", "1")
    C1 = _gemm(A, B, F16)
    monkeypatch.setenv("FM_SPLIT_TAIL", "0")
    C0 = _gemm(A, B, F16)
    assert torch.equal(C1.view(torch.int16), C0.view(torch.int16)), "split tail changed bits"
    rows, cols = sample_coords(M, N, 2000, seed=5, tile=(256, 128))
    assert_close(_at(C1, rows, cols), oracle.gemm_entries(F16, A, B, rows, cols),
                 "split tail samples")
    assert_close(host64(C1), full.gemm(F16, A, B), "split tail, every element")


def test_more_row_tiles_than_the_ordered_table(oracle):
    """65792 rows: 514 row tiles of the chosen 128-row tile, more than the
    256 entries of the M-tile order table, so the AllGather-GEMM and the
    GEMM-ReduceScatter fall back to the plain row order.  Both element by
    element against the oracle (the AllGather with a reversed arrival)."""
    import torch
    import tile_gemm_communication_amd as fm
    M, N, K, n, P = 65792, 64, 64, 4, 2
    chunks, W, _ = wl.ag_inputs(n, M // n, N, K, F16, seed=65)
    order = list(range(n))[::-1]
    say(f"row tiles beyond the order table: {M}x{N}x{K}")
    arr = Arrival(chunks, F16, K)
    arr.poison()
    C = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    ep = arr.next_epoch()
    arr.push(order, ep)
    fm.fm_ag_gemm(arr.X, dev16(W, F16), C, arr.flags, ep, n, order=order, err_word=arr.err)
    arr.join()
    torch.cuda.synchronize()
    assert arr.err.item() == 0
    X = np.concatenate(list(chunks), axis=0)
    assert_close(host64(C), oracle.gemm(F16, X, W), "ag beyond the order table")
    A, W2, seeds = wl.rs_inputs(M, N, K, P, F16, seed=66)
    dst = [devf32(s) for s in seeds]
    fm.fm_gemm_rs(dev16(A, F16), dev16(W2, F16), dst, rank=1)
    torch.cuda.synchronize()
    ref = oracle.gemm_rs(F16, A, W2, list(seeds))
    for r in range(P):
        assert_close(host64(dst[r]) - seeds[r], ref[r] - seeds[r], f"rs slice {r}")
