"""GPU parity of the pull-mode AllGather-GEMM (fm_ag_gemm_pull: every chunk is
read in place from its own buffer) and of the paced signal producer
(fm_chunk_signal_paced), against the CPU oracle and the non-split GEMM."""
import numpy as np
import pytest

import workloads as wl
from oracle import full
from gpu_util import (F16, BF16, assert_close, bits16, dev16, host64, say, sample_coords,
                      side_stream)

pytestmark = pytest.mark.gpu

TILES = ["256x128", "128x128", "256x256", "256x256w8", "256x128w8"]


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Pull:
    """Chunk buffers (each its own allocation, as a peer's mapped buffer), the
    flags, and a side stream that times the signals."""
    _epoch = 1000

    def __init__(self, chunks_bits, dt):
        import torch
        self.n = chunks_bits.shape[0]
        self.chunks = [dev16(chunks_bits[c], dt) for c in range(self.n)]
        self.flags = torch.zeros(self.n, dtype=torch.int32, device="cuda:0")
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        self.side = side_stream()

    def run(self, Wd, N, order, times_ns, hint=None, spin=0, events=None):
        import torch
        import tile_gemm_communication_amd as fm
        Pull._epoch += 1
        epoch = Pull._epoch
        Mc = self.chunks[0].shape[0]
        C = torch.empty((self.n * Mc, N), dtype=Wd.dtype, device="cuda:0")
        self.err.zero_()
        cs = torch.cuda.current_stream()
        self.side.wait_stream(cs)
        if events:
            events[0].record(cs)
        fm.fm_chunk_signal_paced(self.flags, times_ns, epoch, order=list(order), stream=self.side)
        fm.fm_ag_gemm_pull(self.chunks, Wd, C, self.flags, epoch, order=hint,
                           err_word=self.err, spin_limit=spin)
        if events:
            events[1].record(cs)
        cs.wait_stream(self.side)
        torch.cuda.synchronize()
        return C


def _gemm_concat(chunks_bits, Wd, dt):
    import torch
    import tile_gemm_communication_amd as fm
    X = dev16(np.concatenate(list(chunks_bits), axis=0), dt)
    C = torch.empty((X.shape[0], Wd.shape[1]), dtype=Wd.dtype, device="cuda:0")
    fm.fm_gemm(X, Wd, C)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("tile", TILES)
def test_pull_tiny_random_arrival(oracle, monkeypatch, tile):
    """4 chunks of 64 x 512 fp16, signalled in a seeded random order 20 us
    apart.  Each 64-row chunk is its own (partial) row tile.  Equal to the
    oracle and bit-identical to fm_gemm on the concatenated chunks."""
    monkeypatch.setenv("FM_TILE", tile)
    monkeypatch.setenv("FM_SPLIT_TAIL", "0")
    c = wl.TINY_AG
    chunks, W, order = wl.ag_inputs(c["n_chunks"], c["Mc"], c["N"], c["K"], F16, seed=c["seed"],
                                    arrival="random")
    say(f"fm_ag_gemm_pull tiny tile={tile} order={order.tolist()}")
    p = Pull(chunks, F16)
    Wd = dev16(W, F16)
    C = p.run(Wd, c["N"], order, [20_000 * a for a in range(c["n_chunks"])], hint=order)
    assert p.err.item() == 0
    assert_close(host64(C), oracle.ag_gemm(F16, list(chunks), W, arrival=order), "pull tiny")
    assert np.array_equal(bits16(C), bits16(_gemm_concat(chunks, Wd, F16))), \
        "fm_ag_gemm_pull differs from fm_gemm bitwise"


@pytest.mark.parametrize("n_chunks,Mc,dt", [(1, 300, F16), (3, 512, BF16), (5, 200, F16),
                                            (16, 32, BF16), (64, 16, F16)])
def test_pull_chunk_layouts(oracle, n_chunks, Mc, dt):
    """Chunks smaller, equal and larger than a tile, ragged chunk rows and a
    ragged K; every chunk signalled at once."""
    K, N = 136, 264
    chunks, W, order = wl.ag_inputs(n_chunks, Mc, N, K, dt, seed=n_chunks * 11 + Mc,
                                    arrival="random")
    say(f"fm_ag_gemm_pull layout n={n_chunks} Mc={Mc}")
    p = Pull(chunks, dt)
    Wd = dev16(W, dt)
    C = p.run(Wd, N, order, [0] * n_chunks)
    assert p.err.item() == 0
    assert_close(host64(C), oracle.ag_gemm(dt, list(chunks), W, arrival=order), "pull layouts")
    assert np.array_equal(bits16(C), bits16(_gemm_concat(chunks, Wd, dt)))


def test_pull_waits_for_paced_signal():
    """The last chunk is signalled 20 ms after the start: the GEMM cannot end
    before that, and its result is still exact."""
    import torch
    chunks, W, order = wl.ag_inputs(4, 256, 256, 256, F16, seed=77, arrival="ring")
    p = Pull(chunks, F16)
    Wd = dev16(W, F16)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    C = p.run(Wd, 256, order, [0, 0, 0, 20_000_000], events=ev)
    assert p.err.item() == 0
    ms = ev[0].elapsed_time(ev[1])
    say(f"pull GEMM behind a 20 ms signal took {ms:.2f} ms")
    assert ms >= 19.5, ms
    assert np.array_equal(bits16(C), bits16(_gemm_concat(chunks, Wd, F16)))


def test_pull_withheld_signal_times_out():
    """Chunk 3 is never signalled (the paced producer publishes chunks 0..2
    only): the consumers' bounded wait writes FM_ERR_TIMEOUT to err_word and
    the GEMM exits."""
    import torch
    import tile_gemm_communication_amd as fm
    chunks, W, order = wl.ag_inputs(4, 128, 128, 128, F16, seed=78, arrival="ring")
    p = Pull(chunks, F16)
    Pull._epoch += 1
    C = torch.empty((512, 128), dtype=torch.float16, device="cuda:0")
    p.err.zero_()
    cs = torch.cuda.current_stream()
    p.side.wait_stream(cs)
    fm.fm_chunk_signal_paced(p.flags, [0, 0, 0], Pull._epoch, order=[0, 1, 2], stream=p.side)
    fm.fm_ag_gemm_pull(p.chunks, dev16(W, F16), C, p.flags, Pull._epoch, err_word=p.err,
                       spin_limit=2000)
    cs.wait_stream(p.side)
    torch.cuda.synchronize()
    assert p.err.item() == fm.FM_ERR_TIMEOUT


def test_full_pull_ag_gemm_link_paced(oracle):
    """TP=8 rank 0 (8 chunks of 512 x 12288 fp16, W 12288 x 6144), chunks in
    ring order signalled at the one-link rate (12.58 MB at 153 GB/s apart):
    every element against the oracle's every-element form, sampled outputs
    against its loops, and bit-identical to fm_gemm."""
    c = wl.AG_TP8
    n, Mc, N, K = c["n_chunks"], c["Mc"], c["N"], c["K"]
    say(f"full fm_ag_gemm_pull {n}x{Mc} x {N} x {K}, link-paced")
    chunks, W, order = wl.ag_inputs(n, Mc, N, K, F16, seed=c["seed"], arrival="ring")
    p = Pull(chunks, F16)
    Wd = dev16(W, F16)
    step = int(Mc * K * 2 / 153e9 * 1e9)
    C = p.run(Wd, N, order, [a * step for a in range(n)], hint=order)
    assert p.err.item() == 0
    X = np.concatenate(list(chunks), axis=0)
    rows, cols = sample_coords(n * Mc, N, 3000, seed=5, tile=(256, 128))
    import torch
    r = torch.from_numpy(rows).to(C.device)
    cc = torch.from_numpy(cols).to(C.device)
    got = C[r, cc].float().cpu().numpy().astype(np.float64)
    assert_close(got, oracle.gemm_entries(F16, X, W, rows, cols), "full pull samples")
    assert_close(host64(C), full.ag_gemm(F16, list(chunks), W), "full pull, every element")
    assert np.array_equal(bits16(C), bits16(_gemm_concat(chunks, Wd, F16)))



def test_full_pull_ag_gemm_link_parts():
    """TP=8 rank 0 with each 512-row chunk signalled as two 256-row blocks, the
    first once half the chunk has crossed its link (direct schedule: every
    peer's first block at t_link/2, its second at t_link), the tile order
    following that arrival: every element against the oracle's every-element
    form, and bit-identical to fm_gemm on the concatenation."""
    c = wl.AG_TP8
    n, Mc, N, K = c["n_chunks"], c["Mc"], c["N"], c["K"]
    P = 2
    say(f"full fm_ag_gemm_pull {n}x{Mc} x {N} x {K}, {P} link blocks per chunk")
    chunks, W, _ = wl.ag_inputs(n, Mc, N, K, F16, seed=c["seed"], arrival="ring")
    t_link = int(Mc * K * 2 / 153e9 * 1e9)
    times = {ch * P + q: 0 if ch == 0 else (q + 1) * t_link // P
             for ch in range(n) for q in range(P)}
    seq = sorted(times, key=lambda i: (times[i], i))
    p = Pull(chunks.reshape(n * P, Mc // P, K), F16)
    Wd = dev16(W, F16)
    C = p.run(Wd, N, seq, [times[i] for i in seq], hint=seq)
    assert p.err.item() == 0
    assert_close(host64(C), full.ag_gemm(F16, list(chunks), W), "full pull blocks, every element")
    assert np.array_equal(bits16(C), bits16(_gemm_concat(chunks, Wd, F16)))

# ---------------------------------------------------------------------------
# AllGather-GEMM with producer workgroups in the same launch
# ---------------------------------------------------------------------------

def _producers_run(chunks_bits, dt, Wd, N, order, local=(), n_prod=0, counters=None):
    """Sources for every chunk except those in `local` (already in X); returns
    (C, X, flags, counters)."""
    import torch
    import tile_gemm_communication_amd as fm
    n, Mc, K = chunks_bits.shape
    src = [None if c in local else dev16(chunks_bits[c], dt) for c in range(n)]
    X = torch.full((n * Mc, K), float("nan"), dtype=Wd.dtype, device="cuda:0")
    for c in local:
        X[c * Mc:(c + 1) * Mc].copy_(dev16(chunks_bits[c], dt))
    flags = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    if counters is None:
        counters = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    C = torch.empty((n * Mc, N), dtype=Wd.dtype, device="cuda:0")
    Pull._epoch += 1
    fm.fm_ag_gemm_producers(src, X, Wd, C, flags, counters, Pull._epoch, order=list(order),
                            n_producers=n_prod, err_word=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.all(flags == Pull._epoch).item()
    assert torch.count_nonzero(counters).item() == 0
    return C, X


@pytest.mark.parametrize("tile", TILES)
def test_producers_tiny_random_arrival(oracle, monkeypatch, tile):
    """4 chunks of 64 x 512 fp16 copied by 8 producer workgroups in a seeded
    random order: X holds the concatenation afterwards, and C equals the
    oracle and fm_gemm bit for bit."""
    monkeypatch.setenv("FM_TILE", tile)
    c = wl.TINY_AG
    chunks, W, order = wl.ag_inputs(c["n_chunks"], c["Mc"], c["N"], c["K"], F16, seed=c["seed"],
                                    arrival="random")
    say(f"fm_ag_gemm_producers tiny tile={tile} order={order.tolist()}")
    Wd = dev16(W, F16)
    C, X = _producers_run(chunks, F16, Wd, c["N"], order, n_prod=8)
    assert np.array_equal(bits16(X), np.concatenate(list(chunks), axis=0))
    assert_close(host64(C), oracle.ag_gemm(F16, list(chunks), W, arrival=order), "producers")
    assert np.array_equal(bits16(C), bits16(_gemm_concat(chunks, Wd, F16)))


@pytest.mark.parametrize("n_chunks,Mc,dt,n_prod,local", [(1, 300, F16, 8, ()),
                                                         (3, 512, BF16, 16, (0,)),
                                                         (5, 200, F16, 64, (2,)),
                                                         (16, 32, BF16, 24, (0, 1)),
                                                         (8, 64, F16, 8, tuple(range(8)))])
def test_producers_layouts(oracle, n_chunks, Mc, dt, n_prod, local):
    """Chunk sizes around the tile height, a ragged K, local chunks already in
    place (all of them in the last case), and producer counts from 8 to 64."""
    K, N = 136, 264
    chunks, W, order = wl.ag_inputs(n_chunks, Mc, N, K, dt, seed=n_chunks * 13 + Mc,
                                    arrival="random")
    say(f"fm_ag_gemm_producers layout n={n_chunks} Mc={Mc} P={n_prod} local={local}")
    Wd = dev16(W, dt)
    C, X = _producers_run(chunks, dt, Wd, N, order, local=local, n_prod=n_prod)
    assert np.array_equal(bits16(X), np.concatenate(list(chunks), axis=0))
    assert_close(host64(C), oracle.ag_gemm(dt, list(chunks), W, arrival=order), "producers")
    assert np.array_equal(bits16(C), bits16(_gemm_concat(chunks, Wd, dt)))


def test_full_producers_ag_gemm(oracle):
    """TP=8 rank 0 with the default producer count: the local chunk in place,
    seven copied in ring order; every element against the oracle's
    every-element form and sampled outputs against its loops, X and C
    bit-identical to the concatenation and to fm_gemm; a second call with the
    same counters (left at zero) gives the same bits."""
    import torch
    c = wl.AG_TP8
    n, Mc, N, K = c["n_chunks"], c["Mc"], c["N"], c["K"]
    say(f"full fm_ag_gemm_producers {n}x{Mc} x {N} x {K}")
    chunks, W, order = wl.ag_inputs(n, Mc, N, K, F16, seed=c["seed"], arrival="ring")
    Wd = dev16(W, F16)
    counters = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    C, X = _producers_run(chunks, F16, Wd, N, order, local=(0,), counters=counters)
    assert np.array_equal(bits16(X), np.concatenate(list(chunks), axis=0))
    Xh = np.concatenate(list(chunks), axis=0)
    rows, cols = sample_coords(n * Mc, N, 3000, seed=6, tile=(256, 128))
    r = torch.from_numpy(rows).to(C.device)
    cc = torch.from_numpy(cols).to(C.device)
    got = C[r, cc].float().cpu().numpy().astype(np.float64)
    assert_close(got, oracle.gemm_entries(F16, Xh, W, rows, cols), "full producers samples")
    assert_close(host64(C), full.ag_gemm(F16, list(chunks), W), "full producers, every element")
    ref = bits16(_gemm_concat(chunks, Wd, F16))
    assert np.array_equal(bits16(C), ref)
    C2, _ = _producers_run(chunks, F16, Wd, N, order, local=(0,), counters=counters)
    assert np.array_equal(bits16(C2), ref)
