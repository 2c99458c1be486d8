"""Helpers for the GPU parity tests: device upload of the seeded 16-bit
inputs, the parity bar, and the emulated chunk arrival (a side stream pushing
chunks with fm_chunk_push)."""
from __future__ import annotations

import sys

import numpy as np

F16, BF16 = 0, 1

# Parity bar for fp16/bf16 inputs with fp32 accumulation: max-abs <= 2e-2 and
# relative Frobenius <= 5e-3 against the fp64 oracle (on the delta for the
# accumulating operators).
MAX_ABS = 2e-2
REL_FRO = 5e-3


def torch_dtype(dt):
    import torch
    return torch.float16 if dt == F16 else torch.bfloat16


def dev16(bits: np.ndarray, dt: int):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits))
    return t.view(torch_dtype(dt)).to("cuda:0")


def devf32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")


def host64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bits16(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_close(got, ref, what="", max_abs=MAX_ABS, rel_fro=REL_FRO):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    if got.size == 0:
        return
    err = np.abs(got - ref).max()
    nrm = np.linalg.norm(ref)
    fro = np.linalg.norm(got - ref) / nrm if nrm > 0 else np.linalg.norm(got - ref)
    assert err <= max_abs and fro <= rel_fro, \
        f"{what}: max-abs {err:.3e} (bar {max_abs}), rel-Frobenius {fro:.3e} (bar {rel_fro})"


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def sample_coords(M: int, N: int, n: int, seed: int, tile=(256, 256)):
    """Random (row, col) samples plus every tile corner along the edges."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, n))
    cols = list(rng.integers(0, N, n))
    edge_r = sorted({0, M - 1} | {min(M - 1, k) for k in range(tile[0] - 1, M, tile[0])}
                    | {min(M - 1, k) for k in range(tile[0], M, tile[0])})
    edge_c = sorted({0, N - 1} | {min(N - 1, k) for k in range(tile[1] - 1, N, tile[1])})
    for r in edge_r[:64]:
        for c in edge_c[:8]:
            rows.append(r)
            cols.append(c)
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


_SIDE = None


def side_stream():
    """The one side stream every test uses for arrivals.  HIP maps streams
    onto a few hardware queues in turn; a test that created a stream per call
    would after a while get one that shares the compute stream's queue, and
    its producer would then run before, not beside, the consumer."""
    global _SIDE
    import torch
    if _SIDE is None:
        _SIDE = torch.cuda.Stream()
    return _SIDE


class Arrival:
    """Emulated AllGather arrival on one GPU: peer chunk buffers in HBM, a side
    stream that pushes chunks into the gathered buffer and publishes flags."""

    _epoch = 0

    def __init__(self, chunks_bits: np.ndarray, dt: int, K: int):
        import torch
        self.n = chunks_bits.shape[0]
        self.Mc = chunks_bits.shape[1]
        self.peers = [dev16(chunks_bits[c], dt) for c in range(self.n)]
        self.X = torch.empty((self.n * self.Mc, K), dtype=torch_dtype(dt), device="cuda:0")
        self.flags = torch.zeros(self.n, dtype=torch.int32, device="cuda:0")
        self.counters = torch.zeros(self.n, dtype=torch.int32, device="cuda:0")
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        self.side = side_stream()

    def next_epoch(self) -> int:
        Arrival._epoch += 1
        return Arrival._epoch

    def poison(self):
        self.X.fill_(float("nan"))

    def push(self, order, epoch, delay_cycles=0, skip=(), local=None, dma=False):
        """Enqueue pushes of chunks in `order` on the side stream (after the
        current stream's work).  `local` is published without a copy (the
        rank's own chunk, already in place); chunks in `skip` never arrive.
        dma: copy on the copy engines (fm_chunk_push_dma) instead of a kernel."""
        import torch
        import tile_gemm_communication_amd as fm
        if local is not None:   # the rank's own chunk is already in place
            self.X[local * self.Mc:(local + 1) * self.Mc].copy_(self.peers[local])
        self.side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.side):
            if delay_cycles:
                torch.cuda._sleep(delay_cycles)
            for c in order:
                c = int(c)
                if c in skip:
                    continue
                rows = slice(c * self.Mc, (c + 1) * self.Mc)
                src, dst = (None, None) if local is not None and c == local else \
                    (self.peers[c], self.X[rows])
                if dma:
                    fm.fm_chunk_push_dma(src, dst, self.flags[c:c + 1], epoch, stream=self.side)
                else:
                    fm.fm_chunk_push(src, dst, self.flags[c:c + 1], self.counters[c:c + 1],
                                     epoch, stream=self.side)

    def join(self):
        import torch
        torch.cuda.current_stream().wait_stream(self.side)
