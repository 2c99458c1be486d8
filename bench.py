#!/usr/bin/env python3
"""Benchmark of the fused GEMM + tensor/expert-parallel data-movement path on
one MI355X, for one rank's share of a TP=8 / EP=8 layer step.

One step (all on one GPU, inputs resident in HBM):
  1. AllGather-GEMM, dense MLP layer 0 at TP=8: the rank's own 512 x 12288
     chunk is in place; the other seven chunks are pushed into the gathered
     buffer by three side streams, peers round-robin, so that arrivals
     overlap as they do over a full mesh of links (fm_chunk_push, per-chunk
     flags) while
     fm_ag_gemm computes Output1 = X[4096 x 12288] * W1[12288 x 6144] (fp16).
  2. GEMM-ReduceScatter, dense MLP layer 1: Output1 * W2[6144 x 12288] added
     into eight fp32 [512 x 12288] rank slices (fm_gemm_rs).
  3. MoE layer at EP=8, rank 0: 16384 tokens x 4096, 64 experts top-2 with a
     log-Zipf(1.2) router bias, 8 local experts with W1 [4096 x 2816] and
     W2 [2816 x 4096] (bf16): route + gather-GEMM (fm_moe_gather_gemm), then
     GEMM + weighted scatter-reduce (fm_moe_gemm_scatter).

value = algorithmic flops of the whole step / step time, in TFLOP/s.
Also reported: per-operator TFLOP/s and fraction of the 2516.6 TFLOP/s dense
fp16/bf16 MFMA peak, and the effective communication time
ECT = OverallTime - GEMM_non-split (FLUX review, "核心公式") of the fused
AllGather and ReduceScatter operators against the non-split GEMM (this
library's and hipBLASLt's through torch.matmul) and against the naive
chunk-by-chunk launch sequence; the pull forms with link-paced signals, each
chunk signalled as row blocks as they cross the link.  Each comparison is
timed in alternating passes of its variants, so clock drift moves them alike.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2516.6          # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk

# HBM bytes per launch of each step kernel, from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs of `bench.py --steps 2 --warmup 1 --no-ect --no-cpu-baseline
# --serial-arrival` (KiB per dispatch, averaged), scaled by the factors a
# known-size copy (`bench.py --copy-probe 256`) gives: FETCH_SIZE x2.0,
# WRITE_SIZE x1.0.  Keyed by the digest of the kernel sources they were taken
# on: after any change to csrc/ they no longer apply and traffic is null.
TRAFFIC_DIGEST = "5770d0f34cc2c329"
TRAFFIC_BYTES = {             # op name -> (read bytes, written bytes) per call
    "ag_gemm": (1119624959, 50328564),
    "gemm_rs": (1115677704, 201317328),
    "moe_gather_gemm": (1337121233, 172566322),
    "moe_gemm_scatter": (2224136528, 501668013),
}


def source_digest() -> str:
    """sha256 over the library's kernel sources (names and contents)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "tile_gemm_communication_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]
METRIC = "fused AG/RS-GEMM TFLOP/s & % MFMA peak; ECT vs non-split GEMM"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=" ".join(__doc__.split("\n\n")[0].split()))
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ect-iters", type=int, default=20)
    ap.add_argument("--no-ect", action="store_true", help="skip the ECT comparisons")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the one-off cold-cache timing of each op")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of the AllGather-GEMM the CPU oracle computes as its sample")
    ap.add_argument("--serial-arrival", action="store_true",
                    help="let every chunk land before fm_ag_gemm starts (for profilers that "
                         "serialise kernel dispatches, where a concurrent arrival cannot happen)")
    ap.add_argument("--parts", type=int, default=1, choices=(1, 2, 4, 8),
                    help="communication parts per pushed chunk, each with its own flag "
                         "(finer communication tiles)")
    ap.add_argument("--link-parts", type=int, default=2, choices=(1, 2, 4, 8),
                    help="row blocks per chunk in the link-paced pull schedules, each "
                         "signalled once its bytes have crossed the link (2: one 256-row "
                         "tile row of the AllGather-GEMM)")
    ap.add_argument("--moe-link-parts", type=int, default=4, choices=(1, 2, 4, 8),
                    help="token blocks per chunk in the link-paced pull of MoE layer 0")
    ap.add_argument("--arrival", choices=("kernel", "dma"), default="kernel",
                    help="emulated peer push: fm_chunk_push (copy kernel) or "
                         "fm_chunk_push_dma (copy engines, no compute units)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the register-only MFMA loop (fm_probe_mfma) in each form "
                         "and print its TFLOP/s and the shader clock it held")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run fm_chunk_push over MIB MiB three times and exit: the "
                         "known-size copy that calibrates the HBM byte counters")
    return ap.parse_args()


class Workload:
    """Device buffers of the step, filled from the seeded generators."""

    def __init__(self):
        import numpy as np
        import torch

        import workloads as wl
        dev = torch.device("cuda:0")
        self.dev = dev
        ag, rs, moe = wl.AG_TP8, wl.RS_TP8, wl.MOE_EP8
        self.n, self.Mc, self.N1, self.K1 = ag["n_chunks"], ag["Mc"], ag["N"], ag["K"]
        self.M = self.n * self.Mc
        self.N2, self.K2, self.P = rs["N"], rs["K"], rs["n_ranks"]
        assert self.K2 == self.N1 and rs["M"] == self.M
        f16 = torch.float16
        bf16 = torch.bfloat16

        def up(bits, dt):
            return torch.from_numpy(np.ascontiguousarray(bits)).view(dt).to(dev)

        log("generating dense inputs")
        chunks, W1, _ = wl.ag_inputs(self.n, self.Mc, self.N1, self.K1, wl.F16, seed=ag["seed"])
        self.chunks_host = chunks
        self.W1_host = W1
        self.peers = [up(chunks[c], f16) for c in range(self.n)]
        self.X = torch.empty((self.M, self.K1), dtype=f16, device=dev)
        self.X[: self.Mc].copy_(self.peers[0])            # rank 0's own chunk
        self.W1 = up(W1, f16)
        self.Out1 = torch.empty((self.M, self.N1), dtype=f16, device=dev)
        _, W2, seeds = wl.rs_inputs(self.M, self.N2, self.K2, self.P, wl.F16, seed=rs["seed"])
        self.W2 = up(W2, f16)
        self.dst = [torch.from_numpy(seeds[r]).to(dev) for r in range(self.P)]
        # one flag per communication part: each rank's chunk is pushed and
        # published as `parts` row blocks (pull mode and the in-launch
        # producers use the first n flags, one per chunk)
        self.parts = 1
        self.link_parts = 1
        self.moe_link_parts = 1
        self.flags = torch.zeros(self.n * 8, dtype=torch.int32, device=dev)
        self.counters = torch.zeros(self.n * 8, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.epoch = 0

        log("generating MoE inputs")
        self.T, self.hidden, self.ffn = moe["T"], moe["hidden"], moe["ffn"]
        self.n_local, self.topk = moe["n_local"], moe["topk"]
        self.e0 = moe["rank"] * moe["n_local"]
        inp = wl.moe_inputs(self.T, self.hidden, self.ffn, moe["n_experts"], self.n_local,
                            self.topk, wl.BF16, seed=moe["seed"], zipf_s=moe["zipf_s"])
        ids = inp["topk_ids"]
        self.rows_local = int(((ids >= self.e0) & (ids < self.e0 + self.n_local)).sum())
        self.mX = up(inp["X"], bf16)
        self.mW1 = up(inp["W1"], bf16)
        self.mW2 = up(inp["W2"], bf16)
        self.ids = torch.from_numpy(ids).to(dev)
        self.wts = torch.from_numpy(inp["topk_weights"]).to(dev)
        self.mout = torch.from_numpy(inp["out_seed"]).to(dev)
        # token AllGather in front of MoE layer 0: 8 chunks of T/8 tokens, chunk
        # c from peer c (the local chunk 0 already in place)
        self.mTc = self.T // self.n
        self.mpeers = [up(inp["X"][c * self.mTc:(c + 1) * self.mTc], bf16) for c in range(self.n)]
        self.mXg = torch.empty_like(self.mX)
        self.mXg[: self.mTc].copy_(self.mpeers[0])
        self.mflags = torch.zeros(self.n * 8, dtype=torch.int32, device=dev)
        self.mcounters = torch.zeros(self.n * 8, dtype=torch.int32, device=dev)
        self.H = torch.empty((self.T * self.topk, self.ffn), dtype=bf16, device=dev)
        self.sp = torch.empty(self.T * self.topk, dtype=torch.int32, device=dev)
        self.off = torch.zeros(self.n_local + 1, dtype=torch.int32, device=dev)
        import tile_gemm_communication_amd as fm
        self.mws = fm.moe_workspace(self.T, self.topk, self.hidden, self.n_local)

        # three side streams: with the compute stream that is the four hardware
        # queues a process gets by default
        self.sides = [torch.cuda.Stream(device=dev) for _ in range(3)]
        self.serial_arrival = False
        self.arrival = "kernel"
        self.n_sides = len(self.sides)
        self.order = list(range(self.n))                  # local chunk first, then ring order
        self.flop_ag = 2.0 * self.M * self.N1 * self.K1
        self.flop_rs = 2.0 * self.M * self.N2 * self.K2
        self.flop_moe = 2.0 * 2 * self.rows_local * self.hidden * self.ffn
        torch.cuda.synchronize()

    # -- pieces of a step ----------------------------------------------------
    def part_order(self):
        """Arrival order of the communication parts: chunk by chunk in
        self.order, each chunk's parts in row order."""
        return [c * self.parts + q for c in self.order for q in range(self.parts)]

    def push_all(self, epoch, events=None, moe=False):
        """Publish the local chunk and push the seven peer chunks, each as
        self.parts row blocks with a flag of its own, part i of the sequence
        on side stream i % 3.  events: optional per-chunk events recorded
        after each chunk's last part.  moe: the token chunks of MoE layer 0
        instead of the dense AllGather's row chunks."""
        import tile_gemm_communication_amd as fm
        import torch
        peers, X, Mc = (self.mpeers, self.mXg, self.mTc) if moe else (self.peers, self.X, self.Mc)
        flags, counters = (self.mflags, self.mcounters) if moe else (self.flags, self.counters)
        P = self.parts
        rows = Mc // P
        cs = torch.cuda.current_stream()
        for s in self.sides:
            s.wait_stream(cs)
        def push(src, dst, f, s):
            if self.arrival == "dma":
                fm.fm_chunk_push_dma(src, dst, flags[f:f + 1], epoch, stream=s)
            else:
                fm.fm_chunk_push(src, dst, flags[f:f + 1], counters[f:f + 1], epoch, stream=s)
        # the local chunk is in place: its flags are written by the stream
        # itself (no kernel)
        for q in range(P):
            f = self.order[0] * P + q
            fm.fm_chunk_push_dma(None, None, flags[f:f + 1], epoch, stream=self.sides[0])
        i = 0
        for c in self.order[1:]:
            for q in range(P):
                s = self.sides[i % self.n_sides]
                push(peers[c][q * rows:(q + 1) * rows],
                     X[c * Mc + q * rows:c * Mc + (q + 1) * rows], c * P + q, s)
                i += 1
            if events is not None:
                events[c].record(s)

    def join_sides(self):
        import torch
        cs = torch.cuda.current_stream()
        for s in self.sides:
            cs.wait_stream(s)

    def ag(self, epoch):
        import tile_gemm_communication_amd as fm
        n = self.n * self.parts
        fm.fm_ag_gemm(self.X, self.W1, self.Out1, self.flags[:n], epoch, n,
                      order=self.part_order(), err_word=self.err)

    def rs(self):
        import tile_gemm_communication_amd as fm
        fm.fm_gemm_rs(self.Out1, self.W2, self.dst, rank=0)

    def moe0(self):
        import tile_gemm_communication_amd as fm
        fm.fm_moe_gather_gemm(self.mX, self.ids, self.mW1, self.H, self.sp, self.off, self.e0,
                              self.mws)

    def moe0_ag(self, epoch):
        import tile_gemm_communication_amd as fm
        n = self.n * self.parts
        fm.fm_moe_ag_gather_gemm(self.mXg, self.ids, self.mW1, self.H, self.sp, self.off, self.e0,
                                 self.mflags[:n], epoch, n, self.mws, order=self.part_order(),
                                 err_word=self.err)

    def moe1(self):
        import tile_gemm_communication_amd as fm
        fm.fm_moe_gemm_scatter(self.H, self.mW2, self.sp, self.off, self.wts, self.mout, self.mws,
                               err_word=self.err)

    def step(self, evs=None):
        """One full step on the current stream (+ the side streams for arrival).
        evs: optional list of 5 events bracketing AG | RS | MoE0 | MoE1."""
        import torch
        cs = torch.cuda.current_stream()
        self.epoch += 1
        self.push_all(self.epoch)
        if self.serial_arrival:
            self.join_sides()
        if evs: evs[0].record(cs)
        self.ag(self.epoch)
        if evs: evs[1].record(cs)
        # GEMM-RS does not depend on the arrival streams (only the AllGather's
        # tiles wait for their chunks' flags), so the compute stream does not
        # join them here: the next step's pushes wait for the compute stream,
        # and the timed region ends with a device-wide synchronize.
        self.rs()
        if evs: evs[2].record(cs)
        self.moe0()
        if evs: evs[3].record(cs)
        self.moe1()
        if evs: evs[4].record(cs)


LINK_BYTES_PER_S = 153e9   # one MI355X xGMI link, per direction


def check_err(w, what):
    """Stop with the status a kernel wrote to the shared err_word during `what`."""
    import tile_gemm_communication_amd as fm
    code = int(w.err.item())
    if code != 0:
        raise RuntimeError(f"{what}: a kernel reported {fm.status_str(code)}")


def time_rounds(variants, iters, rounds=3, warmup=3):
    """Median over `rounds` passes of each variant's median time (ms).  The
    variants take turns within each pass, so a clock that drifts during the
    run (the chip is power-limited) moves them all alike and the differences
    (ECT) stay fair."""
    per = {name: [] for name, _ in variants}
    for _ in range(rounds):
        for name, fn in variants:
            per[name].append(time_loop(fn, iters, warmup)[0])
    return {name: sorted(v)[len(v) // 2] for name, v in per.items()}


def link_schedule(order, parts, t_link, kind):
    """Arrival times of the chunks' row blocks in the link-paced pull.

    The local chunk (order[0]) is in place at t = 0.  A chunk crosses one
    link in t_link, so its row block q of `parts` has landed (q+1)/parts of
    t_link after its transfer began.  Direct: every peer sends over a link of
    its own, all starting at 0.  Ring: the chunk at ring position a >= 1
    starts at (a-1) * t_link.  Returns the block indices (c * parts + q)
    sorted by arrival and their times in ns."""
    t = {}
    for a, c in enumerate(order):
        start = 0 if kind == "direct" else (a - 1) * t_link
        for q in range(parts):
            t[c * parts + q] = 0 if a == 0 else int(start + (q + 1) * t_link // parts)
    seq = sorted(t, key=lambda i: (t[i], i))
    return seq, [t[i] for i in seq]


def part_views(chunks, parts):
    """Row block q of chunk c at index c * parts + q (views, no copies)."""
    r = chunks[0].shape[0] // parts
    return [x[q * r:(q + 1) * r] for x in chunks for q in range(parts)]


def time_loop(fn, iters, warmup):
    """Median per-iteration time (ms) of fn() on the current stream, with events."""
    import torch
    for _ in range(warmup):
        fn()
    cs = torch.cuda.current_stream()
    times = []
    for _ in range(iters):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(cs)
        fn()
        b.record(cs)
        times.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(x.elapsed_time(y) for x, y in times)
    return ms[len(ms) // 2], ms[0]


def cold_ops(w):
    """Each op of the step once with cold caches: a 512 MiB scratch buffer is
    written before each (more than the 256 MiB Infinity Cache plus the eight
    4 MiB L2s).  The chunks have all landed before the AllGather-GEMM starts,
    so it is timed without arrival."""
    import torch
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cs = torch.cuda.current_stream()
    w.epoch += 1
    w.push_all(w.epoch)
    w.join_sides()
    ops = (("ag_gemm", lambda: w.ag(w.epoch)), ("gemm_rs", w.rs),
           ("moe_gather_gemm", w.moe0), ("moe_gemm_scatter", w.moe1))
    evs = []
    for i, (_, fn) in enumerate(ops):
        scratch.fill_(i + 1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(cs)
        fn()
        b.record(cs)
        evs.append((a, b))
    torch.cuda.synchronize()
    del scratch
    return {n: round(a.elapsed_time(b), 4) for (n, _), (a, b) in zip(ops, evs)}


def moe_baselines(w, iters):
    """The MoE layer (layer 0 + the combine, one call each) against its
    unfused forms on the same inputs and routing: the expert rows gathered
    first (torch index_select), then one fm_gemm per expert and layer and a
    torch index_add_ of the weighted products ("pre-gathered grouped GEMM");
    and a plain torch loop of gather, matmul (hipBLASLt) and index_add_ per
    expert.  The pre-gathered form is checked against the fused result."""
    import torch

    import tile_gemm_communication_amd as fm
    dev = w.mX.device
    w.moe0()
    torch.cuda.synchronize()
    off = [int(v) for v in w.off.cpu().tolist()]
    rows = off[-1]
    sp = w.sp[:rows].long()
    tok = sp // w.topk
    wt = w.wts.reshape(-1)[sp].unsqueeze(1)          # the row's gate weight (fp32)
    Xg = torch.empty((rows, w.hidden), dtype=w.mX.dtype, device=dev)
    Hg = torch.empty((rows, w.ffn), dtype=w.mX.dtype, device=dev)
    Y = torch.empty((rows, w.hidden), dtype=torch.float32, device=dev)
    seed = w.mout.clone()
    experts = [(e, off[e], off[e + 1]) for e in range(w.n_local) if off[e + 1] > off[e]]

    def fused(out):
        w.moe0()
        fm.fm_moe_gemm_scatter(w.H, w.mW2, w.sp, w.off, w.wts, out, w.mws, err_word=w.err)

    def pregathered(out):
        torch.index_select(w.mX, 0, tok, out=Xg)
        for e, a, b in experts:
            fm.fm_gemm(Xg[a:b], w.mW1[e], Hg[a:b])
        for e, a, b in experts:
            fm.fm_gemm(Hg[a:b], w.mW2[e], Y[a:b])
        Y.mul_(wt)
        out.index_add_(0, tok, Y)

    def torch_loop(out):
        for e, a, b in experts:
            xe = w.mX.index_select(0, tok[a:b])
            ye = torch.matmul(torch.matmul(xe, w.mW1[e]), w.mW2[e]).float()
            out.index_add_(0, tok[a:b], ye * wt[a:b])

    o1, o2 = seed.clone(), seed.clone()
    fused(o1)
    pregathered(o2)
    torch.cuda.synchronize()
    check_err(w, "MoE layer (fused)")
    d1, d2 = (o1 - seed).double(), (o2 - seed).double()
    rel = float(torch.linalg.norm(d1 - d2) / torch.linalg.norm(d1))
    if not rel < 1e-3:
        raise RuntimeError(f"pre-gathered MoE layer differs from the fused one: {rel:.3e}")
    res = {"rows_local": rows, "pregathered_vs_fused_rel_frobenius": rel}
    out = seed.clone()
    meds = time_rounds([(name, lambda fn=fn: fn(out))
                        for name, fn in (("fused", fused), ("pregathered_fm_gemm", pregathered),
                                         ("torch_loop", torch_loop))], iters)
    for name, med in meds.items():
        res[f"moe_layer_{name}_ms"] = round(med, 4)
    check_err(w, "MoE layer (fused)")
    return res


def ect_block(w, iters):
    """ECT of the fused AllGather / ReduceScatter operators."""
    import torch

    import tile_gemm_communication_amd as fm
    cs = torch.cuda.current_stream()
    res = {}

    # --- AllGather-GEMM -----------------------------------------------------
    def ns_fm():
        fm.fm_gemm(w.X, w.W1, w.Out1)

    def ns_blas():
        torch.matmul(w.X, w.W1, out=w.Out1)

    # The fused forms end with their last kernel on the compute stream: it
    # cannot finish before every chunk it reads has arrived, and the next
    # iteration's pushes wait for the compute stream, so no join is needed
    # (a cross-stream join only adds its own latency to the measured time).
    def fused():
        w.epoch += 1
        w.push_all(w.epoch)
        if w.serial_arrival:
            w.join_sides()
        w.ag(w.epoch)

    chunk_ev = [torch.cuda.Event() for _ in range(w.n)]

    def producers():
        # the copies run on producer workgroups of the GEMM's own launch
        w.epoch += 1
        fm.fm_ag_gemm_producers([None] + w.peers[1:], w.X, w.W1, w.Out1, w.flags[:w.n],
                                w.counters[:w.n], w.epoch, order=w.order, err_word=w.err)

    def naive():
        # the prior-art sequence: one GEMM launch per chunk, each after its chunk
        w.epoch += 1
        w.push_all(w.epoch, events=chunk_ev)
        for c in w.order:
            if c != w.order[0]:
                cs.wait_event(chunk_ev[c])
            rows = slice(c * w.Mc, (c + 1) * w.Mc)
            fm.fm_gemm(w.X[rows], w.W1, w.Out1[rows])

    log("ECT: AllGather-GEMM")
    meds = time_rounds([("nonsplit_fm_gemm", ns_fm), ("nonsplit_hipblaslt", ns_blas),
                        ("fused", fused), ("naive_chunked", naive), ("producers", producers)],
                       iters)
    for name, med in meds.items():
        res[f"ag_{name}_ms"] = round(med, 4)
    nonsplit = min(res["ag_nonsplit_fm_gemm_ms"], res["ag_nonsplit_hipblaslt_ms"])
    res["ag_ect_ms"] = round(res["ag_fused_ms"] - nonsplit, 4)
    res["ag_ect_vs_fm_gemm_ms"] = round(res["ag_fused_ms"] - res["ag_nonsplit_fm_gemm_ms"], 4)
    res["ag_ect_naive_ms"] = round(res["ag_naive_chunked_ms"] - nonsplit, 4)
    res["ag_ect_producers_ms"] = round(res["ag_producers_ms"] - nonsplit, 4)
    res["ag_ect_frac_of_nonsplit"] = round(res["ag_ect_ms"] / nonsplit, 4)
    assert int(w.err.item()) == 0, "fm_ag_gemm reported a timeout"

    # --- AllGather-GEMM in pull mode, chunks signalled at link speed --------
    # One xGMI link moves a 12.58 MB chunk in t_link = bytes / 153 GB/s.  Ring:
    # the chunk at position a lands at a * t_link.  Direct: every peer pushes
    # over its own link, so all seven land at t_link.  Each chunk is signalled
    # as w.link_parts row blocks, block q once (q+1)/parts of it has crossed
    # the link; the whole-chunk figures (one signal per chunk) are kept beside
    # them.  The chunks are read in place from the peers' buffers: no copy
    # competes with the GEMM.
    t_link = int(w.Mc * w.K1 * 2 / LINK_BYTES_PER_S * 1e9)

    def pull(kind, parts):
        seq, times = link_schedule(w.order, parts, t_link, kind)
        views = part_views(w.peers, parts)
        flags = w.flags[:w.n * parts]

        def fn():
            w.epoch += 1
            s = w.sides[0]
            s.wait_stream(cs)
            fm.fm_chunk_signal_paced(flags, times, w.epoch, order=seq, stream=s)
            fm.fm_ag_gemm_pull(views, w.W1, w.Out1, flags, w.epoch, order=seq, err_word=w.err)
            cs.wait_stream(s)
        return fn

    def pull_naive(kind):
        seq, times = link_schedule(w.order, 1, t_link, kind)

        def fn():
            w.epoch += 1
            s = w.sides[0]
            s.wait_stream(cs)
            fm.fm_chunk_signal_paced(w.flags[:w.n], times, w.epoch, order=seq, stream=s)
            cs.wait_stream(s)                   # the whole AllGather first
            fm.fm_gemm(w.X, w.W1, w.Out1)
        return fn

    log("ECT: pull-mode AllGather-GEMM, link-paced arrival")
    res["pull_link_chunk_us"] = round(t_link / 1e3, 1)
    res["pull_link_parts"] = w.link_parts
    variants = [("nonsplit", ns_fm)]
    for name in ("ring", "direct"):
        variants.append((f"{name}_fused", pull(name, w.link_parts)))
        if w.link_parts != 1:
            variants.append((f"{name}_fused_whole_chunks", pull(name, 1)))
        variants.append((f"{name}_gather_then_gemm", pull_naive(name)))
    meds = time_rounds(variants, iters)
    # baseline: the lower of the non-split GEMM timed in these passes and the
    # one of the AllGather passes above
    ns_pull = min(meds.pop("nonsplit"), nonsplit)
    res["pull_nonsplit_ms"] = round(ns_pull, 4)
    for key, med in meds.items():
        res[f"pull_{key}_ms"] = round(med, 4)
    for name in ("ring", "direct"):
        res[f"pull_{name}_ect_ms"] = round(res[f"pull_{name}_fused_ms"] - ns_pull, 4)
        if w.link_parts != 1:
            res[f"pull_{name}_ect_whole_chunks_ms"] = round(
                res[f"pull_{name}_fused_whole_chunks_ms"] - ns_pull, 4)
        res[f"pull_{name}_ect_naive_ms"] = round(res[f"pull_{name}_gather_then_gemm_ms"]
                                                 - ns_pull, 4)
    assert int(w.err.item()) == 0, "fm_ag_gemm_pull reported a timeout"

    # --- GEMM-ReduceScatter -------------------------------------------------
    tmp16 = torch.empty((w.M, w.N2), dtype=torch.float16, device=w.dev)
    tmp32 = torch.empty((w.M, w.N2), dtype=torch.float32, device=w.dev)
    Ms = w.M // w.P

    def rs_ns_fm():
        fm.fm_gemm(w.Out1, w.W2, tmp16)

    def rs_ns_blas():
        torch.matmul(w.Out1, w.W2, out=tmp16)

    def rs_fused():
        w.rs()

    def rs_naive():
        for s in range(w.P):
            r = (s + 1) % w.P
            rows = slice(r * Ms, (r + 1) * Ms)
            fm.fm_gemm(w.Out1[rows], w.W2, tmp32[rows])
            w.dst[r].add_(tmp32[rows])

    log("ECT: GEMM-ReduceScatter")
    meds = time_rounds([("nonsplit_fm_gemm", rs_ns_fm), ("nonsplit_hipblaslt", rs_ns_blas),
                        ("fused", rs_fused), ("naive_chunked", rs_naive)], iters)
    for name, med in meds.items():
        res[f"rs_{name}_ms"] = round(med, 4)
    nonsplit = min(res["rs_nonsplit_fm_gemm_ms"], res["rs_nonsplit_hipblaslt_ms"])
    res["rs_ect_ms"] = round(res["rs_fused_ms"] - nonsplit, 4)
    res["rs_ect_vs_fm_gemm_ms"] = round(res["rs_fused_ms"] - res["rs_nonsplit_fm_gemm_ms"], 4)
    res["rs_ect_naive_ms"] = round(res["rs_naive_chunked_ms"] - nonsplit, 4)
    res["rs_ect_frac_of_nonsplit"] = round(res["rs_ect_ms"] / nonsplit, 4)

    # --- token AllGather + MoE layer 0 --------------------------------------
    def moe_ns():
        w.moe0()

    def moe_fused():
        w.epoch += 1
        w.push_all(w.epoch, moe=True)
        if w.serial_arrival:
            w.join_sides()
        w.moe0_ag(w.epoch)

    def moe_naive():
        # the whole AllGather first, then the layer
        w.epoch += 1
        w.push_all(w.epoch, moe=True)
        w.join_sides()
        fm.fm_moe_gather_gemm(w.mXg, w.ids, w.mW1, w.H, w.sp, w.off, w.e0, w.mws)

    def moe_producers():
        # the token copies run on producer workgroups of layer 0's own launch
        w.epoch += 1
        fm.fm_moe_ag_gather_gemm_producers([None] + w.mpeers[1:], w.mXg, w.ids, w.mW1, w.H, w.sp,
                                           w.off, w.e0, w.mflags[:w.n], w.mcounters[:w.n],
                                           w.epoch, w.mws, order=w.order, err_word=w.err)

    # pull mode: layer 0 reads each owner's 16 MiB chunk in place, signals
    # timed at one link's rate (direct: all seven land at t_link), each chunk
    # signalled as w.moe_link_parts token blocks (layer 0 gathers its rows
    # token by token, so a block need not be a whole tile row)
    t_link_moe = int(w.mTc * w.hidden * 2 / LINK_BYTES_PER_S * 1e9)

    def moe_pull(kind, parts):
        seq, times = link_schedule(w.order, parts, t_link_moe, kind)
        views = part_views(w.mpeers, parts)
        flags = w.mflags[:w.n * parts]

        def fn():
            w.epoch += 1
            s = w.sides[0]
            s.wait_stream(cs)
            fm.fm_chunk_signal_paced(flags, times, w.epoch, order=seq, stream=s)
            fm.fm_moe_ag_gather_gemm_pull(views, w.ids, w.mW1, w.H, w.sp, w.off, w.e0, flags,
                                          w.epoch, w.mws, order=seq, err_word=w.err)
            cs.wait_stream(s)
        return fn

    def moe_pull_naive(kind):
        seq, times = link_schedule(w.order, 1, t_link_moe, kind)

        def fn():
            w.epoch += 1
            s = w.sides[0]
            s.wait_stream(cs)
            fm.fm_chunk_signal_paced(w.mflags[:w.n], times, w.epoch, order=seq, stream=s)
            cs.wait_stream(s)                   # the whole AllGather first
            w.moe0()
        return fn

    log("ECT: token AllGather + MoE layer 0")
    P = w.moe_link_parts
    variants = [("ag_nonsplit", moe_ns), ("ag_fused", moe_fused),
                ("ag_gather_then_gemm", moe_naive), ("ag_producers", moe_producers)]
    for name in ("direct", "ring"):
        variants.append((f"pull_{name}_fused", moe_pull(name, P)))
        if P != 1:
            variants.append((f"pull_{name}_fused_whole_chunks", moe_pull(name, 1)))
        variants.append((f"pull_{name}_gather_then_gemm", moe_pull_naive(name)))
    meds = time_rounds(variants, iters)
    check_err(w, "MoE layer 0 with its token AllGather")
    for key, med in meds.items():
        res[f"moe_{key}_ms"] = round(med, 4)
    ns = res["moe_ag_nonsplit_ms"]
    res["moe_ag_ect_ms"] = round(res["moe_ag_fused_ms"] - ns, 4)
    res["moe_ag_ect_naive_ms"] = round(res["moe_ag_gather_then_gemm_ms"] - ns, 4)
    res["moe_ag_ect_frac_of_nonsplit"] = round(res["moe_ag_ect_ms"] / ns, 4)
    res["moe_ag_ect_producers_ms"] = round(res["moe_ag_producers_ms"] - ns, 4)
    res["moe_pull_link_chunk_us"] = round(t_link_moe / 1e3, 1)
    res["moe_pull_link_parts"] = P
    for name in ("direct", "ring"):
        res[f"moe_pull_{name}_ect_ms"] = round(res[f"moe_pull_{name}_fused_ms"] - ns, 4)
        if P != 1:
            res[f"moe_pull_{name}_ect_whole_chunks_ms"] = round(
                res[f"moe_pull_{name}_fused_whole_chunks_ms"] - ns, 4)
        res[f"moe_pull_{name}_ect_naive_ms"] = round(
            res[f"moe_pull_{name}_gather_then_gemm_ms"] - ns, 4)
    assert int(w.err.item()) == 0, "fm_moe_ag_gather_gemm reported a timeout"
    res["nonsplit_fm_gemm_tflops_4096x12288x6144"] = round(
        w.flop_rs / (res["rs_nonsplit_fm_gemm_ms"] * 1e-3) / 1e12, 1)
    res["nonsplit_hipblaslt_tflops_4096x12288x6144"] = round(
        w.flop_rs / (res["rs_nonsplit_hipblaslt_ms"] * 1e-3) / 1e12, 1)
    return res


def traffic(op):
    """Measured HBM bytes per launch of `op` (read + written); traffic is None
    when the kernel sources changed since the counters were taken."""
    if op not in TRAFFIC_BYTES or source_digest() != TRAFFIC_DIGEST:
        return {"traffic": None}
    rd, wr = TRAFFIC_BYTES[op]
    return {"traffic": rd + wr, "traffic_read": rd, "traffic_write": wr,
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x2.0 + WRITE_SIZE x1.0)"}


def cpu_baseline(w, rows):
    """The CPU oracle, untuned, on a bounded sample of the AllGather-GEMM:
    `rows` output rows of Output1 = X * W1 (fp64 accumulation)."""
    import numpy as np

    import oracle
    orc = oracle.load()
    X = np.concatenate(list(w.chunks_host), axis=0)[:rows]
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    orc.gemm(0, X, w.W1_host)
    dt = time.perf_counter() - t0
    flop = 2.0 * rows * w.N1 * w.K1
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"AllGather-GEMM rows 0..{rows - 1} of 4096 "
                      f"({rows}x{w.N1}x{w.K1}, fp64 accumulation)"}


def copy_probe(mib):
    """Three fm_chunk_push copies of `mib` MiB: a kernel whose HBM traffic is
    known (read mib, write mib), to scale the profiler's byte counters."""
    import torch

    import tile_gemm_communication_amd as fm
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for e in range(1, 4):
        fm.fm_chunk_push(src, dst, flag, cnt, e)
    torch.cuda.synchronize()
    assert bool((dst == 1).all())
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                      "dispatches": 3}), flush=True)


def mfma_ceiling():
    """The matrix-core rate with no memory traffic (fm_probe_mfma): bf16 and
    fp16, the 32x32x16 and 16x16x32 forms, one and two waves per SIMD,
    N(0,1)-like and all-zero operands.  Each form runs ~0.2 s after a warm-up
    launch; the clock is the median over workgroups of shader cycles per
    100 MHz tick."""
    import torch

    import tile_gemm_communication_amd as fm
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros(4 * cus, dtype=torch.int64, device="cuda:0")
    rows = []
    for dt in (torch.bfloat16, torch.float16):
        for mf16 in (False, True):
            for waves in (1, 2):
                for zero in (False, True):
                    flop_per = (16384 if mf16 else 32768) * 8
                    per_iter = cus * 4 * waves * flop_per
                    iters = 2000
                    fm.fm_probe_mfma(dt, mf16, waves, iters, zero, out)   # warm-up
                    torch.cuda.synchronize()
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    fm.fm_probe_mfma(dt, mf16, waves, iters, zero, out)
                    b.record()
                    torch.cuda.synchronize()
                    ms = a.elapsed_time(b)
                    iters = max(1, int(iters * 200.0 / max(ms, 1e-3)))   # ~0.2 s
                    a.record()
                    fm.fm_probe_mfma(dt, mf16, waves, iters, zero, out)
                    b.record()
                    torch.cuda.synchronize()
                    ms = a.elapsed_time(b)
                    o = out.view(cus, 4).cpu().numpy()
                    ghz = float(sorted(o[:, 0] / o[:, 1])[cus // 2]) * 0.1
                    tf = per_iter * iters / (ms * 1e-3) / 1e12
                    rows.append({"dtype": "bf16" if dt == torch.bfloat16 else "f16",
                                 "mfma": "16x16x32" if mf16 else "32x32x16",
                                 "waves_per_simd": waves, "operands": "zero" if zero else "N(0,1)",
                                 "tflops": round(tf, 1), "clock_ghz": round(ghz, 3),
                                 "frac_of_2516.6": round(tf / PEAK_TFLOPS, 4),
                                 "frac_at_clock": round(tf / (cus * 4096 * ghz * 1e-3), 4)})
                    log(f"mfma ceiling {rows[-1]}")
    print(json.dumps({"mfma_ceiling": rows}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the fused kernels "
                                   "emulate the peers of a TP=8/EP=8 group on one device; "
                                   "run with --gpus 1"}))
        sys.exit(2)
    import torch

    import tile_gemm_communication_amd as fm
    fm.lib()                                   # fail loudly if the library is missing
    log(f"libfluxmi {fm.version()} on {torch.cuda.get_device_name(0)}")
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    w = Workload()
    w.serial_arrival = args.serial_arrival
    w.arrival = args.arrival
    w.parts = args.parts
    w.link_parts = args.link_parts
    w.moe_link_parts = args.moe_link_parts
    cs = torch.cuda.current_stream()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        w.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert int(w.err.item()) == 0, f"a kernel reported {fm.status_str(int(w.err.item()))}"
    ms_step = (t1 - t0) * 1e3 / args.steps
    # Per-operator times: the same K steps again with HIP events between the
    # operators on the compute stream.  Each timing event costs the stream a
    # few microseconds, so `value` comes from the loop above, which has none.
    log(f"timing {args.steps} steps with per-operator events")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(args.steps):
        w.step(evs[k])
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    assert int(w.err.item()) == 0, f"a kernel reported {fm.status_str(int(w.err.item()))}"
    ms_step_events = (t3 - t2) * 1e3 / args.steps
    names = ["ag_gemm", "gemm_rs", "moe_gather_gemm", "moe_gemm_scatter"]
    per_step = {n: sorted(evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps))
                for i, n in enumerate(names)}
    durs = {n: sum(v) / len(v) for n, v in per_step.items()}
    flops = {"ag_gemm": w.flop_ag, "gemm_rs": w.flop_rs,
             "moe_gather_gemm": w.flop_moe / 2, "moe_gemm_scatter": w.flop_moe / 2}
    total_flop = sum(flops.values())
    value = total_flop / (ms_step * 1e-3) / 1e12
    ops = {n: {"ms": round(durs[n], 4),
               "median_ms": round(per_step[n][len(per_step[n]) // 2], 4),
               "min_ms": round(per_step[n][0], 4),
               "tflops": round(flops[n] / (durs[n] * 1e-3) / 1e12, 1),
               "frac_peak": round(flops[n] / (durs[n] * 1e-3) / 1e12 / PEAK_TFLOPS, 4)}
           for n in names}
    dom = max(names, key=lambda n: durs[n])
    achieved = flops[dom] / (durs[dom] * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms, {value:.1f} TFLOP/s; " +
        ", ".join(f"{n} {ops[n]['ms']:.3f} ms {ops[n]['tflops']} TF" for n in names))

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_with_op_events": round(ms_step_events, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/bf16 (fp32 accumulate)",
        "data": "synthetic (seeded N(0,1) activations, N(0,1)/sqrt(K) weights, log-Zipf router)",
        "config": {
            "workload": "one rank of a TP=8/EP=8 layer step: AllGather-GEMM 4096x6144x12288 "
                        "(8 chunks of 512 rows, 7 pushed by 3 side streams) -> GEMM-ReduceScatter "
                        "4096x12288x6144 into 8 fp32 slices (fp16); MoE 16384 tokens x 4096, "
                        "64 experts top-2, 8 local, ffn 2816 (bf16)",
            "moe_rows_local": w.rows_local,
            "arrival": f"{args.arrival} pushes, 3 side streams",
            "step_flop": total_flop,
        },
        "ops": ops,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS, 4), **traffic(dom)},
    }
    if not args.no_cold:
        out["cold_ms"] = cold_ops(w)
    if not args.no_ect:
        out["ect"] = ect_block(w, args.ect_iters)
        log("MoE layer against its unfused forms")
        out["moe_baselines"] = moe_baselines(w, args.ect_iters)
    if not args.no_cpu_baseline:
        log(f"CPU oracle sample ({args.cpu_rows} rows)")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
