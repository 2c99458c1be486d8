"""GPU tests of the MoE combine's scheduling and error reporting
(fm_moe_gemm_scatter): tiles handed out by ticket complete whatever grid the
launch gets, two expert-parallel ranks run side by side on two streams with
their own workspaces, a wait that gives up is reported through err_word (and
the workspace stays usable), and a token routed twice to one expert is
reported instead of silently losing an update.  Parity is against the CPU
oracle's per-token combine (COMET article, "COMET 的技术原理")."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import BF16, assert_close, dev16, devf32, host64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda:0")


class Layer:
    """One rank's MoE layer on the GPU: its own buffers and workspace."""

    def __init__(self, inp, e0, nl, stream=None):
        import torch
        import tile_gemm_communication_amd as fm
        self.inp, self.e0, self.nl = inp, e0, nl
        T, self.topk = inp["topk_ids"].shape
        self.T = T
        self.hidden = inp["X"].shape[1]
        self.ffn = inp["W1"].shape[2]
        dev = "cuda:0"
        self.X = dev16(inp["X"], BF16)
        self.W1 = dev16(inp["W1"], BF16)
        self.W2 = dev16(inp["W2"], BF16)
        self.ids = _i32(inp["topk_ids"])
        self.wts = devf32(inp["topk_weights"])
        self.H = torch.zeros((T * self.topk, self.ffn), dtype=torch.bfloat16, device=dev)
        self.sp = torch.full((T * self.topk,), -1, dtype=torch.int32, device=dev)
        self.off = torch.zeros(nl + 1, dtype=torch.int32, device=dev)
        self.out = devf32(inp["out_seed"])
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ws = fm.moe_workspace(T, self.topk, self.hidden, nl)
        self.stream = stream

    def run(self, spin=0, out=None):
        import tile_gemm_communication_amd as fm
        out = self.out if out is None else out
        fm.fm_moe_gather_gemm(self.X, self.ids, self.W1, self.H, self.sp, self.off, self.e0,
                              self.ws, stream=self.stream)
        fm.fm_moe_gemm_scatter(self.H, self.W2, self.sp, self.off, self.wts, out, self.ws,
                               err_word=self.err, spin_limit=spin, stream=self.stream)


def _oracle_combine(oracle, inp, e0, nl):
    """The oracle's chain: route, layer 0, H rounded to bf16, combine."""
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    Hb = oracle.round_bf16(oracle.moe_layer0(BF16, inp["X"], inp["W1"], rsp, roff,
                                             inp["topk_ids"].shape[1]))
    return oracle.moe_layer1(BF16, Hb, inp["W2"], inp["topk_ids"], inp["topk_weights"], rsp,
                             roff, inp["out_seed"], e0)


@pytest.mark.parametrize("grid,spin", [(1024, 1 << 16), (1, 1 << 16), (37, 1 << 16)])
def test_combine_any_grid(oracle, monkeypatch, grid, spin):
    """More workgroups than compute units (most wait to be dispatched), a
    single workgroup, and an odd count: tickets hand tiles out in expert
    order to running workgroups, so every launch completes with a modest
    spin limit, reports nothing, and matches the oracle element by element."""
    import torch
    monkeypatch.setenv("FM_COMBINE_GRID", str(grid))
    T, hidden, ffn, E, nl, e0 = 3000, 512, 264, 16, 8, 0
    say(f"combine grid={grid} spin={spin} T={T}")
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=900 + grid, zipf_s=1.2)
    lay = Layer(inp, e0, nl)
    lay.run(spin=spin)
    torch.cuda.synchronize()
    assert lay.err.item() == 0, lay.err.item()
    ref = _oracle_combine(oracle, inp, e0, nl)
    assert_close(host64(lay.out) - inp["out_seed"], ref - inp["out_seed"], f"grid {grid}")
    # the same launch again on the same workspace: identical bits
    out2 = devf32(inp["out_seed"])
    lay.run(spin=spin, out=out2)
    torch.cuda.synchronize()
    assert lay.err.item() == 0
    assert torch.equal(out2.view(torch.int32), lay.out.view(torch.int32))


def test_two_ranks_on_two_streams(oracle):
    """Two expert-parallel ranks (experts 0..7 and 8..15) run their whole MoE
    layer at the same time on two streams, each with its own workspace: both
    equal their sequential runs bit for bit and the oracle within the bar."""
    import torch
    T, hidden, ffn, E, nl = 6144, 1024, 512, 16, 8
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=4711, zipf_s=0.8)
    # each rank owns its weights: take rank 1's from a different seed
    inp1 = dict(inp)
    other = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=4712, zipf_s=0.8)
    inp1["W1"], inp1["W2"] = other["W1"], other["W2"]
    ranks = [(inp, 0), (inp1, 8)]
    say("two ranks, sequential")
    seq = []
    for rin, e0 in ranks:
        lay = Layer(rin, e0, nl)
        lay.run()
        torch.cuda.synchronize()
        assert lay.err.item() == 0
        seq.append(lay.out.clone())
    say("two ranks, concurrent on two streams")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    lays = [Layer(rin, e0, nl, stream=s) for (rin, e0), s in zip(ranks, streams)]
    torch.cuda.synchronize()
    for rep in range(3):
        for lay in lays:
            lay.out.copy_(devf32(lay.inp["out_seed"]))
        torch.cuda.synchronize()
        for lay in lays:
            lay.stream.wait_stream(torch.cuda.current_stream())
        for lay in lays:
            lay.run()
        for lay in lays:
            torch.cuda.current_stream().wait_stream(lay.stream)
        torch.cuda.synchronize()
        for r, lay in enumerate(lays):
            assert lay.err.item() == 0, (rep, r, lay.err.item())
            assert torch.equal(lay.out.view(torch.int32), seq[r].view(torch.int32)), (rep, r)
    for (rin, e0), lay in zip(ranks, lays):
        ref = _oracle_combine(oracle, rin, e0, nl)
        assert_close(host64(lay.out) - rin["out_seed"], ref - rin["out_seed"], f"rank e0={e0}")


def test_combine_timeout_is_reported_and_workspace_recovers(oracle):
    """A tile that never completes: hidden = 256 is one tile column, so one
    tile queue, and the test starts that queue's ticket counter (control
    word 8) at 1: expert 0's first row tile is never handed out, and expert
    1's tile over the same tokens waits for it.  With a spin limit of 2000
    polls the launch reports FM_ERR_TIMEOUT (never a silent add) and
    returns; its last workgroup resets the counters, so the next launch on
    the same workspace is complete and correct."""
    import torch
    import tile_gemm_communication_amd as fm
    T, hidden, ffn, nl = 4096, 256, 512, 2
    inp = wl.moe_inputs(T, hidden, ffn, 4, nl, 2, BF16, seed=31)
    inp["topk_ids"] = np.tile(np.array([[0, 1]], dtype=np.int32), (T, 1))
    lay = Layer(inp, 0, nl)
    lay.ws.view(torch.int32)[8] = 1
    lay.run(spin=2000)
    torch.cuda.synchronize()
    assert lay.err.item() == fm.FM_ERR_TIMEOUT
    assert (lay.ws.view(torch.int32)[8:12] == 0).all()    # the ticket counters are reset
    lay.err.zero_()
    out = devf32(inp["out_seed"])
    lay.run(out=out)
    torch.cuda.synchronize()
    assert lay.err.item() == 0
    ref = _oracle_combine(oracle, inp, 0, nl)
    assert_close(host64(out) - inp["out_seed"], ref - inp["out_seed"], "after a timeout")


def test_combine_duplicate_expert_is_reported():
    """Token 5 has both of its pairs in local expert 3: the combine reports
    FM_ERR_INVALID_ARG in err_word instead of racing two adds into one row."""
    import torch
    import tile_gemm_communication_amd as fm
    T, hidden, ffn, nl = 600, 128, 64, 8
    inp = wl.moe_inputs(T, hidden, ffn, 16, nl, 2, BF16, seed=8)
    inp["topk_ids"] = inp["topk_ids"].copy()
    inp["topk_ids"][5] = [3, 3]
    lay = Layer(inp, 0, nl)
    lay.run()
    torch.cuda.synchronize()
    assert lay.err.item() == fm.FM_ERR_INVALID_ARG


def test_eight_emulated_ep_ranks_sum_to_all_experts(oracle):
    """Eight emulated expert-parallel ranks (experts 8r .. 8r+7) each run
    layer 0 and the combine on the GPU, accumulating into one shared out: the
    sum equals the oracle's combine over all 64 experts (the rank split of
    the per-token sum)."""
    import torch
    import tile_gemm_communication_amd as fm
    T, hidden, ffn, E, P = 2048, 512, 256, 64, 8
    nl = E // P
    base = wl.moe_inputs(T, hidden, ffn, E, E, 2, BF16, seed=2024, zipf_s=1.2)
    out = devf32(base["out_seed"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    X, ids, wts = dev16(base["X"], BF16), _i32(base["topk_ids"]), devf32(base["topk_weights"])
    for r in range(P):
        W1 = dev16(base["W1"][r * nl:(r + 1) * nl], BF16)
        W2 = dev16(base["W2"][r * nl:(r + 1) * nl], BF16)
        H = torch.zeros((T * 2, ffn), dtype=torch.bfloat16, device="cuda:0")
        sp = torch.full((T * 2,), -1, dtype=torch.int32, device="cuda:0")
        off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
        ws = fm.moe_workspace(T, 2, hidden, nl)
        fm.fm_moe_gather_gemm(X, ids, W1, H, sp, off, r * nl, ws)
        fm.fm_moe_gemm_scatter(H, W2, sp, off, wts, out, ws, err_word=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref = _oracle_combine(oracle, base, 0, E)
    assert_close(host64(out) - base["out_seed"], ref - base["out_seed"], "8 EP ranks")


def test_combine_and_layer0_beyond_the_cached_tile_ranges(oracle):
    """140000 tokens, top-2 over 8 local experts, hidden = ffn = 64: more
    than 1024 row tiles, so the combine waits on every earlier tile of its
    column (the uncached form) and layer 0 behind a token AllGather has more
    than 256 bands (the index-order form).  Element by element against the
    oracle; the AllGather form bit-identical to the plain layer 0."""
    import torch
    import tile_gemm_communication_amd as fm
    from gpu_util import Arrival
    T, hidden, ffn, E, nl, n = 140000, 64, 64, 8, 8, 8
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=140, zipf_s=1.2)
    roff, rsp = oracle.moe_route(inp["topk_ids"], 0, nl)
    def cdiv(a, b):
        return -(-a // b)
    tiles_e = [cdiv(int(roff[e + 1] - roff[e]), 256) for e in range(nl)]
    tiles, bands = sum(tiles_e), sum(cdiv(t, 2) for t in tiles_e)
    say(f"large T: {tiles} row tiles, {bands} bands")
    assert tiles > 1024 and bands > 256
    lay = Layer(inp, 0, nl)
    lay.run()
    torch.cuda.synchronize()
    assert lay.err.item() == 0
    rows = int(roff[-1])
    assert np.array_equal(lay.off.cpu().numpy(), roff)
    assert np.array_equal(lay.sp.cpu().numpy()[:rows], rsp)
    Href = oracle.moe_layer0(BF16, inp["X"], inp["W1"], rsp, roff, 2)
    assert_close(host64(lay.H[:rows]), Href, "large-T layer 0")
    ref = oracle.moe_layer1(BF16, oracle.round_bf16(Href), inp["W2"], inp["topk_ids"],
                            inp["topk_weights"], rsp, roff, inp["out_seed"], 0)
    assert_close(host64(lay.out) - inp["out_seed"], ref - inp["out_seed"], "large-T combine")
    # token AllGather in front of layer 0: more bands than the ordered form holds
    chunks = inp["X"].reshape(n, T // n, hidden)
    arr = Arrival(chunks, BF16, hidden)
    arr.poison()
    H2 = torch.zeros_like(lay.H)
    sp2 = torch.full_like(lay.sp, -1)
    off2 = torch.zeros_like(lay.off)
    order = wl.permutation(n, seed=141).tolist()
    ep = arr.next_epoch()
    arr.push(order, ep)
    fm.fm_moe_ag_gather_gemm(arr.X, lay.ids, lay.W1, H2, sp2, off2, 0, arr.flags, ep, n,
                             fm.moe_workspace(T, 2, hidden, nl), order=order, err_word=arr.err)
    arr.join()
    torch.cuda.synchronize()
    assert arr.err.item() == 0
    assert np.array_equal(off2.cpu().numpy(), roff)
    assert torch.equal(H2[:rows].view(torch.int16), lay.H[:rows].view(torch.int16))


@pytest.mark.parametrize("T,hidden,ffn,topk", [(3000, 520, 264, 2), (700, 200, 136, 4),
                                                (5000, 1024, 512, 2), (2500, 1672, 256, 2)])
def test_combine_epilogue_forms_bit_identical(oracle, monkeypatch, T, hidden, ffn, topk):
    """The combine's two epilogues, the register-fetch form over a buffer
    resource (the default below 2 GiB of out) and the LDS-DMA form
    (FM_COMBINE_DMA=1, the one for larger outputs), add the same products in
    the same order: out is bit-identical, and both match the oracle.  Hidden
    sizes past a 256-column tile edge, rows past an expert's last tile, a
    ragged K (136: the 4-wave tail kernel, whose epilogue is always the DMA
    form) and top-4 routing; hidden = 1672 is 7 tile columns over the 4
    tile queues (two columns to three queues, one to the last)."""
    import torch
    import tile_gemm_communication_amd as fm
    E, nl, e0 = 16, 8, 8
    say(f"combine epilogue forms T={T} hidden={hidden} ffn={ffn} topk={topk}")
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, topk, BF16, seed=T + hidden, zipf_s=1.2)
    lay = Layer(inp, e0, nl)
    outs = {}
    for form, env in (("vgpr", "0"), ("dma", "1")):
        monkeypatch.setenv("FM_COMBINE_DMA", env)
        out = devf32(inp["out_seed"])
        lay.run(out=out)
        torch.cuda.synchronize()
        assert lay.err.item() == 0
        outs[form] = out
    assert torch.equal(outs["vgpr"].view(torch.int32), outs["dma"].view(torch.int32))
    ref = _oracle_combine(oracle, inp, e0, nl)
    assert_close(host64(outs["vgpr"]) - inp["out_seed"], ref - inp["out_seed"], "combine forms")


@pytest.mark.parametrize("T", [131000, 140000])
def test_combine_outputs_near_and_past_2gib(oracle, T):
    """out of 131000 x 4096 fp32 (2.146e9 bytes: the register-fetch epilogue,
    whose 32-bit offsets then reach just under its limit) and of 140000 x
    4096 (2.29e9 bytes: past the limit, so the LDS-DMA epilogue runs).  H is
    drawn directly (ffn = 64, one K step) and out starts at zero; every token
    matches the oracle's every-element combine (compared in row blocks),
    tokens sampled across the whole range, the last 64 among them, match its
    loops, and the routing is bit-exact."""
    import torch
    import tile_gemm_communication_amd as fm
    hidden, ffn, E, nl, topk, e0 = 4096, 64, 16, 8, 2, 0
    say(f"combine with a {T * hidden * 4 / 1e9:.3f} GB out")
    rng = np.random.default_rng(T)
    first = rng.integers(0, E, T)
    ids = np.stack([first, (first + 1 + rng.integers(0, E - 1, T)) % E], 1).astype(np.int32)
    wts = rng.random((T, topk), dtype=np.float32)
    roff, rsp = oracle.moe_route(ids, e0, nl)
    rows = int(roff[-1])
    Hb = wl.normal_bits((rows, ffn), T + 1, BF16)
    W2b = wl.normal_bits((nl, ffn, hidden), T + 2, BF16, 1.0 / np.sqrt(ffn))
    dev = "cuda:0"
    H = torch.zeros((T * topk, ffn), dtype=torch.bfloat16, device=dev)
    H[:rows] = dev16(Hb, BF16)
    W2 = dev16(W2b, BF16)
    ids_d = _i32(ids)
    wts_d = devf32(wts)
    sp = torch.full((T * topk,), -1, dtype=torch.int32, device=dev)
    off = torch.zeros(nl + 1, dtype=torch.int32, device=dev)
    out = torch.zeros((T, hidden), dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = fm.moe_workspace(T, topk, hidden, nl)
    fm.fm_moe_route(ids_d, e0, nl, sp, off, ws)
    fm.fm_moe_gemm_scatter(H, W2, sp, off, wts_d, out, ws, err_word=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(sp[:rows].cpu().numpy(), rsp)
    toks = np.unique(np.concatenate([rng.integers(0, T, 200), np.arange(T - 64, T)]))
    seed = np.zeros((T, hidden), dtype=np.float32)      # never touched: pages stay unmapped
    ref = oracle.moe_layer1_tokens(BF16, Hb, W2b, ids, wts, rsp, roff, seed, e0, toks)
    got = host64(out[torch.from_numpy(toks).to(dev)])
    assert_close(got, ref, f"combine, out of {T} rows")
    from oracle import full
    want = full.moe_layer1(BF16, Hb, W2b, ids, wts, rsp, roff, seed, e0)
    del seed
    for r0 in range(0, T, 16384):
        r1 = min(T, r0 + 16384)
        assert_close(host64(out[r0:r1]), want[r0:r1],
                     f"combine, out of {T} rows, rows {r0}..{r1}")
