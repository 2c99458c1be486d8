"""HIP-graph capture of the hot path: a step captured once and replayed
several times, with eager work and synchronisations between the replays,
must reproduce the eager result bit for bit on every replay."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import BF16, F16, Arrival, dev16, devf32, say, side_stream

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _capture(body):
    """Warm up on a side stream, then capture body() into a graph."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("act", [None, 2])
def test_graph_moe_layer_replays(act):
    """Route + layer 0 (plain, or with the tanh-form GELU fused) + the combine
    in one graph.  The combine's ordering epoch advances on the device, so
    each replay (and the eager calls between replays, which advance it too)
    orders its tiles correctly."""
    import torch
    import tile_gemm_communication_amd as fm
    T, hidden, ffn, E, nl, e0 = 3072, 256, 264, 16, 8, 0
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=77, zipf_s=1.2)
    X, W1, W2 = dev16(inp["X"], BF16), dev16(inp["W1"], BF16), dev16(inp["W2"], BF16)
    ids = torch.from_numpy(inp["topk_ids"]).to("cuda:0")
    wts = devf32(inp["topk_weights"])
    seed = devf32(inp["out_seed"])
    H = torch.zeros((T * 2, ffn), dtype=torch.bfloat16, device="cuda:0")
    sp = torch.full((T * 2,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    out = torch.empty_like(seed)
    ws = fm.moe_workspace(T, 2, hidden, nl)
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def body():
        out.copy_(seed)
        if act is None:
            fm.fm_moe_gather_gemm(X, ids, W1, H, sp, off, e0, ws)
        else:
            fm.fm_moe_gather_gemm_act(X, ids, W1, H, sp, off, e0, act, ws)
        fm.fm_moe_gemm_scatter(H, W2, sp, off, wts, out, ws, err_word=err)

    body()
    torch.cuda.synchronize()
    ref = out.clone()
    g = _capture(body)
    other = torch.empty_like(seed)
    for r in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say(f"moe graph replay {r} act={act}")
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {r}"
        # eager combine calls between replays move the device epoch on
        other.copy_(seed)
        fm.fm_moe_gemm_scatter(H, W2, sp, off, wts, other, ws, err_word=err)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int32), ref.view(torch.int32))
        assert err.item() == 0


def test_graph_ag_rs_replays():
    """Pushed AllGather chunks, the AllGather-GEMM and the GEMM-ReduceScatter
    in one graph.  The graph repeats one epoch, so it zeroes the flags with a
    fill kernel first; the side stream is forked and joined inside it."""
    import torch
    import tile_gemm_communication_amd as fm
    n, Mc, K, N1, N2, P = 4, 256, 512, 384, 512, 4
    chunks, W1b, _ = wl.ag_inputs(n, Mc, N1, K, F16, seed=91, arrival="ring")
    _, W2b, seeds = wl.rs_inputs(n * Mc, N2, N1, P, F16, seed=92)
    arr = Arrival(chunks, F16, K)
    W1, W2 = dev16(W1b, F16), dev16(W2b, F16)
    C = torch.empty((n * Mc, N1), dtype=torch.float16, device="cuda:0")
    seed_d = [devf32(x) for x in seeds]
    dst = [torch.empty_like(x) for x in seed_d]
    epoch = arr.next_epoch()

    def body():
        arr.flags.zero_()
        for d, s0 in zip(dst, seed_d):
            d.copy_(s0)
        arr.push(list(range(n)), epoch, local=0)
        fm.fm_ag_gemm(arr.X, W1, C, arr.flags, epoch, n, err_word=arr.err)
        arr.join()
        fm.fm_gemm_rs(C, W2, dst, rank=1)

    arr.poison()
    body()
    torch.cuda.synchronize()
    refC = C.clone()
    refD = [d.clone() for d in dst]
    assert arr.err.item() == 0
    g = _capture(body)
    for r in range(4):
        arr.poison()
        C.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say(f"ag/rs graph replay {r}")
        assert arr.err.item() == 0
        assert torch.equal(C.view(torch.int16), refC.view(torch.int16)), f"replay {r}"
        for d, rd in zip(dst, refD):
            assert torch.equal(d.view(torch.int32), rd.view(torch.int32)), f"replay {r}"
        # eager work between replays: the same operators on the same buffers
        body()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int16), refC.view(torch.int16))
