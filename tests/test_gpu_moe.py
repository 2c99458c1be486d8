"""GPU parity of the MoE path (fm_moe_route, fm_moe_gather_gemm,
fm_moe_gemm_scatter) against the CPU oracle: routing buffers bit-exact,
expert outputs and the weighted combine within the parity bar (on the delta
out - seed)."""
import numpy as np
import pytest

import workloads as wl
from oracle import full
from gpu_util import BF16, F16, assert_close, bits16, dev16, devf32, host64, say, side_stream

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda:0")


def _route(ids, e0, nl):
    import torch
    import tile_gemm_communication_amd as fm
    T, k = ids.shape
    sp = torch.full((T * k,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_route(_i32(ids), e0, nl, sp, off, fm.moe_workspace(T, k, 8, nl))
    torch.cuda.synchronize()
    off_h = off.cpu().numpy()
    return off_h, sp.cpu().numpy()[:off_h[-1]]


@pytest.mark.parametrize("T,E,topk,e0,nl", [(256, 16, 2, 4, 4), (5000, 64, 2, 0, 8),
                                            (3, 8, 1, 0, 8), (1000, 64, 4, 56, 8),
                                            (20000, 128, 2, 0, 64), (3000, 64, 2, 3, 5),
                                            (9000, 96, 2, 8, 48), (40000, 128, 2, 0, 64)])
def test_route_bit_exact(oracle, T, E, topk, e0, nl):
    """Chunks of 256 pairs, one workgroup each; expert counts that do not
    divide the 256 threads summing the chunk histograms (5, 48); and 80000
    pairs over 64 local experts, whose histograms need chunks of 512 (two
    rounds per workgroup)."""
    ids, _ = wl.moe_routing(T, E, topk, seed=T + E)
    off, sp = _route(ids, e0, nl)
    roff, rsp = oracle.moe_route(ids, e0, nl)
    assert np.array_equal(off, roff) and np.array_equal(sp, rsp)


def test_route_edges(oracle):
    ids = np.full((50, 2), 9, dtype=np.int32)
    off, sp = _route(ids, 0, 8)        # nothing local
    assert off.tolist() == [0] * 9 and sp.size == 0
    ids = np.zeros((37, 2), dtype=np.int32)
    ids[:, 1] = 3
    off, sp = _route(ids, 0, 4)        # two experts take everything, two are empty
    roff, rsp = oracle.moe_route(ids, 0, 4)
    assert np.array_equal(off, roff) and np.array_equal(sp, rsp)


def _moe_run(inp, e0, nl, dt, H_in=None):
    import torch
    import tile_gemm_communication_amd as fm
    ids, wts = inp["topk_ids"], inp["topk_weights"]
    T, topk = ids.shape
    ffn = inp["W1"].shape[2]
    hidden = inp["X"].shape[1]
    sp = torch.full((T * topk,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    H = torch.zeros((T * topk, ffn), dtype=torch.float16 if dt == F16 else torch.bfloat16,
                    device="cuda:0")
    ws = fm.moe_workspace(T, topk, hidden, nl)
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm(dev16(inp["X"], dt), _i32(ids), dev16(inp["W1"], dt), H, sp, off, e0,
                          ws)
    out = devf32(inp["out_seed"])
    Hsrc = H if H_in is None else dev16(H_in, dt)
    fm.fm_moe_gemm_scatter(Hsrc, dev16(inp["W2"], dt), sp, off, devf32(wts), out, ws,
                           err_word=err)
    torch.cuda.synchronize()
    assert err.item() == 0, fm.status_str(err.item())
    torch.cuda.synchronize()
    return off.cpu().numpy(), sp.cpu().numpy(), H, out


@pytest.mark.parametrize("tile", ["256x256", "256x256w4", "256x256w8", "256x128w8", "128x128"])
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("T,hidden,ffn,E,nl,e0", [(256, 256, 128, 16, 4, 4),
                                                  (300, 136, 264, 8, 8, 0),
                                                  (64, 512, 512, 64, 8, 0)])
def test_moe_small(oracle, monkeypatch, tile, dt, T, hidden, ffn, E, nl, e0):
    monkeypatch.setenv("FM_MOE_TILE", tile)
    monkeypatch.setenv("FM_SPLIT_TAIL", "0")
    say(f"moe T={T} hidden={hidden} ffn={ffn} E={E} nl={nl} e0={e0} dt={dt} tile={tile}")
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, dt, seed=T + hidden, zipf_s=1.2)
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    Href = oracle.moe_layer0(dt, inp["X"], inp["W1"], rsp, roff, 2)
    Hb = oracle.round_bf16(Href) if dt == BF16 else oracle.round_f16(Href)
    off, sp, H, out = _moe_run(inp, e0, nl, dt, H_in=Hb)
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    assert_close(host64(H[:rows]), Href, "moe layer0 H")
    ref = oracle.moe_layer1(dt, Hb, inp["W2"], inp["topk_ids"], inp["topk_weights"], rsp, roff,
                            inp["out_seed"], e0)
    assert_close(host64(out) - inp["out_seed"], ref - inp["out_seed"], "moe combine")


@pytest.mark.parametrize("act", [1, 2, 3])
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("T,hidden,ffn,tile", [(300, 136, 264, "256x256"), (1500, 256, 520, "256x256w4"),
                                               (700, 192, 136, "128x128")])
def test_moe_layer0_activation(oracle, monkeypatch, act, dt, T, hidden, ffn, tile):
    """fm_moe_gather_gemm_act: H = act(gathered X @ W1[e]) against the
    oracle's layer 0 followed by its activation (ragged rows and columns, a
    K tail, the split last wave of the default tile)."""
    import torch
    import tile_gemm_communication_amd as fm
    monkeypatch.setenv("FM_MOE_TILE", tile)
    E, nl, e0 = 16, 8, 0
    say(f"moe layer0 act={act} T={T} hidden={hidden} ffn={ffn} dt={dt} tile={tile}")
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, dt, seed=T + act, zipf_s=1.2)
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    ref = oracle.activation(act, oracle.moe_layer0(dt, inp["X"], inp["W1"], rsp, roff, 2))
    sp = torch.full((T * 2,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    H = torch.zeros((T * 2, ffn), dtype=torch.float16 if dt == F16 else torch.bfloat16,
                    device="cuda:0")
    fm.fm_moe_gather_gemm_act(dev16(inp["X"], dt), _i32(inp["topk_ids"]), dev16(inp["W1"], dt),
                              H, sp, off, e0, act, fm.moe_workspace(T, 2, hidden, nl))
    torch.cuda.synchronize()
    rows = int(roff[-1])
    assert np.array_equal(off.cpu().numpy(), roff)
    assert_close(host64(H[:rows]), ref, f"layer0 act {act}")


def test_moe_layer0_no_activation_is_plain():
    """FM_ACT_NONE gives the bits of fm_moe_gather_gemm."""
    import torch
    import tile_gemm_communication_amd as fm
    T, hidden, ffn, nl = 900, 256, 264, 8
    inp = wl.moe_inputs(T, hidden, ffn, 16, nl, 2, BF16, seed=5, zipf_s=1.2)
    outs = []
    for fn in ("plain", "act"):
        sp = torch.full((T * 2,), -1, dtype=torch.int32, device="cuda:0")
        off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
        H = torch.zeros((T * 2, ffn), dtype=torch.bfloat16, device="cuda:0")
        args = (dev16(inp["X"], BF16), _i32(inp["topk_ids"]), dev16(inp["W1"], BF16), H, sp, off, 0)
        ws = fm.moe_workspace(T, 2, hidden, nl)
        if fn == "plain":
            fm.fm_moe_gather_gemm(*args, ws)
        else:
            fm.fm_moe_gather_gemm_act(*args, fm.FM_ACT_NONE, ws)
        torch.cuda.synchronize()
        outs.append(bits16(H))
    assert np.array_equal(outs[0], outs[1])


def test_moe_one_hot_expert(oracle):
    """All tokens routed to one local expert with weight 1 (top-1): the layer
    reduces to seed + (X W1) W2 for that expert."""
    T, hidden, ffn = 520, 128, 136
    inp = wl.moe_inputs(T, hidden, ffn, 4, 4, 1, BF16, seed=5)
    inp["topk_ids"] = np.full((T, 1), 2, dtype=np.int32)
    inp["topk_weights"] = np.ones((T, 1), dtype=np.float32)
    roff, rsp = oracle.moe_route(inp["topk_ids"], 0, 4)
    Hb = oracle.round_bf16(oracle.moe_layer0(BF16, inp["X"], inp["W1"], rsp, roff, 1))
    off, sp, H, out = _moe_run(inp, 0, 4, BF16, H_in=Hb)
    ref = oracle.moe_layer1(BF16, Hb, inp["W2"], inp["topk_ids"], inp["topk_weights"], rsp, roff,
                            inp["out_seed"], 0)
    assert_close(host64(out) - inp["out_seed"], ref - inp["out_seed"], "one-hot combine")


_EP8: dict = {}


def _ep8_reference(oracle):
    """EP=8 rank-0 inputs, their routing and every row of layer 0 from the
    oracle's every-element form, built once per process and shared by the
    full-size tests of every layer-0 form."""
    if not _EP8:
        c = wl.MOE_EP8
        inp = wl.moe_inputs(c["T"], c["hidden"], c["ffn"], c["n_experts"], c["n_local"],
                            c["topk"], BF16, seed=c["seed"], zipf_s=c["zipf_s"])
        e0 = c["rank"] * c["n_local"]
        roff, rsp = oracle.moe_route(inp["topk_ids"], e0, c["n_local"])
        say("full moe EP=8: oracle layer 0, every row")
        _EP8.update(inp=inp, e0=e0, roff=roff, rsp=rsp,
                    H=full.moe_layer0(BF16, inp["X"], inp["W1"], rsp, roff, c["topk"]))
    return _EP8


def test_full_moe_rank0(oracle):
    """EP=8 rank 0: 16384 tokens x 4096, 64 experts top-2 (log-Zipf bias), 8
    local experts, ffn 2816, bf16, chained on the GPU: layer 0, then the
    combine on the GPU's own H.  Routing bit-exact; every row of layer 0 and
    every token of the combine against the oracle's every-element forms (the
    combine run on the GPU's H bits); sampled rows of layer 0 and over 512
    tokens of the combine (every token of each expert's first and last row
    tile, at least 100 with both pairs local, random ones) against the
    oracle's loops."""
    import torch
    c = wl.MOE_EP8
    say("full moe EP=8 rank 0")
    ep8 = _ep8_reference(oracle)
    inp, e0, nl = ep8["inp"], ep8["e0"], c["n_local"]
    roff, rsp = ep8["roff"], ep8["rsp"]
    off, sp, H, out = _moe_run(inp, e0, nl, BF16)
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    assert_close(host64(H[:rows]), ep8["H"], "full layer0, every row")
    rng = np.random.default_rng(7)
    srows = np.unique(np.concatenate([rng.integers(0, rows, 48), roff[:-1], roff[1:] - 1]))
    srows = srows[(srows >= 0) & (srows < rows)]
    Hs = oracle.moe_layer0_rows(BF16, inp["X"], inp["W1"], rsp, roff, 2, srows)
    idx = torch.from_numpy(srows).to("cuda:0")
    assert_close(host64(H[idx]), Hs, "full layer0 rows")
    # tokens of every expert's first and last 256-row tile
    edge = []
    for e in range(nl):
        r0, r1 = int(roff[e]), int(roff[e + 1])
        if r1 > r0:
            last0 = r0 + (r1 - r0 - 1) // 256 * 256
            edge.append(rsp[r0:min(r0 + 256, r1)] // 2)
            edge.append(rsp[last0:r1] // 2)
    ids = inp["topk_ids"]
    local = (ids >= e0) & (ids < e0 + nl)
    both = np.nonzero(local.all(axis=1))[0]
    toks = np.unique(np.concatenate(edge + [rng.choice(both, 128, replace=False),
                                            rng.integers(0, c["T"], 64)]))
    assert toks.size >= 512 and np.isin(toks, both).sum() >= 100
    say(f"full moe combine: {toks.size} tokens checked")
    Hbits = H[:rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.moe_layer1_tokens(BF16, Hbits, inp["W2"], ids, inp["topk_weights"], rsp, roff,
                                   inp["out_seed"], e0, toks)
    tidx = torch.from_numpy(toks).to("cuda:0")
    assert_close(host64(out[tidx]) - inp["out_seed"][toks], ref - inp["out_seed"][toks],
                 "full combine tokens")
    want = full.moe_layer1(BF16, Hbits, inp["W2"], ids, inp["topk_weights"], rsp, roff,
                           inp["out_seed"], e0)
    assert_close(host64(out) - inp["out_seed"], want - inp["out_seed"],
                 "full combine, every token")


def test_full_moe_rank0_f16(oracle):
    """The EP=8 rank-0 layer with fp16 inputs: routing bit-exact, every row of
    layer 0 and every token of the combine (run on the GPU's own H) against
    the oracle's every-element forms."""
    import torch
    c = wl.MOE_EP8
    say("full moe EP=8 rank 0, fp16")
    inp = wl.moe_inputs(c["T"], c["hidden"], c["ffn"], c["n_experts"], c["n_local"], c["topk"],
                        F16, seed=c["seed"] + 11, zipf_s=c["zipf_s"])
    e0, nl = c["rank"] * c["n_local"], c["n_local"]
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    off, sp, H, out = _moe_run(inp, e0, nl, F16)
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    assert_close(host64(H[:rows]), full.moe_layer0(F16, inp["X"], inp["W1"], rsp, roff, 2),
                 "full fp16 layer0, every row")
    Hbits = H[:rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    want = full.moe_layer1(F16, Hbits, inp["W2"], inp["topk_ids"], inp["topk_weights"], rsp,
                           roff, inp["out_seed"], e0)
    assert_close(host64(out) - inp["out_seed"], want - inp["out_seed"],
                 "full fp16 combine, every token")


@pytest.mark.parametrize("act", [1, 2, 3])
def test_full_moe_layer0_activation(oracle, act):
    """EP=8 rank 0 layer 0 with the fused activation (ReLU, tanh-form GELU,
    SiLU): every row against the oracle's every-element layer 0 followed by
    its activation."""
    import torch
    import tile_gemm_communication_amd as fm
    c = wl.MOE_EP8
    say(f"full moe layer0 EP=8 rank 0, act={act}")
    ep8 = _ep8_reference(oracle)
    inp, e0, nl, T = ep8["inp"], ep8["e0"], c["n_local"], c["T"]
    roff = ep8["roff"]
    rows = int(roff[-1])
    sp = torch.full((T * 2,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    H = torch.zeros((T * 2, c["ffn"]), dtype=torch.bfloat16, device="cuda:0")
    fm.fm_moe_gather_gemm_act(dev16(inp["X"], BF16), _i32(inp["topk_ids"]),
                              dev16(inp["W1"], BF16), H, sp, off, e0, act,
                              fm.moe_workspace(T, 2, c["hidden"], nl))
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), roff)
    assert_close(host64(H[:rows]), oracle.activation(act, ep8["H"]),
                 f"full layer0 act {act}, every row")


@pytest.mark.parametrize("T,hidden,ffn,E,nl,topk", [(4096, 1024, 512, 16, 8, 2),
                                                    (1500, 392, 200, 8, 8, 4)])
def test_moe_combine_deterministic(oracle, T, hidden, ffn, E, nl, topk):
    """The combine applies a token's local contributions in expert order
    without atomics: repeated calls give identical bits, also when every
    token has up to four local pairs, and the result meets the parity bar."""
    import torch
    import tile_gemm_communication_amd as fm
    say(f"moe combine determinism T={T} hidden={hidden} ffn={ffn} topk={topk}")
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, topk, BF16, seed=T + topk, zipf_s=1.2)
    roff, rsp = oracle.moe_route(inp["topk_ids"], 0, nl)
    Hb = oracle.round_bf16(oracle.moe_layer0(BF16, inp["X"], inp["W1"], rsp, roff, topk))
    rows = int(roff[-1])
    Hd = torch.zeros((T * topk, ffn), dtype=torch.bfloat16, device="cuda:0")
    Hd[:rows] = dev16(Hb, BF16)
    sp = torch.full((T * topk,), -1, dtype=torch.int32, device="cuda:0")
    sp[:rows] = _i32(rsp)
    off = _i32(roff)
    W2 = dev16(inp["W2"], BF16)
    wts = devf32(inp["topk_weights"])
    outs = []
    ws = fm.moe_workspace(T, topk, hidden, nl)
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for _ in range(3):
        out = devf32(inp["out_seed"])
        fm.fm_moe_gemm_scatter(Hd, W2, sp, off, wts, out, ws, err_word=err)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert err.item() == 0
    assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])
    ref = oracle.moe_layer1(BF16, Hb, inp["W2"], inp["topk_ids"], inp["topk_weights"], rsp, roff,
                            inp["out_seed"], 0)
    assert_close(outs[0].astype(np.float64) - inp["out_seed"], ref - inp["out_seed"],
                 "deterministic combine")


@pytest.mark.parametrize("T,ffn", [(20000, 504), (600, 264), (9000, 256)])
def test_moe_gather_split_tail(oracle, monkeypatch, T, ffn):
    """Layer 0 runs a half-empty last wave of 256x256 tiles as 256x128 halves
    (a second launch).  Each H element is still summed over K by one
    workgroup in the same order, so H is bit-identical to the unsplit run,
    and every row of H meets the parity bar.  Shapes: about 330 tiles (one
    full wave plus a tail) with a ragged last column, a few tiles only
    (halves alone), and a tail of about a third of a wave."""
    import torch
    import tile_gemm_communication_amd as fm
    hidden, E, nl = 64, 8, 8
    say(f"moe split tail T={T} ffn={ffn}")
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=T + ffn, zipf_s=1.2)
    roff, rsp = oracle.moe_route(inp["topk_ids"], 0, nl)
    rows = int(roff[-1])
    X, W1, ids = dev16(inp["X"], BF16), dev16(inp["W1"], BF16), _i32(inp["topk_ids"])
    ws = fm.moe_workspace(T, 2, hidden, nl)
    outs = {}
    for mode, env in (("halves", "1"), ("none", "0")):
        monkeypatch.setenv("FM_SPLIT_TAIL", env)
        H = torch.zeros((T * 2, ffn), dtype=torch.bfloat16, device="cuda:0")
        sp = torch.full((T * 2,), -1, dtype=torch.int32, device="cuda:0")
        off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
        fm.fm_moe_gather_gemm(X, ids, W1, H, sp, off, 0, ws)
        torch.cuda.synchronize()
        outs[mode] = H
    assert torch.equal(outs["halves"].view(torch.int16), outs["none"].view(torch.int16))
    Href = oracle.moe_layer0(BF16, inp["X"], inp["W1"], rsp, roff, 2)
    assert_close(host64(outs["halves"][:rows]), Href, "layer0 split tail")


@pytest.mark.parametrize("act", [1, 2])
def test_moe_gather_split_tail_activation(oracle, act):
    """The split tail with an activation: the 256x128 halves apply it in
    their epilogue as the full tiles do (T = 9000 gives a tail of about a
    third of a wave)."""
    import torch
    import tile_gemm_communication_amd as fm
    T, hidden, ffn, E, nl = 9000, 128, 256, 8, 8
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=T + act, zipf_s=1.2)
    roff, rsp = oracle.moe_route(inp["topk_ids"], 0, nl)
    rows = int(roff[-1])
    ref = oracle.activation(act, oracle.moe_layer0(BF16, inp["X"], inp["W1"], rsp, roff, 2))
    H = torch.zeros((T * 2, ffn), dtype=torch.bfloat16, device="cuda:0")
    sp = torch.full((T * 2,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm_act(dev16(inp["X"], BF16), _i32(inp["topk_ids"]),
                              dev16(inp["W1"], BF16), H, sp, off, 0, act,
                              fm.moe_workspace(T, 2, hidden, nl))
    torch.cuda.synchronize()
    assert_close(host64(H[:rows]), ref, f"split tail act {act}")


@pytest.mark.parametrize("T,hidden,ffn", [(0, 64, 32), (300, 64, 0), (300, 0, 40)])
def test_moe_empty_sizes(oracle, T, hidden, ffn):
    """Degenerate sizes against the oracle: no tokens (the route writes zero
    offsets, nothing else runs); ffn = 0 (H has no columns, each local pair
    adds weight x 0 to out); hidden = 0 (layer 0 sums over an empty K: the
    local rows of H become 0, and the combine has no columns to add)."""
    import torch
    import tile_gemm_communication_amd as fm
    E, nl, e0, topk = 16, 8, 4, 2
    say(f"moe empty sizes T={T} hidden={hidden} ffn={ffn}")
    inp = wl.moe_inputs(max(T, 1), max(hidden, 8), max(ffn, 8), E, nl, topk, BF16, seed=91)
    ids = inp["topk_ids"][:T]
    X = torch.zeros((T, hidden), dtype=torch.bfloat16, device="cuda:0")
    if T and hidden:
        X.copy_(dev16(inp["X"][:T, :hidden], BF16))
    W1 = torch.randn(nl, hidden, ffn, device="cuda:0").to(torch.bfloat16)
    W2 = torch.randn(nl, ffn, hidden, device="cuda:0").to(torch.bfloat16)
    H = torch.full((T * topk, ffn), 7.0, dtype=torch.bfloat16, device="cuda:0")
    sp = torch.full((T * topk,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.full((nl + 1,), -5, dtype=torch.int32, device="cuda:0")
    ws = fm.moe_workspace(T, topk, hidden, nl)
    fm.fm_moe_gather_gemm(X, _i32(ids), W1, H, sp, off, e0, ws)
    seed = inp["out_seed"][:T, :hidden].astype(np.float32)
    out = torch.from_numpy(np.ascontiguousarray(seed)).to("cuda:0")
    wts = torch.from_numpy(np.ascontiguousarray(inp["topk_weights"][:T])).to("cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gemm_scatter(H, W2, sp, off, wts, out, ws, err_word=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    roff, rsp = oracle.moe_route(ids.reshape(T, topk), e0, nl)
    assert np.array_equal(off.cpu().numpy(), roff)
    rows = int(roff[-1])
    assert np.array_equal(sp.cpu().numpy()[:rows], rsp)
    if T == 0:
        return
    if hidden == 0:   # layer 0's local rows are 0, the rest of H untouched
        assert torch.count_nonzero(H[:rows]).item() == 0
        assert bool((H[rows:] == 7.0).all())
        return
    # ffn = 0: out = seed + (weight x 0) for the local pairs, as the oracle
    Hb = np.zeros((rows, 0), dtype=np.uint16)
    W2b = np.zeros((nl, 0, hidden), dtype=np.uint16)
    ref = oracle.moe_layer1(BF16, Hb, W2b, ids, inp["topk_weights"][:T], rsp, roff, seed, e0)
    assert np.array_equal(host64(out), ref)


def test_moe_nothing_local_leaves_buffers():
    """No pair routed to this rank's experts: every local expert is empty, H
    keeps its contents and the combine adds nothing."""
    import torch
    import tile_gemm_communication_amd as fm
    T, hidden, ffn, nl = 300, 128, 64, 4
    inp = wl.moe_inputs(T, hidden, ffn, 16, nl, 2, BF16, seed=11)
    ids = np.full((T, 2), 12, dtype=np.int32)            # experts 12, never local (0..3)
    H = torch.full((T * 2, ffn), 7.0, dtype=torch.bfloat16, device="cuda:0")
    sp = torch.full((T * 2,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.full((nl + 1,), 99, dtype=torch.int32, device="cuda:0")
    out = devf32(inp["out_seed"])
    ws = fm.moe_workspace(T, 2, hidden, nl)
    fm.fm_moe_gather_gemm(dev16(inp["X"], BF16), _i32(ids), dev16(inp["W1"], BF16), H, sp, off, 0,
                          ws)
    fm.fm_moe_gemm_scatter(H, dev16(inp["W2"], BF16), sp, off, devf32(inp["topk_weights"]), out,
                           ws)
    torch.cuda.synchronize()
    assert off.cpu().numpy().tolist() == [0] * (nl + 1)
    assert bool((H.float() == 7.0).all()) and bool((sp == -1).all())
    assert np.array_equal(out.cpu().numpy(), inp["out_seed"])


@pytest.mark.parametrize("topk,nl,e0", [(1, 1, 3), (4, 64, 0)])
def test_moe_extreme_expert_counts(oracle, topk, nl, e0):
    """One local expert with top-1 routing, and 64 local experts with top-4
    (up to four ordered contributions per token)."""
    T, hidden, ffn = 700, 192, 136
    E = max(nl + e0, 8)
    say(f"moe topk={topk} n_local={nl} e0={e0}")
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, topk, BF16, seed=T + topk, zipf_s=0.6)
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    Href = oracle.moe_layer0(BF16, inp["X"], inp["W1"], rsp, roff, topk)
    Hb = oracle.round_bf16(Href)
    off, sp, H, out = _moe_run(inp, e0, nl, BF16, H_in=Hb)
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    assert_close(host64(H[:rows]), Href, "layer0 H")
    ref = oracle.moe_layer1(BF16, Hb, inp["W2"], inp["topk_ids"], inp["topk_weights"], rsp, roff,
                            inp["out_seed"], e0)
    assert_close(host64(out) - inp["out_seed"], ref - inp["out_seed"], "combine")


def _moe_ag_run(arr, inp, e0, nl, order, epoch, dt=BF16, spin=0, hint=None, **push_kw):
    """Token chunks pushed by the side stream (Arrival) while the fused
    AllGather + gather-GEMM runs; returns (off, sp, H)."""
    import torch
    import tile_gemm_communication_amd as fm
    ids = inp["topk_ids"]
    T, topk = ids.shape
    ffn = inp["W1"].shape[2]
    H = torch.zeros((T * topk, ffn), dtype=torch.float16 if dt == F16 else torch.bfloat16,
                    device="cuda:0")
    sp = torch.full((T * topk,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    arr.err.zero_()
    arr.push(order, epoch, **push_kw)
    hidden = inp["X"].shape[1]
    fm.fm_moe_ag_gather_gemm(arr.X, _i32(ids), dev16(inp["W1"], dt), H, sp, off, e0, arr.flags,
                             epoch, arr.n, fm.moe_workspace(T, topk, hidden, nl), order=hint,
                             err_word=arr.err, spin_limit=spin)
    arr.join()
    torch.cuda.synchronize()
    return off.cpu().numpy(), sp.cpu().numpy(), H


@pytest.mark.parametrize("T,n,delay,hint", [(1024, 4, 0, "none"), (3000, 8, 3_000_000, "same"),
                                            (4096, 8, 1_000_000, "reversed"),
                                            (2048, 2, 0, "same")])
def test_moe_ag_gather_random_arrival(oracle, monkeypatch, T, n, delay, hint):
    """Token chunks arriving in a seeded random order (optionally late), with
    the arrival hint absent, right or wrong: the fused layer 0 equals the
    oracle on the gathered tokens and reproduces fm_moe_gather_gemm on the
    gathered buffer bit for bit."""
    import torch
    import tile_gemm_communication_amd as fm
    from gpu_util import Arrival
    hidden, ffn, E, nl, e0 = 256, 264, 16, 8, 0
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=T + n, zipf_s=1.2)
    chunks = inp["X"].reshape(n, T // n, hidden)
    order = wl.permutation(n, seed=T)
    hint_order = {"none": None, "same": order.tolist(), "reversed": order.tolist()[::-1]}[hint]
    if T == 2048:
        monkeypatch.setenv("FM_MOE_AG_GROUP", "1")   # one band per M-tile
    say(f"moe ag T={T} chunks={n} order={order.tolist()} delay={delay} hint={hint}")
    arr = Arrival(chunks, BF16, hidden)
    arr.poison()
    off, sp, H = _moe_ag_run(arr, inp, e0, nl, order, arr.next_epoch(), hint=hint_order,
                             delay_cycles=delay)
    assert arr.err.item() == 0
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    ref = oracle.moe_ag_layer0(BF16, list(chunks), inp["W1"], rsp, roff, 2, arrival=order)
    assert_close(host64(H[:rows]), ref, "moe ag layer0")
    H2 = torch.zeros_like(H)
    sp2 = torch.full_like(torch.from_numpy(sp).to("cuda:0"), -1)
    off2 = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm(arr.X, _i32(inp["topk_ids"]), dev16(inp["W1"], BF16), H2, sp2, off2,
                          e0, fm.moe_workspace(T, 2, hidden, nl))
    torch.cuda.synchronize()
    assert torch.equal(H[:rows].view(torch.int16), H2[:rows].view(torch.int16))


@pytest.mark.parametrize("T,n,topk,nl,e0", [(640, 1, 2, 8, 0), (1200, 4, 4, 16, 16)])
def test_moe_ag_f16_layouts(oracle, T, n, topk, nl, e0):
    """fp16, a single chunk (nothing to gather but the local one) and top-4
    over 16 local experts: routing bit-exact, H within the bar of the oracle
    and bit-identical to the non-fused layer 0."""
    import torch
    import tile_gemm_communication_amd as fm
    from gpu_util import Arrival
    hidden, ffn, E = 192, 136, 64
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, topk, F16, seed=T + topk)
    chunks = inp["X"].reshape(n, T // n, hidden)
    order = list(range(n))
    say(f"moe ag fp16 T={T} chunks={n} topk={topk} experts {e0}..{e0 + nl - 1}")
    arr = Arrival(chunks, F16, hidden)
    arr.poison()
    off, sp, H = _moe_ag_run(arr, inp, e0, nl, order, arr.next_epoch(), dt=F16, local=0)
    assert arr.err.item() == 0
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    ref = oracle.moe_ag_layer0(F16, list(chunks), inp["W1"], rsp, roff, topk, arrival=order)
    assert_close(host64(H[:rows]), ref, "moe ag fp16")
    H2 = torch.zeros_like(H)
    sp2 = torch.full((T * topk,), -1, dtype=torch.int32, device="cuda:0")
    off2 = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm(arr.X, _i32(inp["topk_ids"]), dev16(inp["W1"], F16), H2, sp2, off2, e0,
                          fm.moe_workspace(T, topk, hidden, nl))
    torch.cuda.synchronize()
    assert torch.equal(H[:rows].view(torch.int16), H2[:rows].view(torch.int16))


def test_moe_ag_nothing_local_waits_for_nothing():
    """No pair is routed to this rank: no tile exists, so no chunk is waited
    for (none is ever pushed) and the call neither times out nor writes H."""
    import torch
    from gpu_util import Arrival
    T, hidden, ffn, nl, n = 512, 128, 64, 4, 4
    inp = wl.moe_inputs(T, hidden, ffn, 16, nl, 2, BF16, seed=12)
    inp["topk_ids"] = np.full((T, 2), 12, dtype=np.int32)
    arr = Arrival(inp["X"].reshape(n, T // n, hidden), BF16, hidden)
    off, sp, H = _moe_ag_run(arr, inp, 0, nl, list(range(n)), arr.next_epoch(), spin=2000,
                             skip=tuple(range(n)))
    assert arr.err.item() == 0
    assert off.tolist() == [0] * (nl + 1) and bool((sp == -1).all())
    assert torch.count_nonzero(H).item() == 0


def test_moe_layer_end_to_end(oracle):
    """A whole MoE layer on one rank, each stage fed by the previous one on the
    GPU: token AllGather (8 chunks, seeded random arrival) into layer 0, then
    layer 1 with the weighted combine on the GPU's own H.  Compared with the
    oracle's chain (layer 0, H rounded to bf16, layer 1) on the delta of out."""
    import torch
    import tile_gemm_communication_amd as fm
    from gpu_util import Arrival
    T, hidden, ffn, E, nl, e0, n = 4096, 384, 264, 32, 8, 8, 8
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=4242, zipf_s=1.2)
    chunks = inp["X"].reshape(n, T // n, hidden)
    order = wl.permutation(n, seed=4243)
    say(f"moe layer end to end T={T} experts {e0}..{e0 + nl - 1} order={order.tolist()}")
    arr = Arrival(chunks, BF16, hidden)
    arr.poison()
    off, sp, H = _moe_ag_run(arr, inp, e0, nl, order, arr.next_epoch(), hint=order.tolist())
    assert arr.err.item() == 0
    out = devf32(inp["out_seed"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gemm_scatter(H, dev16(inp["W2"], BF16), _i32(sp), _i32(off),
                           devf32(inp["topk_weights"]), out, fm.moe_workspace(T, 2, hidden, nl),
                           err_word=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    assert np.array_equal(off, roff)
    Href = oracle.moe_ag_layer0(BF16, list(chunks), inp["W1"], rsp, roff, 2, arrival=order)
    ref = oracle.moe_layer1(BF16, oracle.round_bf16(Href), inp["W2"], inp["topk_ids"],
                            inp["topk_weights"], rsp, roff, inp["out_seed"], e0)
    assert_close(host64(out) - inp["out_seed"], ref - inp["out_seed"], "moe layer end to end")


def _moe_prod_run(inp, chunks, e0, nl, order, local, n_prod, dt=BF16, counters=None):
    """fm_moe_ag_gather_gemm_producers with sources for every chunk not in
    `local`; returns (off, sp, H, X)."""
    import torch
    import tile_gemm_communication_amd as fm
    n, Tc, hidden = chunks.shape
    T = n * Tc
    topk = inp["topk_ids"].shape[1]
    ffn = inp["W1"].shape[2]
    src = [None if c in local else dev16(chunks[c], dt) for c in range(n)]
    X = torch.full((T, hidden), float("nan"), dtype=torch.bfloat16 if dt == BF16
                   else torch.float16, device="cuda:0")
    for c in local:
        X[c * Tc:(c + 1) * Tc].copy_(dev16(chunks[c], dt))
    H = torch.zeros((T * topk, ffn), dtype=X.dtype, device="cuda:0")
    sp = torch.full((T * topk,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    flags = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    if counters is None:
        counters = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_ag_gather_gemm_producers(src, X, _i32(inp["topk_ids"]), dev16(inp["W1"], dt), H,
                                       sp, off, e0, flags, counters, 7,
                                       fm.moe_workspace(T, topk, hidden, nl), order=order,
                                       n_producers=n_prod, err_word=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.all(flags == 7).item() and torch.count_nonzero(counters).item() == 0
    return off.cpu().numpy(), sp.cpu().numpy(), H, X


@pytest.mark.parametrize("T,n,n_prod,local", [(3000, 8, 8, (0,)), (2048, 4, 16, ()),
                                              (1000, 2, 64, (0, 1))])
def test_moe_ag_producers(oracle, T, n, n_prod, local):
    """Producer workgroups of layer 0's own launch copy the token chunks in a
    seeded random order: X holds the gathered tokens, H equals the oracle and
    fm_moe_gather_gemm on the gathered X bit for bit."""
    import torch
    import tile_gemm_communication_amd as fm
    hidden, ffn, E, nl, e0 = 256, 264, 16, 8, 0
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=T + 7 * n, zipf_s=1.2)
    chunks = inp["X"].reshape(n, T // n, hidden)
    order = wl.permutation(n, seed=T + 1).tolist()
    say(f"moe ag producers T={T} chunks={n} P={n_prod} local={local} order={order}")
    off, sp, H, X = _moe_prod_run(inp, chunks, e0, nl, order, local, n_prod)
    assert np.array_equal(bits16(X), inp["X"])
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    ref = oracle.moe_ag_layer0(BF16, list(chunks), inp["W1"], rsp, roff, 2, arrival=order)
    assert_close(host64(H[:rows]), ref, "moe ag producers")
    H2 = torch.zeros_like(H)
    sp2 = torch.full_like(H2[:, 0], 0, dtype=torch.int32)
    off2 = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm(X, _i32(inp["topk_ids"]), dev16(inp["W1"], BF16), H2, sp2, off2, e0,
                          fm.moe_workspace(T, 2, hidden, nl))
    torch.cuda.synchronize()
    assert torch.equal(H[:rows].view(torch.int16), H2[:rows].view(torch.int16))


def test_full_moe_ag_producers_rank0(oracle):
    """EP=8 rank 0 with the default producer count, the local chunk in place
    and seven copied: every row against the oracle's every-element form,
    sampled rows against its loops, bit-identical to the non-fused layer 0,
    and a second call on the same counters."""
    import torch
    import tile_gemm_communication_amd as fm
    c = wl.MOE_EP8
    say("full moe ag producers EP=8 rank 0")
    inp = wl.moe_inputs(c["T"], c["hidden"], c["ffn"], c["n_experts"], c["n_local"], c["topk"],
                        BF16, seed=c["seed"], zipf_s=c["zipf_s"])
    e0, n = c["rank"] * c["n_local"], 8
    chunks = inp["X"].reshape(n, c["T"] // n, c["hidden"])
    counters = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    off, sp, H, X = _moe_prod_run(inp, chunks, e0, c["n_local"], list(range(n)), (0,), 0,
                                  counters=counters)
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, c["n_local"])
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    rng = np.random.default_rng(10)
    srows = np.unique(np.concatenate([rng.integers(0, rows, 48), roff[:-1], roff[1:] - 1]))
    srows = srows[(srows >= 0) & (srows < rows)]
    Hs = oracle.moe_layer0_rows(BF16, inp["X"], inp["W1"], rsp, roff, 2, srows)
    idx = torch.from_numpy(srows).to("cuda:0")
    assert_close(host64(H[idx]), Hs, "full moe ag producers rows")
    assert_close(host64(H[:rows]), _ep8_reference(oracle)["H"],
                 "full moe ag producers, every row")
    H2 = torch.zeros_like(H)
    sp2 = torch.full((c["T"] * 2,), -1, dtype=torch.int32, device="cuda:0")
    off2 = torch.zeros(c["n_local"] + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm(X, _i32(inp["topk_ids"]), dev16(inp["W1"], BF16), H2, sp2, off2, e0,
                          fm.moe_workspace(c["T"], 2, c["hidden"], c["n_local"]))
    torch.cuda.synchronize()
    assert torch.equal(H[:rows].view(torch.int16), H2[:rows].view(torch.int16))
    _, _, H3, _ = _moe_prod_run(inp, chunks, e0, c["n_local"], list(range(n)), (0,), 0,
                                counters=counters)
    assert torch.equal(H3[:rows].view(torch.int16), H[:rows].view(torch.int16))


def _moe_pull_run(inp, chunks, e0, nl, order, times_ns, dt=BF16, spin=0, signal=None):
    """fm_moe_ag_gather_gemm_pull with the chunk flags published by
    fm_chunk_signal_paced on a side stream (signal: the chunks published, in
    that order; default `order`); returns (off, sp, H, err)."""
    import torch
    import tile_gemm_communication_amd as fm
    n, Tc, hidden = chunks.shape
    T = n * Tc
    topk = inp["topk_ids"].shape[1]
    ffn = inp["W1"].shape[2]
    src = [dev16(chunks[c], dt) for c in range(n)]
    H = torch.zeros((T * topk, ffn), dtype=src[0].dtype, device="cuda:0")
    sp = torch.full((T * topk,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    flags = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    side = side_stream()
    cs = torch.cuda.current_stream()
    side.wait_stream(cs)
    fm.fm_chunk_signal_paced(flags, times_ns, 5, order=order if signal is None else signal,
                             stream=side)
    fm.fm_moe_ag_gather_gemm_pull(src, _i32(inp["topk_ids"]), dev16(inp["W1"], dt), H, sp, off,
                                  e0, flags, 5, fm.moe_workspace(T, topk, hidden, nl),
                                  order=order, err_word=err, spin_limit=spin)
    cs.wait_stream(side)
    torch.cuda.synchronize()
    return off.cpu().numpy(), sp.cpu().numpy(), H, err.item()


@pytest.mark.parametrize("T,n,gap_us", [(3000, 8, 20), (2048, 4, 0), (1000, 1, 0)])
def test_moe_ag_pull(oracle, T, n, gap_us):
    """Token rows read in place from per-owner chunk buffers, signalled in a
    seeded random order: H equals the oracle and fm_moe_gather_gemm on the
    concatenated tokens bit for bit."""
    import torch
    import tile_gemm_communication_amd as fm
    hidden, ffn, E, nl, e0 = 256, 264, 16, 8, 8
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=T + 11 * n, zipf_s=1.2)
    chunks = inp["X"].reshape(n, T // n, hidden)
    order = wl.permutation(n, seed=T + 3).tolist()
    say(f"moe ag pull T={T} chunks={n} order={order} gap={gap_us} us")
    off, sp, H, err = _moe_pull_run(inp, chunks, e0, nl, order,
                                    [a * gap_us * 1000 for a in range(n)])
    assert err == 0
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    ref = oracle.moe_ag_layer0(BF16, list(chunks), inp["W1"], rsp, roff, 2, arrival=order)
    assert_close(host64(H[:rows]), ref, "moe ag pull")
    H2 = torch.zeros_like(H)
    sp2 = torch.full((T * 2,), -1, dtype=torch.int32, device="cuda:0")
    off2 = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm(dev16(inp["X"], BF16), _i32(inp["topk_ids"]), dev16(inp["W1"], BF16),
                          H2, sp2, off2, e0, fm.moe_workspace(T, 2, hidden, nl))
    torch.cuda.synchronize()
    assert torch.equal(H[:rows].view(torch.int16), H2[:rows].view(torch.int16))


def test_moe_ag_pull_and_producers_fp16_nothing_local(oracle):
    """fp16 through both forms, then a routing with no local pair: the pull
    form reads nothing and the producer form still gathers X and publishes
    every flag, with no tile to run."""
    import torch
    T, hidden, ffn, E, nl, e0, n = 1536, 192, 136, 32, 8, 8, 4
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, F16, seed=31, zipf_s=1.2)
    chunks = inp["X"].reshape(n, T // n, hidden)
    order = [2, 0, 3, 1]
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
    rows = int(roff[-1])
    ref = oracle.moe_ag_layer0(F16, list(chunks), inp["W1"], rsp, roff, 2, arrival=order)
    off, sp, H, err = _moe_pull_run(inp, chunks, e0, nl, order, [0, 5000, 10000, 15000], dt=F16)
    assert err == 0 and np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    assert_close(host64(H[:rows]), ref, "moe ag pull fp16")
    off2, sp2, H2, X2 = _moe_prod_run(inp, chunks, e0, nl, order, (0,), 8, dt=F16)
    assert np.array_equal(off2, roff) and np.array_equal(bits16(X2), inp["X"])
    assert torch.equal(H2[:rows].view(torch.int16), H[:rows].view(torch.int16))
    # nothing local
    inp["topk_ids"] = np.full((T, 2), 0, dtype=np.int32)
    off, sp, H, err = _moe_pull_run(inp, chunks, e0, nl, order, [0, 0, 0, 0], dt=F16, spin=2000)
    assert err == 0 and off.tolist() == [0] * (nl + 1)
    assert torch.count_nonzero(H).item() == 0
    off2, sp2, H2, X2 = _moe_prod_run(inp, chunks, e0, nl, order, (), 8, dt=F16)
    assert off2.tolist() == [0] * (nl + 1) and np.array_equal(bits16(X2), inp["X"])


def test_moe_ag_pull_withheld_chunk_times_out():
    """Chunk 3 is never signalled: the bounded wait reports FM_ERR_TIMEOUT."""
    import tile_gemm_communication_amd as fm
    T, hidden, ffn, n = 512, 128, 64, 4
    inp = wl.moe_inputs(T, hidden, ffn, 8, 8, 2, BF16, seed=13)
    chunks = inp["X"].reshape(n, T // n, hidden)
    _, _, _, err = _moe_pull_run(inp, chunks, 0, 8, [0, 1, 2, 3], [0, 0, 0], spin=2000,
                                 signal=[0, 1, 2])
    assert err == fm.FM_ERR_TIMEOUT


def test_full_moe_ag_pull_link_paced(oracle):
    """EP=8 rank 0 reading the 8 owners' 2048-token chunks in place, signalled
    in ring order at the one-link rate (16 MiB at 153 GB/s apart): every row
    against the oracle's every-element form, sampled rows against its loops,
    bit-identical to the non-fused layer 0."""
    import torch
    import tile_gemm_communication_amd as fm
    c = wl.MOE_EP8
    say("full moe ag pull EP=8 rank 0, link-paced")
    inp = wl.moe_inputs(c["T"], c["hidden"], c["ffn"], c["n_experts"], c["n_local"], c["topk"],
                        BF16, seed=c["seed"], zipf_s=c["zipf_s"])
    e0, n = c["rank"] * c["n_local"], 8
    chunks = inp["X"].reshape(n, c["T"] // n, c["hidden"])
    step = int(chunks[0].size * 2 / 153e9 * 1e9)
    off, sp, H, err = _moe_pull_run(inp, chunks, e0, c["n_local"], list(range(n)),
                                    [a * step for a in range(n)])
    assert err == 0
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, c["n_local"])
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    rng = np.random.default_rng(11)
    srows = np.unique(np.concatenate([rng.integers(0, rows, 48), roff[:-1], roff[1:] - 1]))
    srows = srows[(srows >= 0) & (srows < rows)]
    Hs = oracle.moe_layer0_rows(BF16, inp["X"], inp["W1"], rsp, roff, 2, srows)
    idx = torch.from_numpy(srows).to("cuda:0")
    assert_close(host64(H[idx]), Hs, "full moe ag pull rows")
    assert_close(host64(H[:rows]), _ep8_reference(oracle)["H"], "full moe ag pull, every row")
    H2 = torch.zeros_like(H)
    sp2 = torch.full((c["T"] * 2,), -1, dtype=torch.int32, device="cuda:0")
    off2 = torch.zeros(c["n_local"] + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm(dev16(inp["X"], BF16), _i32(inp["topk_ids"]), dev16(inp["W1"], BF16),
                          H2, sp2, off2, e0, fm.moe_workspace(c["T"], 2, c["hidden"], c["n_local"]))
    torch.cuda.synchronize()
    assert torch.equal(H[:rows].view(torch.int16), H2[:rows].view(torch.int16))


@pytest.mark.parametrize("P", [2, 4])
def test_full_moe_ag_pull_link_parts(oracle, P):
    """EP=8 rank 0 reading the 8 owners' chunks in place, each signalled as P
    token blocks (4 is the benchmark's default), block q once (q+1)/P of the
    chunk has crossed its link (direct schedule), the bands ordered by that
    arrival: routing bit-exact and every row against the oracle's
    every-element form."""
    c = wl.MOE_EP8
    n = 8
    say(f"full moe ag pull EP=8 rank 0, {P} link blocks per chunk")
    ep8 = _ep8_reference(oracle)
    inp, e0 = ep8["inp"], ep8["e0"]
    blocks = inp["X"].reshape(n * P, c["T"] // (n * P), c["hidden"])
    t_link = int(blocks[0].size * 2 * P / 153e9 * 1e9)
    times = {ch * P + q: 0 if ch == 0 else (q + 1) * t_link // P
             for ch in range(n) for q in range(P)}
    seq = sorted(times, key=lambda i: (times[i], i))
    off, sp, H, err = _moe_pull_run(inp, blocks, e0, c["n_local"], seq, [times[i] for i in seq])
    assert err == 0
    roff, rsp = ep8["roff"], ep8["rsp"]
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    assert_close(host64(H[:rows]), ep8["H"], "full moe ag pull blocks, every row")

def test_moe_ag_withheld_chunk_times_out():
    """A token chunk that never arrives: the bounded wait writes
    FM_ERR_TIMEOUT to err_word and the kernel exits (no hang)."""
    import tile_gemm_communication_amd as fm
    from gpu_util import Arrival
    T, hidden, ffn, n = 512, 128, 64, 4
    inp = wl.moe_inputs(T, hidden, ffn, 8, 8, 2, BF16, seed=5)
    arr = Arrival(inp["X"].reshape(n, T // n, hidden), BF16, hidden)
    _moe_ag_run(arr, inp, 0, 8, [0, 1, 2, 3], arr.next_epoch(), spin=2000, skip=(2,))
    assert arr.err.item() == fm.FM_ERR_TIMEOUT


def test_full_moe_ag_rank0(oracle):
    """EP=8 rank 0 with the 16384 tokens gathered from 8 ranks (2048 each,
    the local chunk first, then ring order): routing bit-exact, every row
    against the oracle's every-element form, sampled rows against its loops,
    and bit-identical to the non-fused layer 0."""
    import torch
    import tile_gemm_communication_amd as fm
    from gpu_util import Arrival
    c = wl.MOE_EP8
    say("full moe ag EP=8 rank 0")
    inp = wl.moe_inputs(c["T"], c["hidden"], c["ffn"], c["n_experts"], c["n_local"], c["topk"],
                        BF16, seed=c["seed"], zipf_s=c["zipf_s"])
    e0, n = c["rank"] * c["n_local"], 8
    chunks = inp["X"].reshape(n, c["T"] // n, c["hidden"])
    arr = Arrival(chunks, BF16, c["hidden"])
    arr.poison()
    order = list(range(n))
    off, sp, H = _moe_ag_run(arr, inp, e0, c["n_local"], order, arr.next_epoch(), local=0)
    assert arr.err.item() == 0
    roff, rsp = oracle.moe_route(inp["topk_ids"], e0, c["n_local"])
    rows = int(roff[-1])
    assert np.array_equal(off, roff) and np.array_equal(sp[:rows], rsp)
    rng = np.random.default_rng(9)
    srows = np.unique(np.concatenate([rng.integers(0, rows, 48), roff[:-1], roff[1:] - 1]))
    srows = srows[(srows >= 0) & (srows < rows)]
    Hs = oracle.moe_layer0_rows(BF16, inp["X"], inp["W1"], rsp, roff, 2, srows)
    idx = torch.from_numpy(srows).to("cuda:0")
    assert_close(host64(H[idx]), Hs, "full moe ag rows")
    assert_close(host64(H[:rows]), _ep8_reference(oracle)["H"], "full moe ag, every row")
    H2 = torch.zeros_like(H)
    sp2 = torch.full((c["T"] * 2,), -1, dtype=torch.int32, device="cuda:0")
    off2 = torch.zeros(c["n_local"] + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm(arr.X, _i32(inp["topk_ids"]), dev16(inp["W1"], BF16), H2, sp2, off2,
                          e0, fm.moe_workspace(c["T"], 2, c["hidden"], c["n_local"]))
    torch.cuda.synchronize()
    assert torch.equal(H[:rows].view(torch.int16), H2[:rows].view(torch.int16))

