"""Out-of-bounds guards for the read-modify-write and gathered epilogues:
each destination lives inside a larger allocation whose surrounding words
hold a sentinel, and ragged shapes (rows and columns that end inside a tile)
must leave every sentinel untouched.  Lanes past the last row or column are
sent to the library's own sink, never to the caller's memory."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import BF16, F16, dev16, devf32, say

pytestmark = pytest.mark.gpu
GUARD = 4096          # sentinel words on each side


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _guarded(n_words, dtype, sentinel):
    """A tensor of n_words inside a sentinel-filled buffer; returns (big, view)."""
    import torch
    big = torch.full((n_words + 2 * GUARD,), sentinel, dtype=dtype, device="cuda:0")
    return big, big[GUARD:GUARD + n_words]


def _guards_intact(big, n_words, sentinel):
    head = big[:GUARD].cpu().numpy()
    tail = big[GUARD + n_words:].cpu().numpy()
    return bool((head == sentinel).all() and (tail == sentinel).all())


@pytest.mark.parametrize("T,hidden,ffn,tile", [(700, 200, 136, "256x256"), (1100, 328, 264, "256x256w8"),
                                               (300, 72, 520, "128x128"), (9000, 128, 200, "256x256"),
                                               (2000, 328, 256, "256x256"), (1500, 200, 192, "128x128")])
def test_moe_epilogues_stay_in_bounds(monkeypatch, T, hidden, ffn, tile):
    """Layer 0's H stores and the combine's out read-modify-writes stay in
    their buffers (sentinels on both sides).  A ragged K runs the tail
    kernels (the combine's LDS-DMA epilogue); K a multiple of 64 with a
    ragged hidden size runs the combine's register-fetch epilogue, whose
    lanes past the last column or row address past the end of out."""
    import torch
    import tile_gemm_communication_amd as fm
    monkeypatch.setenv("FM_MOE_TILE", tile)
    E, nl, e0, topk = 16, 8, 0, 2
    say(f"guards moe T={T} hidden={hidden} ffn={ffn} tile={tile}")
    inp = wl.moe_inputs(T, hidden, ffn, E, nl, topk, BF16, seed=T + hidden, zipf_s=1.2)
    X, W1, W2 = dev16(inp["X"], BF16), dev16(inp["W1"], BF16), dev16(inp["W2"], BF16)
    ids = torch.from_numpy(np.ascontiguousarray(inp["topk_ids"], dtype=np.int32)).to("cuda:0")
    # H: capacity T*topk rows inside a guarded buffer; rows past the routed
    # ones must keep their sentinel too
    h_words = T * topk * ffn
    Hbig, Hflat = _guarded(h_words, torch.int16, 0x7ABC)
    H = Hflat.view(torch.bfloat16).view(T * topk, ffn)
    sp = torch.full((T * topk,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    ws = fm.moe_workspace(T, topk, hidden, nl)
    fm.fm_moe_gather_gemm(X, ids, W1, H, sp, off, e0, ws)
    torch.cuda.synchronize()
    rows = int(off[-1].item())
    assert _guards_intact(Hbig, h_words, 0x7ABC)
    assert (Hflat[rows * ffn:].cpu().numpy() == 0x7ABC).all()
    # out: fp32 [T, hidden] inside a guarded buffer (sentinel: a NaN pattern)
    o_words = T * hidden
    Obig, Oflat = _guarded(o_words, torch.int32, 0x7FC0DEAD)
    Oflat.view(torch.float32).copy_(devf32(inp["out_seed"]).view(-1))
    fm.fm_moe_gemm_scatter(H, W2, sp, off, devf32(inp["topk_weights"]),
                           Oflat.view(torch.float32).view(T, hidden), ws)
    torch.cuda.synchronize()
    assert _guards_intact(Obig, o_words, 0x7FC0DEAD)
    assert torch.isfinite(Oflat.view(torch.float32)).all()


@pytest.mark.parametrize("M,N,K,P,tile", [(1024, 520, 200, 2, "256x256"), (520, 200, 136, 4, "256x128"),
                                          (768, 264, 64, 3, "128x128")])
def test_rs_epilogue_stays_in_bounds(monkeypatch, M, N, K, P, tile):
    import torch
    import tile_gemm_communication_amd as fm
    monkeypatch.setenv("FM_TILE", tile)
    say(f"guards rs M={M} N={N} K={K} P={P} tile={tile}")
    A, W, seeds = wl.rs_inputs(M, N, K, P, F16, seed=M + N)
    rows = M // P
    bigs, dst = [], []
    for r in range(P):
        big, flat = _guarded(rows * N, torch.int32, 0x7FC0BEEF)
        flat.view(torch.float32).copy_(devf32(seeds[r]).view(-1))
        bigs.append(big)
        dst.append(flat.view(torch.float32).view(rows, N))
    fm.fm_gemm_rs(dev16(A, F16), dev16(W, F16), dst, rank=P - 1)
    torch.cuda.synchronize()
    for r in range(P):
        assert _guards_intact(bigs[r], rows * N, 0x7FC0BEEF), f"slice {r}"
        assert torch.isfinite(dst[r]).all()


@pytest.mark.parametrize("out32", [False, True])
@pytest.mark.parametrize("M,N,K,tile", [(200, 136, 72, "256x256"), (300, 264, 1000, "256x128"),
                                        (130, 520, 64, "128x128")])
def test_gemm_store_stays_in_bounds(monkeypatch, out32, M, N, K, tile):
    import torch
    import tile_gemm_communication_amd as fm
    monkeypatch.setenv("FM_TILE", tile)
    say(f"guards gemm {M}x{N}x{K} tile={tile} out32={out32}")
    A = dev16(wl.normal_bits((M, K), M + 1, F16), F16)
    B = dev16(wl.normal_bits((K, N), N + 2, F16, 1.0 / np.sqrt(K)), F16)
    if out32:
        big, flat = _guarded(M * N, torch.int32, 0x7FC0F00D)
        C = flat.view(torch.float32).view(M, N)
    else:
        big, flat = _guarded(M * N, torch.int16, 0x7ABC)
        C = flat.view(torch.float16).view(M, N)
    fm.fm_gemm(A, B, C)
    torch.cuda.synchronize()
    assert _guards_intact(big, M * N, 0x7FC0F00D if out32 else 0x7ABC)
    assert torch.isfinite(C.float()).all()
