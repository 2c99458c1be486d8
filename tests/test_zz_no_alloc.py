"""fm_moe_gemm_scatter_noalloc (the combine on the library's static per-GPU
scratch, for callers that cannot allocate) against fm_moe_gemm_scatter with a
caller workspace: bit-identical outputs on two calls in a row, the second on a
smaller input, and both within the parity bar of the CPU oracle."""
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


def _layer0(inp, e0, nl):
    """Route + layer 0 on the GPU; returns the combine's inputs."""
    import torch
    import tile_gemm_communication_amd as fm
    T, topk = inp["topk_ids"].shape
    hidden, ffn = inp["X"].shape[1], inp["W1"].shape[2]
    H = torch.zeros((T * topk, ffn), dtype=torch.bfloat16, device="cuda:0")
    sp = torch.full((T * topk,), -1, dtype=torch.int32, device="cuda:0")
    off = torch.zeros(nl + 1, dtype=torch.int32, device="cuda:0")
    fm.fm_moe_gather_gemm(dev16(inp["X"], BF16), _i32(inp["topk_ids"]), dev16(inp["W1"], BF16),
                          H, sp, off, e0, fm.moe_workspace(T, topk, hidden, nl))
    return H, sp, off


def test_noalloc_combine_matches_workspace_combine(oracle):
    import torch
    import tile_gemm_communication_amd as fm
    for call, (T, hidden, ffn, E, nl, e0) in enumerate([(3000, 512, 264, 16, 8, 0),
                                                         (700, 256, 136, 16, 8, 8)]):
        say(f"no-alloc combine call {call}: T={T} hidden={hidden} ffn={ffn}")
        inp = wl.moe_inputs(T, hidden, ffn, E, nl, 2, BF16, seed=5150 + call, zipf_s=1.2)
        H, sp, off = _layer0(inp, e0, nl)
        W2, wts = dev16(inp["W2"], BF16), devf32(inp["topk_weights"])
        err = torch.zeros(2, dtype=torch.int32, device="cuda:0")
        ref_out = devf32(inp["out_seed"])
        fm.fm_moe_gemm_scatter(H, W2, sp, off, wts, ref_out, fm.moe_workspace(T, 2, hidden, nl),
                               err_word=err[0:1])
        out = devf32(inp["out_seed"])
        fm.fm_moe_gemm_scatter_noalloc(H, W2, sp, off, wts, out, err_word=err[1:2])
        torch.cuda.synchronize()
        assert err.cpu().tolist() == [0, 0]
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), f"call {call}"
        roff, rsp = oracle.moe_route(inp["topk_ids"], e0, nl)
        Hb = oracle.round_bf16(oracle.moe_layer0(BF16, inp["X"], inp["W1"], rsp, roff, 2))
        ref = oracle.moe_layer1(BF16, Hb, inp["W2"], inp["topk_ids"], inp["topk_weights"], rsp,
                                roff, inp["out_seed"], e0)
        assert_close(host64(out) - inp["out_seed"], ref - inp["out_seed"], f"no-alloc {call}")
