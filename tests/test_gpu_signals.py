"""The chunk-arrival protocol on the GPU: producer pushes on a side stream,
consumer waits inside the fused AllGather-GEMM.  Late arrival, withheld flags
(bounded wait -> FM_ERR_TIMEOUT, no hang), epoch reuse without resetting
flags, and a wrong order hint."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import F16, Arrival, bits16, dev16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _reference(arr, W, N):
    import torch
    import tile_gemm_communication_amd as fm
    C = torch.empty((arr.X.shape[0], N), dtype=arr.X.dtype, device="cuda:0")
    fm.fm_gemm(arr.X, W, C)
    torch.cuda.synchronize()
    return bits16(C)


def _ag(arr, W, N, order, epoch, hint=None, **kw):
    import torch
    import tile_gemm_communication_amd as fm
    C = torch.empty((arr.X.shape[0], N), dtype=arr.X.dtype, device="cuda:0")
    arr.err.zero_()
    arr.push(order, epoch, **kw)
    fm.fm_ag_gemm(arr.X, W, C, arr.flags, epoch, arr.n,
                  order=list(order if hint is None else hint), err_word=arr.err,
                  spin_limit=0)
    arr.join()
    torch.cuda.synchronize()
    return C


def test_push_copies_and_publishes():
    import torch
    import tile_gemm_communication_amd as fm
    src = torch.randint(-30000, 30000, (1 << 20,), dtype=torch.int16, device="cuda:0")
    dst = torch.zeros_like(src)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    counter = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for wg in (0, 1, 7, 200):
        dst.zero_()
        fm.fm_chunk_push(src, dst, flag, counter, epoch=10 + wg, n_workgroups=wg)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
        assert flag.item() == 10 + wg and counter.item() == 0


def test_push_dma_copies_and_publishes():
    import torch
    import tile_gemm_communication_amd as fm
    src = torch.randint(-30000, 30000, (3 << 20,), dtype=torch.int16, device="cuda:0")
    dst = torch.zeros_like(src)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for e in (5, 6):
        dst.zero_()
        fm.fm_chunk_push_dma(src, dst, flag, epoch=e)
        torch.cuda.synchronize()
        assert torch.equal(src, dst) and flag.item() == e
    fm.fm_chunk_push_dma(None, None, flag, epoch=9)
    torch.cuda.synchronize()
    assert flag.item() == 9


@pytest.mark.parametrize("delay", [0, 5_000_000])
def test_dma_arrival_bit_identical(delay):
    """Chunks delivered by the copy engines with a flag write behind each: the
    fused kernel waits for them and reproduces the non-split GEMM's bits."""
    chunks, W, order = wl.ag_inputs(8, 256, 768, 1024, F16, seed=905, arrival="random")
    arr = Arrival(chunks, F16, 1024)
    Wd = dev16(W, F16)
    arr.poison()
    say(f"dma arrival delay={delay}")
    C = _ag(arr, Wd, 768, order, arr.next_epoch(), delay_cycles=delay, dma=True)
    assert arr.err.item() == 0
    assert np.array_equal(bits16(C), _reference(arr, Wd, 768))


def test_late_arrival_is_waited_for():
    """Chunks are pushed only after a ~ms spin on the side stream while the
    gathered buffer holds NaN: the fused kernel must wait and still produce
    exactly the non-split GEMM's bits."""
    chunks, W, order = wl.ag_inputs(8, 128, 512, 512, F16, seed=901, arrival="random")
    arr = Arrival(chunks, F16, 512)
    Wd = dev16(W, F16)
    arr.poison()
    say("late arrival")
    C = _ag(arr, Wd, 512, order, arr.next_epoch(), delay_cycles=5_000_000)
    assert arr.err.item() == 0
    assert np.array_equal(bits16(C), _reference(arr, Wd, 512))


def test_withheld_flag_times_out():
    """A chunk whose flag is never published: the bounded wait gives up,
    FM_ERR_TIMEOUT lands in err_word and the kernel exits (no hang)."""
    import torch
    import tile_gemm_communication_amd as fm
    chunks, W, order = wl.ag_inputs(4, 64, 256, 128, F16, seed=902, arrival="ring")
    arr = Arrival(chunks, F16, 128)
    Wd = dev16(W, F16)
    epoch = arr.next_epoch()
    C = torch.empty((256, 256), dtype=torch.float16, device="cuda:0")
    arr.err.zero_()
    arr.push(order, epoch, skip=(2,))
    fm.fm_ag_gemm(arr.X, Wd, C, arr.flags, epoch, 4, order=list(order), err_word=arr.err,
                  spin_limit=2000)
    arr.join()
    torch.cuda.synchronize()
    assert arr.err.item() == fm.FM_ERR_TIMEOUT
    # the same buffers work again on the next epoch once every chunk arrives
    arr.poison()
    C2 = _ag(arr, Wd, 256, order, arr.next_epoch())
    assert arr.err.item() == 0
    assert np.array_equal(bits16(C2), _reference(arr, Wd, 256))


def test_epoch_reuse_without_reset():
    chunks, W, order = wl.ag_inputs(4, 96, 256, 256, F16, seed=903, arrival="random")
    arr = Arrival(chunks, F16, 256)
    Wd = dev16(W, F16)
    want = None
    for it in range(40):
        arr.poison()
        C = _ag(arr, Wd, 256, np.roll(order, it), arr.next_epoch())
        assert arr.err.item() == 0
        b = bits16(C)
        if want is None:
            want = _reference(arr, Wd, 256)
        assert np.array_equal(b, want), it


def test_wrong_order_hint_is_still_correct():
    chunks, W, order = wl.ag_inputs(8, 64, 128, 256, F16, seed=904, arrival="random")
    arr = Arrival(chunks, F16, 256)
    Wd = dev16(W, F16)
    arr.poison()
    C = _ag(arr, Wd, 128, order, arr.next_epoch(), hint=list(reversed(order.tolist())))
    assert arr.err.item() == 0
    assert np.array_equal(bits16(C), _reference(arr, Wd, 128))


def test_readme_example_runs():
    """The Python example in README.md runs as written and its AllGather-GEMM
    equals fm_gemm on the gathered buffer bit for bit."""
    import os
    import re
    import torch
    import tile_gemm_communication_amd as fm
    text = open(os.path.join(os.path.dirname(__file__), "..", "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    ns = {}
    exec(compile(code, "README.md", "exec"), ns)
    torch.cuda.synchronize()
    ref = torch.empty_like(ns["C"])
    fm.fm_gemm(ns["X"], ns["W"], ref)
    torch.cuda.synchronize()
    assert torch.equal(ns["C"].view(torch.int16), ref.view(torch.int16))
