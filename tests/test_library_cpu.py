"""libfluxmi on the CPU side: the shared library loads, exports every entry
point include/fluxmi.h declares, and rejects invalid arguments before any
launch (these calls return during validation, so no GPU is touched)."""
import ctypes
import os
import re

import pytest

import tile_gemm_communication_amd as fm

pytestmark = pytest.mark.usefixtures("built_library")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(fm_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = fm.lib()
    declared = _declared()
    assert set(declared) == set(fm.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert fm.version() >= 100
    for code, name in [(0, "FM_OK"), (1, "FM_ERR_INVALID_ARG"), (2, "FM_ERR_UNSUPPORTED"),
                       (3, "FM_ERR_HIP"), (4, "FM_ERR_TIMEOUT")]:
        assert fm.status_str(code) == name
    assert fm.status_str(99) == "FM_ERR_UNKNOWN"


# Fake, 16-byte-aligned device addresses: validation rejects the call before
# any pointer is dereferenced or any kernel is launched.
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
P3 = ctypes.c_void_p(0x30000)
ODD = ctypes.c_void_p(0x10008)


@pytest.mark.parametrize("args,want", [
    ((0, 0, 64, 12, 64, P, P2, P3, None), fm.FM_ERR_INVALID_ARG),      # N % 8
    ((0, 0, 64, 64, 60, P, P2, P3, None), fm.FM_ERR_INVALID_ARG),      # K % 8
    ((0, 0, -1, 64, 64, P, P2, P3, None), fm.FM_ERR_INVALID_ARG),      # negative M
    ((0, 0, 64, 64, 64, None, P2, P3, None), fm.FM_ERR_INVALID_ARG),   # null A
    ((0, 0, 64, 64, 64, ODD, P2, P3, None), fm.FM_ERR_INVALID_ARG),    # misaligned A
    ((0, 1, 64, 64, 64, P, P2, P3, None), fm.FM_ERR_UNSUPPORTED),      # f16 in, bf16 out
    ((2, 2, 64, 64, 64, P, P2, P3, None), fm.FM_ERR_UNSUPPORTED),      # fp32 inputs
    ((0, 0, 0, 64, 64, P, P2, P3, None), fm.FM_OK),                    # empty M: no-op
])
def test_gemm_validation(args, want):
    assert fm.lib().fm_gemm(*args) == want


def test_ag_gemm_validation():
    L = fm.lib()
    bad_order = (ctypes.c_int32 * 4)(0, 1, 1, 3)
    ok_order = (ctypes.c_int32 * 4)(3, 1, 0, 2)
    # M not divisible by n_chunks
    assert L.fm_ag_gemm(0, 250, 64, 64, 4, P, P2, P3, P, 1, None, None, 0, None) == \
        fm.FM_ERR_INVALID_ARG
    # order is not a permutation
    assert L.fm_ag_gemm(0, 256, 64, 64, 4, P, P2, P3, P, 1, ctypes.cast(bad_order, ctypes.c_void_p),
                        None, 0, None) == fm.FM_ERR_INVALID_ARG
    # null flags
    assert L.fm_ag_gemm(0, 256, 64, 64, 4, P, P2, P3, None, 1,
                        ctypes.cast(ok_order, ctypes.c_void_p), None, 0, None) == \
        fm.FM_ERR_INVALID_ARG
    # too many chunks
    assert L.fm_ag_gemm(0, 130, 64, 64, 65, P, P2, P3, P, 1, None, None, 0, None) == \
        fm.FM_ERR_INVALID_ARG
    # negative spin limit
    assert L.fm_ag_gemm(0, 256, 64, 64, 4, P, P2, P3, P, 1, None, None, -5, None) == \
        fm.FM_ERR_INVALID_ARG
    # empty problem with valid arguments is a no-op
    assert L.fm_ag_gemm(0, 0, 64, 64, 4, P, P2, P3, P, 1, ctypes.cast(ok_order, ctypes.c_void_p),
                        None, 0, None) == fm.FM_OK


def test_gemm_rs_validation():
    L = fm.lib()
    dst = (ctypes.c_void_p * 4)(0x40000, 0x50000, 0x60000, 0x70000)
    dst_bad = (ctypes.c_void_p * 4)(0x40000, 0x50004, 0x60000, 0x70000)
    d = ctypes.cast(dst, ctypes.c_void_p)
    assert L.fm_gemm_rs(0, 250, 64, 64, 4, 0, P, P2, d, 0, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_gemm_rs(0, 256, 64, 64, 4, 4, P, P2, d, 0, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_gemm_rs(0, 256, 64, 64, 4, 0, P, P2, d, 2, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_gemm_rs(0, 256, 64, 64, 17, 0, P, P2, d, 0, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_gemm_rs(0, 256, 64, 64, 4, 0, P, P2, ctypes.cast(dst_bad, ctypes.c_void_p), 0,
                        None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_gemm_rs(0, 256, 64, 64, 4, 0, P, P2, None, 0, None) == fm.FM_ERR_INVALID_ARG


# a fake workspace: aligned, and reported large enough for the small shapes
WS = ctypes.c_void_p(0x800000)
WS_BYTES = 1 << 24


def test_moe_validation():
    L = fm.lib()
    assert L.fm_moe_route(16, 2, 0, 65, P, P2, P3, WS, WS_BYTES, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_moe_route(16, 0, 0, 8, P, P2, P3, WS, WS_BYTES, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_moe_route(16, 2, 0, 8, P, P2, None, WS, WS_BYTES, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_moe_gather_gemm(2, 16, 64, 64, 2, 0, 8, P, P, P, P, P, P, WS, WS_BYTES,
                                None) == fm.FM_ERR_UNSUPPORTED
    assert L.fm_moe_gather_gemm(1, 16, 60, 64, 2, 0, 8, P, P, P, P, P, P, WS, WS_BYTES,
                                None) == fm.FM_ERR_INVALID_ARG
    # the activation is checked first; a valid one still meets the dtype check
    for bad_act in (-1, 4, 100):
        assert L.fm_moe_gather_gemm_act(1, 16, 64, 64, 2, 0, 8, P, P, P, P, P, P, bad_act,
                                        WS, WS_BYTES, None) == fm.FM_ERR_INVALID_ARG
    for act in (fm.FM_ACT_NONE, fm.FM_ACT_RELU, fm.FM_ACT_GELU_TANH, fm.FM_ACT_SILU):
        assert L.fm_moe_gather_gemm_act(2, 16, 64, 64, 2, 0, 8, P, P, P, P, P, P, act,
                                        WS, WS_BYTES, None) == fm.FM_ERR_UNSUPPORTED
    assert L.fm_moe_gemm_scatter(1, 16, 64, 64, 2, 8, ODD, P, P, P, P, P3, None, 0, WS,
                                 WS_BYTES, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_moe_gemm_scatter(1, 16, 64, 64, 2, 0, P, P, P, P, P, P3, None, 0, WS,
                                 WS_BYTES, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_moe_gemm_scatter(1, 16, 64, 64, 2, 8, P, P, P, P, P, P3, None, -1, WS,
                                 WS_BYTES, None) == fm.FM_ERR_INVALID_ARG   # spin_limit < 0


def test_moe_workspace_size_query():
    """The size query grows with the tokens and the hidden size, covers the
    fixed regions, and rejects out-of-range arguments with 0."""
    L = fm.lib()
    q = L.fm_moe_workspace_bytes
    small = q(16, 2, 64, 8)
    assert small > 0 and small % 256 == 0
    assert q(16384, 2, 4096, 8) > q(1024, 2, 4096, 8) > small
    assert q(16384, 2, 4096, 8) > q(16384, 2, 1024, 8)
    assert q(16384, 4, 4096, 8) > q(16384, 2, 4096, 8)
    assert q(16384, 2, 4096, 64) > q(16384, 2, 4096, 8)
    # the EP=8 workload: fixed regions (control, sink, route histograms) plus
    # one flag per (128-row tile, 128-column tile) of up to 32768 + 8 x 128 rows
    assert q(16384, 2, 4096, 8) >= 4 * (16704 + (256 + 8) * 32)
    for bad in [(-1, 2, 64, 8), (16, 0, 64, 8), (16, 2, -8, 8), (16, 2, 64, 0), (16, 2, 64, 65)]:
        assert q(*bad) == 0, bad
    assert fm.fm_moe_workspace_bytes(16, 2, 64, 8) == small


def test_moe_workspace_too_small_or_missing():
    """A missing, misaligned or too small workspace is refused before any
    launch, by the route, every layer-0 form and the combine."""
    L = fm.lib()
    T, topk, hidden, ffn, nl = 1024, 2, 512, 256, 8
    need = L.fm_moe_workspace_bytes(T, topk, hidden, nl)
    route_need = 4 * (320 + 16384)          # the route uses the fixed regions only
    odd_ws = ctypes.c_void_p(0x800008)
    for ws, nb in [(None, need), (odd_ws, need), (WS, route_need - 4)]:
        assert L.fm_moe_route(T, topk, 0, nl, P, P2, P3, ws, nb, None) == fm.FM_ERR_INVALID_ARG
        assert L.fm_moe_gather_gemm(1, T, hidden, ffn, topk, 0, nl, P, P, P, P, P, P, ws, nb,
                                    None) == fm.FM_ERR_INVALID_ARG
        assert L.fm_moe_ag_gather_gemm(1, T, hidden, ffn, topk, 0, nl, P, P, P, P, P, P, 4, P3,
                                       1, None, None, 0, ws, nb, None) == fm.FM_ERR_INVALID_ARG
    for ws, nb in [(None, need), (odd_ws, need), (WS, need - 256), (WS, route_need)]:
        assert L.fm_moe_gemm_scatter(1, T, hidden, ffn, topk, nl, P, P, P, P, P, P3, None, 0,
                                     ws, nb, None) == fm.FM_ERR_INVALID_ARG, (ws, nb)


def test_chunk_push_validation():
    L = fm.lib()
    assert L.fm_chunk_push(P, P2, 100, P3, P3, 1, 0, None) == fm.FM_ERR_INVALID_ARG   # 16 B
    assert L.fm_chunk_push(P, P, 4096, P3, P3, 1, 0, None) == fm.FM_ERR_INVALID_ARG   # overlap
    assert L.fm_chunk_push(P, P2, 64, None, P3, 1, 0, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_chunk_push(P, P2, 64, P3, None, 1, 0, None) == fm.FM_ERR_INVALID_ARG


def test_chunk_push_dma_validation():
    L = fm.lib()
    assert L.fm_chunk_push_dma(P, P2, 100, P3, 1, None) == fm.FM_ERR_INVALID_ARG   # 16 B
    assert L.fm_chunk_push_dma(P, P, 4096, P3, 1, None) == fm.FM_ERR_INVALID_ARG   # overlap
    assert L.fm_chunk_push_dma(P, P2, 64, None, 1, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_chunk_push_dma(P, P2, 64, ctypes.c_void_p(0x30002), 1, None) == \
        fm.FM_ERR_INVALID_ARG   # flag alignment
    assert L.fm_chunk_push_dma(None, P2, 64, P3, 1, None) == fm.FM_ERR_INVALID_ARG


def _arr(ctype, vals):
    return ctypes.cast((ctype * len(vals))(*vals), ctypes.c_void_p)


def test_ag_gemm_pull_validation():
    L = fm.lib()
    chunks4 = _arr(ctypes.c_void_p, [0x10000, 0x20000, 0x30000, 0x40000])

    def call(M=256, n=4, chunks=chunks4, W=P, C=P2, flags=P3, order=None, spin=0, K=64):
        return L.fm_ag_gemm_pull(0, M, 64, K, n, chunks, W, C, flags, 1, order, None, spin, None)
    assert call(n=3) == fm.FM_ERR_INVALID_ARG                          # M % n_chunks
    assert call(n=0) == fm.FM_ERR_INVALID_ARG
    assert call(chunks=None) == fm.FM_ERR_INVALID_ARG
    assert call(flags=None) == fm.FM_ERR_INVALID_ARG
    assert call(K=60) == fm.FM_ERR_INVALID_ARG                         # K % 8
    assert call(spin=-1) == fm.FM_ERR_INVALID_ARG
    assert call(chunks=_arr(ctypes.c_void_p, [0x10000, 0x20000, 0, 0x40000])) == \
        fm.FM_ERR_INVALID_ARG                                          # a null chunk
    assert call(chunks=_arr(ctypes.c_void_p, [0x10000, 0x20008, 0x30000, 0x40000])) == \
        fm.FM_ERR_INVALID_ARG                                          # misaligned chunk
    assert call(order=_arr(ctypes.c_int32, [0, 0, 1, 2])) == fm.FM_ERR_INVALID_ARG
    assert L.fm_ag_gemm_pull(2, 256, 64, 64, 4, chunks4, P, P2, P3, 1, None, None, 0, None) == \
        fm.FM_ERR_UNSUPPORTED                                          # fp32 operands
    assert call(M=0) == fm.FM_OK                                       # nothing to do


def test_ag_gemm_producers_validation():
    L = fm.lib()
    src4 = _arr(ctypes.c_void_p, [0, 0x50000, 0x60000, 0x70000])
    X = ctypes.c_void_p(0x100000)

    def call(M=256, n=4, src=src4, X=X, flags=P3, counters=P2, order=None, nprod=0, spin=0):
        return L.fm_ag_gemm_producers(0, M, 64, 64, n, src, X, P, P, flags, counters, 1, order,
                                      nprod, None, spin, None)
    assert call(src=None) == fm.FM_ERR_INVALID_ARG
    assert call(counters=None) == fm.FM_ERR_INVALID_ARG
    assert call(counters=ctypes.c_void_p(0x20002)) == fm.FM_ERR_INVALID_ARG
    assert call(n=3) == fm.FM_ERR_INVALID_ARG                          # M % n_chunks
    assert call(nprod=4) == fm.FM_ERR_INVALID_ARG                      # below 8
    assert call(nprod=12) == fm.FM_ERR_INVALID_ARG                     # not a multiple of 8
    assert call(spin=-1) == fm.FM_ERR_INVALID_ARG
    assert call(src=_arr(ctypes.c_void_p, [0, 0x50008, 0x60000, 0x70000])) == \
        fm.FM_ERR_INVALID_ARG                                          # misaligned source
    assert call(src=_arr(ctypes.c_void_p, [0, 0x100000 + 4096, 0, 0])) == \
        fm.FM_ERR_INVALID_ARG                                          # source inside X
    assert call(order=_arr(ctypes.c_int32, [3, 3, 1, 0])) == fm.FM_ERR_INVALID_ARG
    assert call(M=0) == fm.FM_OK


def test_moe_ag_producers_validation():
    L = fm.lib()
    X = ctypes.c_void_p(0x100000)
    src4 = _arr(ctypes.c_void_p, [0, 0x50000, 0x60000, 0x70000])

    def call(n=4, src=src4, flags=P3, counters=P2, nprod=0, order=None):
        return L.fm_moe_ag_gather_gemm_producers(1, 64, 64, 64, 2, 0, 8, X, P, P, P, P, P, n, src,
                                                 flags, counters, 1, order, nprod, None, 0, WS,
                                                 WS_BYTES, None)
    assert call(src=None) == fm.FM_ERR_INVALID_ARG
    assert call(flags=None) == fm.FM_ERR_INVALID_ARG
    assert call(counters=None) == fm.FM_ERR_INVALID_ARG
    assert call(nprod=12) == fm.FM_ERR_INVALID_ARG
    assert call(nprod=4) == fm.FM_ERR_INVALID_ARG
    assert call(n=3) == fm.FM_ERR_INVALID_ARG                          # T % n_chunks
    assert call(src=_arr(ctypes.c_void_p, [0, 0x50008, 0, 0])) == fm.FM_ERR_INVALID_ARG
    assert call(src=_arr(ctypes.c_void_p, [0, 0x100000 + 1024, 0, 0])) == fm.FM_ERR_INVALID_ARG
    assert call(order=_arr(ctypes.c_int32, [0, 0, 1, 2])) == fm.FM_ERR_INVALID_ARG


def test_moe_ag_pull_validation():
    L = fm.lib()
    ch4 = _arr(ctypes.c_void_p, [0x50000, 0x60000, 0x70000, 0x80000])

    def call(n=4, chunks=ch4, flags=P3, order=None):
        return L.fm_moe_ag_gather_gemm_pull(1, 64, 64, 64, 2, 0, 8, chunks, P, P, P, P, P, n,
                                            flags, 1, order, None, 0, WS, WS_BYTES, None)
    assert call(chunks=None) == fm.FM_ERR_INVALID_ARG
    assert call(flags=None) == fm.FM_ERR_INVALID_ARG
    assert call(n=3) == fm.FM_ERR_INVALID_ARG                          # T % n_chunks
    assert call(n=0) == fm.FM_ERR_INVALID_ARG
    assert call(chunks=_arr(ctypes.c_void_p, [0x50000, 0, 0x70000, 0x80000])) == \
        fm.FM_ERR_INVALID_ARG                                          # a null chunk
    assert call(chunks=_arr(ctypes.c_void_p, [0x50000, 0x60008, 0x70000, 0x80000])) == \
        fm.FM_ERR_INVALID_ARG                                          # misaligned chunk
    assert call(order=_arr(ctypes.c_int32, [1, 1, 2, 3])) == fm.FM_ERR_INVALID_ARG


def test_chunk_signal_paced_validation():
    L = fm.lib()
    t = _arr(ctypes.c_int64, [0, 10, 20, 30])
    assert L.fm_chunk_signal_paced(None, 4, None, t, 1, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_chunk_signal_paced(ctypes.c_void_p(0x30002), 4, None, t, 1, None) == \
        fm.FM_ERR_INVALID_ARG                                          # flag alignment
    assert L.fm_chunk_signal_paced(P3, 0, None, t, 1, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_chunk_signal_paced(P3, 65, None, t, 1, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_chunk_signal_paced(P3, 4, None, None, 1, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_chunk_signal_paced(P3, 4, None, _arr(ctypes.c_int64, [0, 20, 10, 30]), 1,
                                   None) == fm.FM_ERR_INVALID_ARG     # decreasing
    assert L.fm_chunk_signal_paced(P3, 4, None, _arr(ctypes.c_int64, [0, 0, 0, 2 * 10**9]), 1,
                                   None) == fm.FM_ERR_INVALID_ARG     # beyond one second
    assert L.fm_chunk_signal_paced(P3, 4, None, _arr(ctypes.c_int64, [-1, 0, 0, 0]), 1,
                                   None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_chunk_signal_paced(P3, 4, _arr(ctypes.c_int32, [0, 1, 2, 2]), t, 1, None) == \
        fm.FM_ERR_INVALID_ARG                                          # not a permutation


def test_moe_ag_gather_validation():
    L = fm.lib()
    args = (1, 64, 64, 64, 2, 0, 8, P, P, P, P, P, P)
    def call(n, flags, order=None, spin=0):
        o = None if order is None else ctypes.cast((ctypes.c_int32 * len(order))(*order),
                                                   ctypes.c_void_p)
        return L.fm_moe_ag_gather_gemm(*args, n, flags, 1, o, None, spin, WS, WS_BYTES, None)
    assert call(4, None) == fm.FM_ERR_INVALID_ARG                 # flags required
    assert call(0, P3) == fm.FM_ERR_INVALID_ARG
    assert call(3, P3) == fm.FM_ERR_INVALID_ARG                   # T % n_chunks
    assert call(65, P3) == fm.FM_ERR_INVALID_ARG
    assert call(4, P3, spin=-1) == fm.FM_ERR_INVALID_ARG
    assert call(4, P3, order=[0, 1, 1, 2]) == fm.FM_ERR_INVALID_ARG   # not a permutation
    assert call(4, P3, order=[0, 1, 2, 4]) == fm.FM_ERR_INVALID_ARG


def test_oracle_is_not_reachable_from_the_product():
    pkg = os.path.join(ROOT, "tile_gemm_communication_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in txt and "fm_oracle" not in txt, f


def test_noalloc_combine_limit_and_validation():
    """The no-alloc combine refuses shapes beyond its static scratch and
    invalid arguments before touching the GPU."""
    L = fm.lib()
    # (2^20/128 + 8) x 32 column tiles: beyond the 65216 flags of the scratch
    assert L.fm_moe_gemm_scatter_noalloc(1, 1 << 19, 4096, 8, 2, 8, P, P, P, P, P, P3, None, 0,
                                         None) == fm.FM_ERR_UNSUPPORTED
    assert L.fm_moe_gemm_scatter_noalloc(1, 16, 64, 64, 2, 8, ODD, P, P, P, P, P3, None, 0,
                                         None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_moe_gemm_scatter_noalloc(0, 16, 64, 60, 2, 8, P, P, P, P, P, P3, None, 0,
                                         None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_moe_gemm_scatter_noalloc(2, 16, 64, 64, 2, 8, P, P, P, P, P, P3, None, 0,
                                         None) == fm.FM_ERR_UNSUPPORTED


def test_probe_validation():
    L = fm.lib()
    out = ctypes.c_void_p(0x40000)
    n = 1 << 16
    assert L.fm_probe_mfma(2, 0, 1, 10, 0, out, n, None) == fm.FM_ERR_UNSUPPORTED
    assert L.fm_probe_mfma(1, 2, 1, 10, 0, out, n, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_probe_mfma(1, 0, 3, 10, 0, out, n, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_probe_mfma(1, 0, 1, 0, 0, out, n, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_probe_mfma(1, 0, 1, 10, 0, None, n, None) == fm.FM_ERR_INVALID_ARG
    assert L.fm_probe_mfma(1, 0, 1, 10, 0, ctypes.c_void_p(0x40004), n, None) == \
        fm.FM_ERR_INVALID_ARG
    assert L.fm_probe_mfma(1, 0, 1, 10, 0, out, 4, None) == fm.FM_ERR_INVALID_ARG   # too small
