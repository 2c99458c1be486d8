"""Python binding of libfluxmi (argument marshalling only).

Each function has the name of the C-ABI entry point it calls (declared in
include/fluxmi.h) and takes torch tensors that already live on the GPU; the
binding checks shapes and dtypes, pulls out device pointers and the current
HIP stream, and calls the library.  Every step of the computation runs in the
library's HIP kernels: there is no fallback, and calling any function without
the built library raises.

torch supplies device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfluxmi.so")

FM_OK, FM_ERR_INVALID_ARG, FM_ERR_UNSUPPORTED, FM_ERR_HIP, FM_ERR_TIMEOUT = range(5)
FM_F16, FM_BF16, FM_F32 = 0, 1, 2

EXPORTS = ("fm_version", "fm_status_str", "fm_gemm", "fm_ag_gemm", "fm_ag_gemm_pull", "fm_ag_gemm_producers",
           "fm_chunk_push", "fm_chunk_push_dma", "fm_chunk_signal_paced",
           "fm_gemm_rs", "fm_moe_workspace_bytes", "fm_moe_route", "fm_moe_gather_gemm",
           "fm_moe_gather_gemm_act",
           "fm_moe_ag_gather_gemm",
           "fm_moe_ag_gather_gemm_producers", "fm_moe_ag_gather_gemm_pull",
           "fm_moe_gemm_scatter", "fm_moe_gemm_scatter_noalloc", "fm_probe_mfma")

# fm_act_t: activation of MoE layer 0's result (fm_moe_gather_gemm_act)
FM_ACT_NONE, FM_ACT_RELU, FM_ACT_GELU_TANH, FM_ACT_SILU = 0, 1, 2, 3


class FluxMIError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfluxmi.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libfluxmi.so not found at {LIB_PATH}; build it with "
            "`python tile_gemm_communication_amd/build.py` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, u32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p
    L.fm_version.restype = ctypes.c_int
    L.fm_version.argtypes = []
    L.fm_status_str.restype = ctypes.c_char_p
    L.fm_status_str.argtypes = [ctypes.c_int]
    L.fm_gemm.restype = ctypes.c_int
    L.fm_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, p, p, p, p]
    L.fm_ag_gemm.restype = ctypes.c_int
    L.fm_ag_gemm.argtypes = [ctypes.c_int, i64, i64, i64, i32, p, p, p, p, u32, p, p, i64, p]
    L.fm_ag_gemm_pull.restype = ctypes.c_int
    L.fm_ag_gemm_pull.argtypes = [ctypes.c_int, i64, i64, i64, i32, p, p, p, p, u32, p, p, i64,
                                  p]
    L.fm_ag_gemm_producers.restype = ctypes.c_int
    L.fm_ag_gemm_producers.argtypes = [ctypes.c_int, i64, i64, i64, i32, p, p, p, p, p, p, u32,
                                       p, i32, p, i64, p]
    L.fm_chunk_signal_paced.restype = ctypes.c_int
    L.fm_chunk_signal_paced.argtypes = [p, i32, p, p, u32, p]
    L.fm_chunk_push.restype = ctypes.c_int
    L.fm_chunk_push.argtypes = [p, p, i64, p, p, u32, i32, p]
    L.fm_chunk_push_dma.restype = ctypes.c_int
    L.fm_chunk_push_dma.argtypes = [p, p, i64, p, u32, p]
    L.fm_gemm_rs.restype = ctypes.c_int
    L.fm_gemm_rs.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, p, p, p, i32, p]
    sz = ctypes.c_size_t
    L.fm_moe_workspace_bytes.restype = sz
    L.fm_moe_workspace_bytes.argtypes = [i64, i32, i64, i32]
    L.fm_moe_route.restype = ctypes.c_int
    L.fm_moe_route.argtypes = [i64, i32, i32, i32, p, p, p, p, sz, p]
    L.fm_moe_gather_gemm.restype = ctypes.c_int
    L.fm_moe_gather_gemm.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, i32, p, p, p, p, p,
                                     p, p, sz, p]
    L.fm_moe_gather_gemm_act.restype = ctypes.c_int
    L.fm_moe_gather_gemm_act.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, i32, p, p, p, p,
                                         p, p, ctypes.c_int, p, sz, p]
    L.fm_moe_ag_gather_gemm.restype = ctypes.c_int
    L.fm_moe_ag_gather_gemm.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, i32, p, p, p, p,
                                        p, p, i32, p, u32, p, p, i64, p, sz, p]
    L.fm_moe_ag_gather_gemm_producers.restype = ctypes.c_int
    L.fm_moe_ag_gather_gemm_producers.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, i32, p,
                                                  p, p, p, p, p, i32, p, p, p, u32, p, i32, p,
                                                  i64, p, sz, p]
    L.fm_moe_ag_gather_gemm_pull.restype = ctypes.c_int
    L.fm_moe_ag_gather_gemm_pull.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, i32, p, p, p,
                                             p, p, p, i32, p, u32, p, p, i64, p, sz, p]
    L.fm_moe_gemm_scatter.restype = ctypes.c_int
    L.fm_moe_gemm_scatter.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, p, p, p, p, p, p, p,
                                      i64, p, sz, p]
    L.fm_probe_mfma.restype = ctypes.c_int
    L.fm_probe_mfma.argtypes = [ctypes.c_int, i32, i32, i64, i32, p, i64, p]
    L.fm_moe_gemm_scatter_noalloc.restype = ctypes.c_int
    L.fm_moe_gemm_scatter_noalloc.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32, p, p, p, p,
                                              p, p, p, i64, p]
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().fm_status_str(int(status)).decode()


def version() -> int:
    return lib().fm_version()


def _check(fn: str, status: int) -> None:
    if status != FM_OK:
        raise FluxMIError(fn, status)


# -- marshalling helpers -------------------------------------------------------

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return FM_F16
    if t.dtype == torch.bfloat16:
        return FM_BF16
    if t.dtype == torch.float32:
        return FM_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# -- operators -------------------------------------------------------------------

def fm_gemm(A, B, C, stream=None) -> None:
    """C = A @ B (A [M,K], B [K,N], C [M,N]; A/B fp16 or bf16, C same or fp32)."""
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N) or B.dtype != A.dtype:
        raise ValueError("fm_gemm: shape or dtype mismatch")
    _check("fm_gemm", lib().fm_gemm(_dt(A), _dt(C), M, N, K, _ptr(A), _ptr(B), _ptr(C),
                                    _stream(stream)))


def fm_ag_gemm(X, W, C, flags, epoch: int, n_chunks: int, order=None, err_word=None,
               spin_limit: int = 0, stream=None) -> None:
    """C = AllGather(X) @ W, reading row chunk c of X only after flags[c] >= epoch."""
    M, K = X.shape
    K2, N = W.shape
    if K2 != K or tuple(C.shape) != (M, N) or C.dtype != X.dtype or W.dtype != X.dtype:
        raise ValueError("fm_ag_gemm: shape or dtype mismatch")
    order_arr = None
    if order is not None:
        order = [int(c) for c in order]
        order_arr = (ctypes.c_int32 * len(order))(*order)
    _check("fm_ag_gemm", lib().fm_ag_gemm(
        _dt(X), M, N, K, int(n_chunks), _ptr(X), _ptr(W), _ptr(C), _ptr(flags),
        ctypes.c_uint32(epoch & 0xFFFFFFFF),
        ctypes.cast(order_arr, ctypes.c_void_p) if order_arr is not None else None,
        _ptr(err_word), int(spin_limit), _stream(stream)))


def _order_arg(order):
    if order is None:
        return None
    order = [int(c) for c in order]
    return (ctypes.c_int32 * len(order))(*order)


def fm_ag_gemm_pull(chunks, W, C, flags, epoch: int, order=None, err_word=None,
                    spin_limit: int = 0, stream=None) -> None:
    """C = concat(chunks) @ W, each chunk read in place after flags[c] >= epoch."""
    n = len(chunks)
    Mc, K = chunks[0].shape
    K2, N = W.shape
    M = n * Mc
    if (K2 != K or tuple(C.shape) != (M, N) or C.dtype != W.dtype
            or any(tuple(x.shape) != (Mc, K) or x.dtype != W.dtype for x in chunks)):
        raise ValueError("fm_ag_gemm_pull: shape or dtype mismatch")
    ptrs = (ctypes.c_void_p * n)(*[_ptr(x) for x in chunks])
    o = _order_arg(order)
    _check("fm_ag_gemm_pull", lib().fm_ag_gemm_pull(
        _dt(W), M, N, K, n, ctypes.cast(ptrs, ctypes.c_void_p), _ptr(W), _ptr(C), _ptr(flags),
        ctypes.c_uint32(epoch & 0xFFFFFFFF),
        ctypes.cast(o, ctypes.c_void_p) if o is not None else None,
        _ptr(err_word), int(spin_limit), _stream(stream)))


def fm_ag_gemm_producers(src, X, W, C, flags, counters, epoch: int, order=None,
                         n_producers: int = 0, err_word=None, spin_limit: int = 0,
                         stream=None) -> None:
    """C = X @ W where producer workgroups of the same launch copy src[c] (None:
    already in X) into X's chunk c and publish flags[c] = epoch."""
    n = len(src)
    M, K = X.shape
    K2, N = W.shape
    Mc = M // n
    if (K2 != K or tuple(C.shape) != (M, N) or C.dtype != X.dtype or W.dtype != X.dtype
            or any(x is not None and (tuple(x.shape) != (Mc, K) or x.dtype != X.dtype)
                   for x in src)):
        raise ValueError("fm_ag_gemm_producers: shape or dtype mismatch")
    ptrs = (ctypes.c_void_p * n)(*[_ptr(x) if x is not None else None for x in src])
    o = _order_arg(order)
    _check("fm_ag_gemm_producers", lib().fm_ag_gemm_producers(
        _dt(X), M, N, K, n, ctypes.cast(ptrs, ctypes.c_void_p), _ptr(X), _ptr(W), _ptr(C),
        _ptr(flags), _ptr(counters), ctypes.c_uint32(epoch & 0xFFFFFFFF),
        ctypes.cast(o, ctypes.c_void_p) if o is not None else None, int(n_producers),
        _ptr(err_word), int(spin_limit), _stream(stream)))


def fm_chunk_signal_paced(flags, arrive_ns, epoch: int, order=None, stream=None) -> None:
    """Publish flags[order[a]] = epoch once arrive_ns[a] ns have passed on the device."""
    n = len(arrive_ns)
    t = (ctypes.c_int64 * n)(*[int(x) for x in arrive_ns])
    o = _order_arg(order)
    _check("fm_chunk_signal_paced", lib().fm_chunk_signal_paced(
        _ptr(flags), n, ctypes.cast(o, ctypes.c_void_p) if o is not None else None,
        ctypes.cast(t, ctypes.c_void_p), ctypes.c_uint32(epoch & 0xFFFFFFFF), _stream(stream)))


def fm_chunk_push(src, dst, flag, counter, epoch: int, n_workgroups: int = 0,
                  stream=None) -> None:
    """Copy src into dst, then publish flag = epoch (release)."""
    nbytes = src.numel() * src.element_size() if src is not None else 0
    if src is not None and dst.numel() * dst.element_size() < nbytes:
        raise ValueError("fm_chunk_push: dst smaller than src")
    _check("fm_chunk_push", lib().fm_chunk_push(
        _ptr(src) if nbytes else None, _ptr(dst) if nbytes else None, nbytes, _ptr(flag),
        _ptr(counter), ctypes.c_uint32(epoch & 0xFFFFFFFF), int(n_workgroups),
        _stream(stream)))


def fm_chunk_push_dma(src, dst, flag, epoch: int, stream=None) -> None:
    """Copy src into dst on the copy engines, then write flag = epoch."""
    nbytes = src.numel() * src.element_size() if src is not None else 0
    if src is not None and dst.numel() * dst.element_size() < nbytes:
        raise ValueError("fm_chunk_push_dma: dst smaller than src")
    _check("fm_chunk_push_dma", lib().fm_chunk_push_dma(
        _ptr(src) if nbytes else None, _ptr(dst) if nbytes else None, nbytes, _ptr(flag),
        ctypes.c_uint32(epoch & 0xFFFFFFFF), _stream(stream)))


def fm_gemm_rs(A, W, dst, rank: int, atomic: bool = False, stream=None) -> None:
    """dst[r] += (A @ W)[rows of slice r] for every rank slice r (fp32 slices)."""
    M, K = A.shape
    K2, N = W.shape
    P = len(dst)
    if K2 != K or W.dtype != A.dtype or M % P:
        raise ValueError("fm_gemm_rs: shape or dtype mismatch")
    torch = _torch()
    for d in dst:
        if d.dtype != torch.float32 or tuple(d.shape) != (M // P, N):
            raise ValueError("fm_gemm_rs: each slice must be fp32 [M/n_ranks, N]")
    ptrs = (ctypes.c_void_p * P)(*[_ptr(d) for d in dst])
    _check("fm_gemm_rs", lib().fm_gemm_rs(_dt(A), M, N, K, P, int(rank), _ptr(A), _ptr(W),
                                          ctypes.cast(ptrs, ctypes.c_void_p), int(bool(atomic)),
                                          _stream(stream)))


def fm_moe_workspace_bytes(T: int, topk: int, hidden: int, n_local: int) -> int:
    """Bytes of MoE workspace for T tokens, top-k, hidden size and local experts."""
    return int(lib().fm_moe_workspace_bytes(int(T), int(topk), int(hidden), int(n_local)))


def moe_workspace(T: int, topk: int, hidden: int, n_local: int, device="cuda:0"):
    """A zero-filled uint8 device tensor of fm_moe_workspace_bytes bytes."""
    torch = _torch()
    n = fm_moe_workspace_bytes(T, topk, hidden, n_local)
    if n <= 0:
        raise ValueError("fm_moe_workspace_bytes: arguments out of range")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _ws(ws):
    """(pointer, bytes) of a workspace tensor."""
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def fm_moe_route(topk_ids, expert_begin: int, n_local: int, sorted_pairs, expert_offsets, ws,
                 stream=None) -> None:
    T, topk = topk_ids.shape
    wp, wn = _ws(ws)
    _check("fm_moe_route", lib().fm_moe_route(T, topk, int(expert_begin), int(n_local),
                                              _ptr(topk_ids), _ptr(sorted_pairs),
                                              _ptr(expert_offsets), wp, wn, _stream(stream)))


def fm_moe_gather_gemm(X, topk_ids, W1, H, sorted_pairs, expert_offsets, expert_begin: int,
                       ws, stream=None) -> None:
    """Route, then H[rows of expert e] = X[gathered tokens] @ W1[e]."""
    T, hidden = X.shape
    n_local, h2, ffn = W1.shape
    topk = topk_ids.shape[1]
    if h2 != hidden or H.shape[1] != ffn or H.shape[0] < T * topk or W1.dtype != X.dtype:
        raise ValueError("fm_moe_gather_gemm: shape or dtype mismatch")
    wp, wn = _ws(ws)
    _check("fm_moe_gather_gemm", lib().fm_moe_gather_gemm(
        _dt(X), T, hidden, ffn, topk, int(expert_begin), n_local, _ptr(X), _ptr(topk_ids),
        _ptr(W1), _ptr(H), _ptr(sorted_pairs), _ptr(expert_offsets), wp, wn, _stream(stream)))


def fm_moe_gather_gemm_act(X, topk_ids, W1, H, sorted_pairs, expert_offsets, expert_begin: int,
                           act: int, ws, stream=None) -> None:
    """fm_moe_gather_gemm with act (FM_ACT_*) applied to the fp32 result
    before it is rounded into H."""
    T, hidden = X.shape
    n_local, h2, ffn = W1.shape
    topk = topk_ids.shape[1]
    if h2 != hidden or H.shape[1] != ffn or H.shape[0] < T * topk or W1.dtype != X.dtype:
        raise ValueError("fm_moe_gather_gemm_act: shape or dtype mismatch")
    wp, wn = _ws(ws)
    _check("fm_moe_gather_gemm_act", lib().fm_moe_gather_gemm_act(
        _dt(X), T, hidden, ffn, topk, int(expert_begin), n_local, _ptr(X), _ptr(topk_ids),
        _ptr(W1), _ptr(H), _ptr(sorted_pairs), _ptr(expert_offsets), int(act), wp, wn,
        _stream(stream)))


def fm_moe_ag_gather_gemm(X, topk_ids, W1, H, sorted_pairs, expert_offsets, expert_begin: int,
                          flags, epoch: int, n_chunks: int, ws, order=None, err_word=None,
                          spin_limit: int = 0, stream=None) -> None:
    """fm_moe_gather_gemm behind a token AllGather: token chunk c of X is read
    after flags[c] >= epoch; `order` is the expected arrival order."""
    T, hidden = X.shape
    n_local, h2, ffn = W1.shape
    topk = topk_ids.shape[1]
    if h2 != hidden or H.shape[1] != ffn or H.shape[0] < T * topk or W1.dtype != X.dtype:
        raise ValueError("fm_moe_ag_gather_gemm: shape or dtype mismatch")
    order_arr = None
    if order is not None:
        order = [int(c) for c in order]
        order_arr = (ctypes.c_int32 * len(order))(*order)
    _check("fm_moe_ag_gather_gemm", lib().fm_moe_ag_gather_gemm(
        _dt(X), T, hidden, ffn, topk, int(expert_begin), n_local, _ptr(X), _ptr(topk_ids),
        _ptr(W1), _ptr(H), _ptr(sorted_pairs), _ptr(expert_offsets), int(n_chunks), _ptr(flags),
        ctypes.c_uint32(epoch & 0xFFFFFFFF),
        ctypes.cast(order_arr, ctypes.c_void_p) if order_arr is not None else None,
        _ptr(err_word), int(spin_limit), *_ws(ws), _stream(stream)))


def fm_moe_ag_gather_gemm_producers(src, X, topk_ids, W1, H, sorted_pairs, expert_offsets,
                                    expert_begin: int, flags, counters, epoch: int, ws,
                                    order=None, n_producers: int = 0, err_word=None,
                                    spin_limit: int = 0, stream=None) -> None:
    """fm_moe_ag_gather_gemm whose own producer workgroups copy token chunk c
    from src[c] (None: already in X) into X and publish flags[c] = epoch."""
    T, hidden = X.shape
    n_local, h2, ffn = W1.shape
    topk = topk_ids.shape[1]
    n = len(src)
    if (h2 != hidden or H.shape[1] != ffn or H.shape[0] < T * topk or W1.dtype != X.dtype
            or T % n or any(x is not None and (tuple(x.shape) != (T // n, hidden)
                                               or x.dtype != X.dtype) for x in src)):
        raise ValueError("fm_moe_ag_gather_gemm_producers: shape or dtype mismatch")
    ptrs = (ctypes.c_void_p * n)(*[_ptr(x) if x is not None else None for x in src])
    o = _order_arg(order)
    _check("fm_moe_ag_gather_gemm_producers", lib().fm_moe_ag_gather_gemm_producers(
        _dt(X), T, hidden, ffn, topk, int(expert_begin), n_local, _ptr(X), _ptr(topk_ids),
        _ptr(W1), _ptr(H), _ptr(sorted_pairs), _ptr(expert_offsets), n,
        ctypes.cast(ptrs, ctypes.c_void_p), _ptr(flags), _ptr(counters),
        ctypes.c_uint32(epoch & 0xFFFFFFFF),
        ctypes.cast(o, ctypes.c_void_p) if o is not None else None, int(n_producers),
        _ptr(err_word), int(spin_limit), *_ws(ws), _stream(stream)))


def fm_moe_ag_gather_gemm_pull(chunks, topk_ids, W1, H, sorted_pairs, expert_offsets,
                               expert_begin: int, flags, epoch: int, ws, order=None,
                               err_word=None, spin_limit: int = 0, stream=None) -> None:
    """MoE layer 0 reading token chunk c in place from chunks[c] after
    flags[c] >= epoch (no gathered buffer)."""
    n = len(chunks)
    Tc, hidden = chunks[0].shape
    T = n * Tc
    n_local, h2, ffn = W1.shape
    topk = topk_ids.shape[1]
    if (h2 != hidden or H.shape[1] != ffn or H.shape[0] < T * topk or topk_ids.shape[0] != T
            or any(tuple(x.shape) != (Tc, hidden) or x.dtype != W1.dtype for x in chunks)):
        raise ValueError("fm_moe_ag_gather_gemm_pull: shape or dtype mismatch")
    ptrs = (ctypes.c_void_p * n)(*[_ptr(x) for x in chunks])
    o = _order_arg(order)
    _check("fm_moe_ag_gather_gemm_pull", lib().fm_moe_ag_gather_gemm_pull(
        _dt(W1), T, hidden, ffn, topk, int(expert_begin), n_local,
        ctypes.cast(ptrs, ctypes.c_void_p), _ptr(topk_ids), _ptr(W1), _ptr(H), _ptr(sorted_pairs),
        _ptr(expert_offsets), n, _ptr(flags), ctypes.c_uint32(epoch & 0xFFFFFFFF),
        ctypes.cast(o, ctypes.c_void_p) if o is not None else None, _ptr(err_word),
        int(spin_limit), *_ws(ws), _stream(stream)))


def fm_moe_gemm_scatter(H, W2, sorted_pairs, expert_offsets, topk_weights, out, ws,
                        err_word=None, spin_limit: int = 0, stream=None) -> None:
    """out[t] += sum_k w[t,k] * (H[row(t,k)] @ W2[e(t,k)]) over local pairs."""
    T, topk = topk_weights.shape
    n_local, ffn, hidden = W2.shape
    if H.shape[1] != ffn or tuple(out.shape) != (T, hidden) or W2.dtype != H.dtype:
        raise ValueError("fm_moe_gemm_scatter: shape or dtype mismatch")
    _check("fm_moe_gemm_scatter", lib().fm_moe_gemm_scatter(
        _dt(H), T, hidden, ffn, topk, n_local, _ptr(H), _ptr(W2), _ptr(sorted_pairs),
        _ptr(expert_offsets), _ptr(topk_weights), _ptr(out), _ptr(err_word), int(spin_limit),
        *_ws(ws), _stream(stream)))


def fm_moe_gemm_scatter_noalloc(H, W2, sorted_pairs, expert_offsets, topk_weights, out,
                                err_word=None, spin_limit: int = 0, stream=None) -> None:
    """fm_moe_gemm_scatter with the library's static per-GPU scratch instead of
    a workspace (for callers that cannot allocate)."""
    T, topk = topk_weights.shape
    n_local, ffn, hidden = W2.shape
    if H.shape[1] != ffn or tuple(out.shape) != (T, hidden) or W2.dtype != H.dtype:
        raise ValueError("fm_moe_gemm_scatter_noalloc: shape or dtype mismatch")
    _check("fm_moe_gemm_scatter_noalloc", lib().fm_moe_gemm_scatter_noalloc(
        _dt(H), T, hidden, ffn, topk, n_local, _ptr(H), _ptr(W2), _ptr(sorted_pairs),
        _ptr(expert_offsets), _ptr(topk_weights), _ptr(out), _ptr(err_word), int(spin_limit),
        _stream(stream)))


def fm_probe_mfma(dtype, mfma16: bool, waves_per_simd: int, iters: int, zero: bool, out,
                  stream=None) -> None:
    """The register-only MFMA ceiling loop (include/fluxmi_probe.h); `out` is a
    device int64 tensor of at least 4 x CU-count words."""
    torch = _torch()
    dt = FM_F16 if dtype == torch.float16 else FM_BF16
    _check("fm_probe_mfma", lib().fm_probe_mfma(dt, int(bool(mfma16)), int(waves_per_simd),
                                                int(iters), int(bool(zero)), _ptr(out),
                                                out.numel() * out.element_size() // 8,
                                                _stream(stream)))
