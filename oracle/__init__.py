"""CPU oracle for the fused GEMM + tensor-parallel data-movement operators.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
reference that the GPU library is checked against.  Only ``tests/``, the
``smoke()`` check and the benchmark's CPU-baseline leg may import it; the
product path never does, and it shares no code with the HIP library.

The arithmetic lives in ``fm_oracle.c`` (fp64 accumulation, explicit gather,
scatter and reduce loops).  This module only marshals numpy arrays into it.
``full.py`` computes the same definitions for every element of the full-size
workloads, with numpy's float64 matrix product as the one library step.

Sources, by page and section:
  * FLUX paper review ("FLUX: Fast Software-based Communication Overlap On GPUs
    Through Kernel Fusion"), section 三: "核心公式" (ECT) and "MLP 前向传播"
    (Output1 = GEMM(AllGather(X), W1), Output2 = ReduceScatter(GEMM(Output1, W2))).
  * COMET article, "COMET 的技术原理": token-dimension decomposition of the MoE
    shared tensor (gather per expert, per-token weighted combine).

Every function below has a pin in ``tests/test_oracle_cpu.py`` that checks it
against something other than itself (textbook routine, closed form, invariant
or brute force).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fm_oracle.c")

F16, BF16 = 0, 1

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def lib_path(mutant: int = 0) -> str:
    name = "libfm_oracle.so" if mutant == 0 else f"libfm_oracle_mutant{mutant}.so"
    return os.path.join(_HERE, name)


def build(mutant: int = 0, out: str | None = None) -> str:
    """Compile the oracle with gcc (optionally with one planted mistake)."""
    out = out or lib_path(mutant)
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           f"-DFM_ORACLE_MUTANT={int(mutant)}", _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes view of one build of fm_oracle.c."""

    def __init__(self, path: str):
        self.path = path
        L = ctypes.CDLL(path)
        self._L = L
        L.or_f16_to_double.restype = ctypes.c_double
        L.or_f16_to_double.argtypes = [ctypes.c_uint16]
        L.or_bf16_to_double.restype = ctypes.c_double
        L.or_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.or_double_to_bf16.restype = ctypes.c_uint16
        L.or_double_to_bf16.argtypes = [ctypes.c_double]
        L.or_double_to_f16.restype = ctypes.c_uint16
        L.or_double_to_f16.argtypes = [ctypes.c_double]
        L.or_round_to_bf16.argtypes = [_i64, _p, _p]
        L.or_round_to_f16.argtypes = [_i64, _p, _p]
        L.or_gemm.argtypes = [ctypes.c_int, _i64, _i64, _i64, _p, _p, _p]
        L.or_activation.argtypes = [ctypes.c_int, _i64, _p]
        L.or_gemm_entries.argtypes = [ctypes.c_int, _i64, _i64, _i64, _p, _p, _i64, _p, _p, _p]
        L.or_ag_gemm.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _p, _p, _p, _p]
        L.or_gemm_rs.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _p, _p, _p, _p]
        L.or_moe_route.restype = _i64
        L.or_moe_route.argtypes = [_i64, _i64, _i64, _i64, _p, _p, _p]
        L.or_moe_layer0.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p]
        L.or_moe_ag_layer0.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p,
                                       _p, _p, _p, _p]
        L.or_moe_layer0_rows.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _p, _p, _p, _p,
                                         _i64, _p, _p]
        L.or_moe_layer1.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p, _p,
                                    _p, _p, _p, _p, _p]
        L.or_moe_layer1_tokens.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _i64, _p,
                                           _p, _p, _p, _p, _p, _p, _i64, _p, _p]
        L.or_ect.restype = ctypes.c_double
        L.or_ect.argtypes = [ctypes.c_double, ctypes.c_double]
        L.or_mutant_id.restype = ctypes.c_int

    # -- element formats -------------------------------------------------
    def f16_to_double(self, bits: int) -> float:
        return self._L.or_f16_to_double(int(bits))

    def bf16_to_double(self, bits: int) -> float:
        return self._L.or_bf16_to_double(int(bits))

    def decode(self, dt: int, bits: np.ndarray) -> np.ndarray:
        f = self._L.or_f16_to_double if dt == F16 else self._L.or_bf16_to_double
        flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
        return np.array([f(int(b)) for b in flat], dtype=np.float64).reshape(bits.shape)

    def round_bf16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        self._L.or_round_to_bf16(x.size, x.ctypes.data, out.ctypes.data)
        return out

    def round_f16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        self._L.or_round_to_f16(x.size, x.ctypes.data, out.ctypes.data)
        return out

    # -- O1 GEMM -----------------------------------------------------------
    def gemm(self, dt: int, A: np.ndarray, B: np.ndarray) -> np.ndarray:
        A = _u16(A)
        B = _u16(B)
        M, K = A.shape
        K2, N = B.shape
        assert K == K2
        C = np.empty((M, N), dtype=np.float64)
        self._L.or_gemm(dt, M, N, K, A.ctypes.data, B.ctypes.data, C.ctypes.data)
        return C

    def gemm_entries(self, dt: int, A: np.ndarray, B: np.ndarray, rows, cols) -> np.ndarray:
        A = _u16(A)
        B = _u16(B)
        M, K = A.shape
        N = B.shape[1]
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        out = np.empty(rows.shape[0], dtype=np.float64)
        self._L.or_gemm_entries(dt, M, N, K, A.ctypes.data, B.ctypes.data, rows.shape[0],
                                rows.ctypes.data, cols.ctypes.data, out.ctypes.data)
        return out

    # -- O2 AG-GEMM --------------------------------------------------------
    def ag_gemm(self, dt: int, chunks, W: np.ndarray, arrival=None) -> np.ndarray:
        chunks = [_u16(c) for c in chunks]
        n = len(chunks)
        Mc, K = chunks[0].shape
        W = _u16(W)
        N = W.shape[1]
        ptrs = (ctypes.c_void_p * n)(*[c.ctypes.data for c in chunks])
        arr = None
        if arrival is not None:
            arr = np.ascontiguousarray(arrival, dtype=np.int32)
            assert sorted(arr.tolist()) == list(range(n))
        C = np.empty((n * Mc, N), dtype=np.float64)
        self._L.or_ag_gemm(dt, n, Mc, N, K, ptrs, None if arr is None else arr.ctypes.data,
                           W.ctypes.data, C.ctypes.data)
        return C

    # -- O3 GEMM-RS --------------------------------------------------------
    def gemm_rs(self, dt: int, A: np.ndarray, W: np.ndarray, seeds) -> list:
        A = _u16(A)
        W = _u16(W)
        M, K = A.shape
        N = W.shape[1]
        P = len(seeds)
        assert M % P == 0
        seeds = [np.ascontiguousarray(s, dtype=np.float32) for s in seeds]
        dst = [np.empty((M // P, N), dtype=np.float64) for _ in range(P)]
        sp = (ctypes.c_void_p * P)(*[s.ctypes.data for s in seeds])
        dp = (ctypes.c_void_p * P)(*[d.ctypes.data for d in dst])
        self._L.or_gemm_rs(dt, M, N, K, P, A.ctypes.data, W.ctypes.data, sp, dp)
        return dst

    # -- O4 route ----------------------------------------------------------
    def moe_route(self, topk_ids: np.ndarray, e0: int, n_local: int):
        ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
        T, topk = ids.shape
        offsets = np.empty(n_local + 1, dtype=np.int32)
        sp = np.full(T * topk, -1, dtype=np.int32)
        rows = self._L.or_moe_route(T, topk, e0, n_local, ids.ctypes.data, offsets.ctypes.data,
                                    sp.ctypes.data)
        return offsets, sp[:rows].copy()

    # -- O5 layer 0 --------------------------------------------------------
    def moe_layer0(self, dt, X, W1, sorted_pairs, offsets, topk) -> np.ndarray:
        X = _u16(X)
        W1 = _u16(W1)
        T, hidden = X.shape
        n_local, h2, ffn = W1.shape
        assert h2 == hidden
        sp = np.ascontiguousarray(sorted_pairs, dtype=np.int32)
        off = np.ascontiguousarray(offsets, dtype=np.int32)
        H = np.empty((int(off[-1]), ffn), dtype=np.float64)
        self._L.or_moe_layer0(dt, T, hidden, ffn, topk, n_local, X.ctypes.data, W1.ctypes.data,
                              sp.ctypes.data, off.ctypes.data, H.ctypes.data)
        return H

    def activation(self, act: int, x: np.ndarray) -> np.ndarray:
        """O5a: act (0 none, 1 ReLU, 2 tanh-form GELU, 3 SiLU) of x, in fp64."""
        y = np.array(x, dtype=np.float64, order="C", copy=True)
        self._L.or_activation(int(act), y.size, y.ctypes.data)
        return y

    def moe_ag_layer0(self, dt, chunks, W1, sorted_pairs, offsets, topk, arrival=None):
        """Layer 0 on the token chunks gathered in `arrival` order (by index)."""
        chunks = [_u16(c) for c in chunks]
        n = len(chunks)
        Tc, hidden = chunks[0].shape
        W1 = _u16(W1)
        n_local, h2, ffn = W1.shape
        assert h2 == hidden
        ptrs = (ctypes.c_void_p * n)(*[c.ctypes.data for c in chunks])
        arr = None
        if arrival is not None:
            arr = np.ascontiguousarray(arrival, dtype=np.int32)
            assert sorted(arr.tolist()) == list(range(n))
        sp = np.ascontiguousarray(sorted_pairs, dtype=np.int32)
        off = np.ascontiguousarray(offsets, dtype=np.int32)
        H = np.empty((int(off[-1]), ffn), dtype=np.float64)
        self._L.or_moe_ag_layer0(dt, n, Tc, hidden, ffn, topk, n_local, ptrs,
                                 None if arr is None else arr.ctypes.data, W1.ctypes.data,
                                 sp.ctypes.data, off.ctypes.data, H.ctypes.data)
        return H

    def moe_layer0_rows(self, dt, X, W1, sorted_pairs, offsets, topk, rows) -> np.ndarray:
        X = _u16(X)
        W1 = _u16(W1)
        T, hidden = X.shape
        n_local, _, ffn = W1.shape
        sp = np.ascontiguousarray(sorted_pairs, dtype=np.int32)
        off = np.ascontiguousarray(offsets, dtype=np.int32)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.shape[0], ffn), dtype=np.float64)
        self._L.or_moe_layer0_rows(dt, hidden, ffn, topk, n_local, X.ctypes.data, W1.ctypes.data,
                                   sp.ctypes.data, off.ctypes.data, rows.shape[0],
                                   rows.ctypes.data, out.ctypes.data)
        return out

    # -- O6 layer 1 + combine ----------------------------------------------
    def moe_layer1(self, dt, H, W2, topk_ids, topk_weights, sorted_pairs, offsets, seed, e0):
        H = _u16(H)
        W2 = _u16(W2)
        ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
        wts = np.ascontiguousarray(topk_weights, dtype=np.float32)
        T, topk = ids.shape
        n_local, ffn, hidden = W2.shape
        sp = np.ascontiguousarray(sorted_pairs, dtype=np.int32)
        off = np.ascontiguousarray(offsets, dtype=np.int32)
        seed = np.ascontiguousarray(seed, dtype=np.float32)
        out = np.empty((T, hidden), dtype=np.float64)
        self._L.or_moe_layer1(dt, T, hidden, ffn, topk, e0, n_local, H.ctypes.data,
                              W2.ctypes.data, ids.ctypes.data, wts.ctypes.data, sp.ctypes.data,
                              off.ctypes.data, seed.ctypes.data, out.ctypes.data)
        return out

    def moe_layer1_tokens(self, dt, H, W2, topk_ids, topk_weights, sorted_pairs, offsets, seed,
                          e0, toks):
        H = _u16(H)
        W2 = _u16(W2)
        ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
        wts = np.ascontiguousarray(topk_weights, dtype=np.float32)
        T, topk = ids.shape
        n_local, ffn, hidden = W2.shape
        sp = np.ascontiguousarray(sorted_pairs, dtype=np.int32)
        off = np.ascontiguousarray(offsets, dtype=np.int32)
        seed = np.ascontiguousarray(seed, dtype=np.float32)
        toks = np.ascontiguousarray(toks, dtype=np.int64)
        out = np.empty((toks.shape[0], hidden), dtype=np.float64)
        self._L.or_moe_layer1_tokens(dt, T, hidden, ffn, topk, e0, n_local, H.ctypes.data,
                                     W2.ctypes.data, ids.ctypes.data, wts.ctypes.data,
                                     sp.ctypes.data, off.ctypes.data, seed.ctypes.data,
                                     toks.shape[0], toks.ctypes.data, out.ctypes.data)
        return out

    # -- ECT ---------------------------------------------------------------
    def ect(self, overall_time: float, gemm_non_split_time: float) -> float:
        return self._L.or_ect(float(overall_time), float(gemm_non_split_time))


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return np.ascontiguousarray(a)


_cache: dict = {}


def load(mutant: int = 0) -> Oracle:
    """Load (building on first use if needed) the oracle library."""
    if mutant in _cache:
        return _cache[mutant]
    path = lib_path(mutant)
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        build(mutant)
    o = Oracle(path)
    _cache[mutant] = o
    return o
