"""CPU oracle for a chain of dependent GEMMs -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP path: it is a plain fp64
triple loop in C (oracle_chain.c) behind ctypes, plus numpy marshalling.

Definition followed (CTA-Pipelining, arXiv 2607.07862): the two-layer GEMM
running example of §III-B, one GEMM per layer for longer chains (§IV-A),
Y = X A B (§IV-B), BF16 storage with an FP32 accumulator (§III-C) -- here
accumulated in fp64 -- and the tanh-GeLU between the products named in the
pith.science review's "What would settle it".
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32 = 0
BF16 = 1
ACT_NONE = 0
ACT_GELU_TANH = 1

class Oracle:
    """ctypes front end of one build of oracle_chain.c (the default build, or
    a deliberately mutated copy compiled by the planted-mistake tests)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        L.oracle_chain.restype = ctypes.c_int
        L.oracle_chain.argtypes = [
            ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_int32,
            ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int32),
            ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
            ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
        L.oracle_round_bf16_array.restype = None
        L.oracle_round_bf16_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.oracle_gelu_tanh_array.restype = None
        L.oracle_gelu_tanh_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        self.lib = L

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def chain(self, X, Ws, dtype, acts=None, round_intermediates=True, rows=None,
              return_intermediates=False):
        """Run the fp64 chain.

        X: (M, K0) float32 values, or uint16 bf16 bit patterns when dtype == BF16.
        Ws: list of (K_l, N_l) arrays of the same storage type.
        acts: per-layer activation codes (ACT_NONE / ACT_GELU_TANH) or None.
        rows: optional 1-D int array of row indices; only those rows are computed.
        Returns Y (n_rows, N_L) float64 (unrounded), plus the list of stored
        intermediates (fp64 values) when return_intermediates.
        """
        X = _storage(X, dtype)
        Ws = [_storage(w, dtype) for w in Ws]
        M, K0 = X.shape
        L = len(Ws)
        widths = [K0]
        for w in Ws:
            if w.shape[0] != widths[-1]:
                raise ValueError("inner dimensions do not chain")
            widths.append(w.shape[1])
        widths_c = (ctypes.c_int64 * (L + 1))(*widths)
        w_ptrs = (ctypes.c_void_p * L)(*[w.ctypes.data for w in Ws])
        acts_c = None
        if acts is not None:
            acts_c = (ctypes.c_int32 * L)(*[int(a) for a in acts])
        if rows is None:
            n_rows = M
            rows_c = None
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            n_rows = rows_arr.shape[0]
            rows_c = rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        Y = np.empty((n_rows, widths[-1]), dtype=np.float64)
        Hs = [np.empty((n_rows, widths[l + 1]), dtype=np.float64) for l in range(L - 1)]
        h_ptrs = (ctypes.c_void_p * max(L - 1, 1))(*([h.ctypes.data for h in Hs] or [None]))
        rc = self.lib.oracle_chain(M, L, widths_c, dtype, X.ctypes.data, w_ptrs, acts_c,
                                   1 if round_intermediates else 0, rows_c, n_rows,
                                   Y.ctypes.data, h_ptrs if Hs else None)
        if rc != 0:
            raise ValueError(f"oracle_chain rejected its arguments (rc={rc})")
        if return_intermediates:
            return Y, Hs
        return Y

    def round_bf16(self, x) -> np.ndarray:
        """fp64 -> bf16 bit patterns, round-to-nearest-even."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_round_bf16_array(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def gelu_tanh(self, x) -> np.ndarray:
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(x.shape, dtype=np.float64)
        self.lib.oracle_gelu_tanh_array(x.ctypes.data, out.ctypes.data, x.size)
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def num_threads() -> int:
    return default().num_threads()


def _storage(a: np.ndarray, dtype: int) -> np.ndarray:
    want = np.uint16 if dtype == BF16 else np.float32
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"oracle input must be {want.__name__} for dtype {dtype}, got {a.dtype}")
    return a


def chain(*args, **kwargs):
    return default().chain(*args, **kwargs)


def round_bf16(x) -> np.ndarray:
    return default().round_bf16(x)


def gelu_tanh(x) -> np.ndarray:
    return default().gelu_tanh(x)


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (marshalling only)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rel_err(got, ref) -> float:
    """max|got - ref| / max|ref|, in fp64 (the parity metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
