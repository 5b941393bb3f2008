"""ctypes binding of libcpchain.so -- argument marshalling only.

The functions keep the C names of include/cp_chain.h.  Every step of the
path runs in the HIP library; there is no Python or CPU fallback: if the
library is missing the import of this module raises.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcpchain.so")

CP_F32, CP_BF16 = 0, 1
CP_ACT_NONE, CP_ACT_GELU_TANH = 0, 1
CP_MODE_PIPELINED, CP_MODE_SEQUENTIAL, CP_MODE_MICROBATCH, CP_MODE_SPATIAL = 0, 1, 2, 3
CP_OK = 0
CP_ERR_INVALID_ARG = -1
CP_ERR_SHAPE = -2
CP_ERR_UNSUPPORTED = -3
CP_ERR_OOM = -4
CP_ERR_HIP = -5
CP_ERR_TIMEOUT = -6
CP_ERR_NO_DEVICE = -7
CP_ERR_INVARIANT = -8
CP_FLAG_DEBUG = 1
CP_FLAG_TRACE = 2
CP_FLAG_POISON = 4
CP_FLAG_DELAY_INJECT = 8
CP_FLAG_STARVE_LAST = 16
CP_FLAG_EAGER = 32
CP_FLAG_COOPERATIVE = 64
CP_FLAG_FENCE_RELEASE = 128
CP_FLAG_TIMING = 256
CP_FLAG_NO_SPLIT = 512
CP_FLAG_LAMPORT = 1024
CP_FLAG_EARLY_DISPATCH = 2048
CP_MAX_LAYERS = 8

# every symbol include/cp_chain.h declares
EXPORTS = ("cp_chain_plan", "cp_chain_run", "cp_chain_stats", "cp_chain_trace",
           "cp_chain_intermediate", "cp_chain_destroy", "cp_chain_run_noalloc", "cp_chain_tile_graph", "cp_chain_tile_graph_split",
           "cp_chain_error_string", "cp_chain_last_error")


class cp_chain_stats_t(ctypes.Structure):
    _fields_ = [
        ("status", ctypes.c_int32), ("mode", ctypes.c_int32), ("n_tiles", ctypes.c_int32),
        ("n_first", ctypes.c_int32), ("n_edges", ctypes.c_int32), ("n_workers", ctypes.c_int32),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("nonzero_scores", ctypes.c_int32), ("bad_dequeues", ctypes.c_int32),
        ("queue_is_perm", ctypes.c_int32), ("head", ctypes.c_uint32), ("tail", ctypes.c_uint32),
        ("n_queues", ctypes.c_int32), ("queues_drained", ctypes.c_int32),
        ("order_violations", ctypes.c_int32), ("last_run_ms", ctypes.c_double),
        ("last_kernel_ms", ctypes.c_double), ("nonzero_arrivals", ctypes.c_int32),
        ("nsplit", ctypes.c_int32 * 8), ("fenced", ctypes.c_int32), ("lamport", ctypes.c_int32),
        ("lamport_rereads", ctypes.c_int32),
    ]

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["nsplit"] = list(self.nsplit)
        return d


class CpError(RuntimeError):
    def __init__(self, code, where, detail=""):
        self.code = code
        msg = f"{where} failed: {code} ({error_string(code)})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m tile_dependency_pipelined_amd.build` "
                      "(the chain has no CPU fallback)")

# PyTorch must load its HIP runtime before this library is opened: opened
# first, the library's runtime instance and PyTorch's end up separate and the
# second one to initialise sees no device.  Loading torch first makes both
# share one runtime, so PyTorch's streams and allocations are valid here.
try:
    import torch  # noqa: F401
except ImportError:  # a C-only user of the library; its own runtime then serves
    torch = None

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _i64, _u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)

_lib.cp_chain_plan.restype = ctypes.c_int
_lib.cp_chain_plan.argtypes = [ctypes.POINTER(_vp), _i64, _i32, _pi64, _i32, _i32, _i32, _pi32, _u32]
_lib.cp_chain_run.restype = ctypes.c_int
_lib.cp_chain_run.argtypes = [_vp, _vp, ctypes.POINTER(_vp), _vp, _vp, _i32, _i64]
_lib.cp_chain_stats.restype = ctypes.c_int
_lib.cp_chain_stats.argtypes = [_vp, ctypes.POINTER(cp_chain_stats_t)]
_lib.cp_chain_trace.restype = ctypes.c_int
_lib.cp_chain_trace.argtypes = [_vp, ctypes.POINTER(ctypes.c_uint64), _i64]
_lib.cp_chain_intermediate.restype = ctypes.c_int
_lib.cp_chain_intermediate.argtypes = [_vp, _i32, _vp, _i64]
_lib.cp_chain_run_noalloc.restype = ctypes.c_int
_lib.cp_chain_run_noalloc.argtypes = [_i64, _i32, _pi64, _i32, _i32, _i32, _pi32, _vp, ctypes.POINTER(_vp), _vp,
                                      _vp, _pi32]
_lib.cp_chain_destroy.restype = ctypes.c_int
_lib.cp_chain_destroy.argtypes = [_vp]
_lib.cp_chain_tile_graph.restype = ctypes.c_int
_lib.cp_chain_tile_graph.argtypes = [_i64, _i32, _pi64, _i32, _i32, _pi32, _pi32, _pi32, _pi32,
                                     _pi32, _pi32]
_lib.cp_chain_tile_graph_split.restype = ctypes.c_int
_lib.cp_chain_tile_graph_split.argtypes = [_i64, _i32, _pi64, _i32, _i32, _pi32, _pi32, _pi32, _pi32, _pi32,
                                                _pi32, _pi32]
_lib.cp_chain_error_string.restype = ctypes.c_char_p
_lib.cp_chain_error_string.argtypes = [ctypes.c_int]
_lib.cp_chain_last_error.restype = ctypes.c_char_p
_lib.cp_chain_last_error.argtypes = []


def lib():
    return _lib


def error_string(code: int) -> str:
    return _lib.cp_chain_error_string(int(code)).decode()


def cp_chain_error_string(code: int) -> str:
    return error_string(code)


def cp_chain_last_error() -> str:
    return _lib.cp_chain_last_error().decode()


def _check(rc, where):
    if rc != CP_OK:
        raise CpError(rc, where, cp_chain_last_error())
    return rc


def _i64_array(vals):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def cp_chain_plan(M, widths, dtype, tile_m, tile_n, acts=None, flags=0):
    """Returns an opaque plan handle (int)."""
    L = len(widths) - 1
    h = _vp()
    acts_c = (ctypes.c_int32 * L)(*[int(a) for a in acts]) if acts is not None else None
    _check(_lib.cp_chain_plan(ctypes.byref(h), int(M), L, _i64_array(widths), int(dtype),
                              int(tile_m), int(tile_n), acts_c, int(flags)), "cp_chain_plan")
    return h.value


def cp_chain_run(plan, X_ptr, W_ptrs, Y_ptr, stream_ptr, mode, microbatch_rows=0):
    w = (ctypes.c_void_p * len(W_ptrs))(*[int(p) for p in W_ptrs])
    return _check(_lib.cp_chain_run(plan, int(X_ptr), w, int(Y_ptr), stream_ptr or None,
                                     int(mode), int(microbatch_rows)), "cp_chain_run")


def cp_chain_stats(plan, check=True):
    st = cp_chain_stats_t()
    rc = _lib.cp_chain_stats(plan, ctypes.byref(st))
    if check:
        _check(rc, "cp_chain_stats")
    d = st.as_dict()
    d["rc"] = rc
    return d


CP_TRACE_WORDS = 8


def cp_chain_trace(plan, n_tiles):
    buf = (ctypes.c_uint64 * (CP_TRACE_WORDS * n_tiles))()
    _check(_lib.cp_chain_trace(plan, buf, CP_TRACE_WORDS * n_tiles), "cp_chain_trace")
    return list(buf)


def cp_chain_intermediate(plan, layer, dst_ptr, capacity):
    """Copy intermediate C_layer of the last run to host or device memory at dst_ptr."""
    return _check(_lib.cp_chain_intermediate(plan, int(layer), int(dst_ptr), int(capacity)),
                  "cp_chain_intermediate")


def cp_chain_run_noalloc(M, widths, dtype, tile_m, tile_n, acts, X_ptr, W_ptrs, Y_ptr, stream_ptr, sync=True):
    """Pipelined run without a plan or any allocation.  With sync the call
    waits for the run and raises on its device status; returns the status."""
    L = len(widths) - 1
    acts_c = (ctypes.c_int32 * L)(*[int(a) for a in acts]) if acts is not None else None
    w = (ctypes.c_void_p * len(W_ptrs))(*[int(p) for p in W_ptrs])
    st = ctypes.c_int32(0)
    _check(_lib.cp_chain_run_noalloc(int(M), L, _i64_array(widths), int(dtype), int(tile_m), int(tile_n), acts_c,
                                     int(X_ptr), w, int(Y_ptr), stream_ptr or None,
                                     ctypes.byref(st) if sync else None), "cp_chain_run_noalloc")
    return st.value


def cp_chain_destroy(plan):
    if plan:
        _check(_lib.cp_chain_destroy(plan), "cp_chain_destroy")


def cp_chain_tile_graph(M, widths, tile_m, tile_n, nsplit=None):
    """Host-only dependency table: dict of n_tiles, n_edges, layer_off, indeg,
    dep_off, dep_ids (python lists).  nsplit: split-K items per tile of each
    layer (cp_chain_tile_graph_split), or None."""
    L = len(widths) - 1
    w = _i64_array(widths)
    T, E = ctypes.c_int32(), ctypes.c_int32()
    if nsplit is None:
        def call(*outs):
            return _lib.cp_chain_tile_graph(int(M), L, w, int(tile_m), int(tile_n), *outs)
        where = "cp_chain_tile_graph"
    else:
        ns = (ctypes.c_int32 * L)(*[int(x) for x in nsplit])

        def call(*outs):
            return _lib.cp_chain_tile_graph_split(int(M), L, w, int(tile_m), int(tile_n), ns, *outs)
        where = "cp_chain_tile_graph_split"
    _check(call(ctypes.byref(T), ctypes.byref(E), None, None, None, None), where)
    off = (ctypes.c_int32 * (L + 1))()
    indeg = (ctypes.c_int32 * max(T.value, 1))()
    doff = (ctypes.c_int32 * (T.value + 1))()
    dids = (ctypes.c_int32 * max(E.value, 1))()
    _check(call(ctypes.byref(T), ctypes.byref(E), off, indeg, doff, dids), where)
    return {"n_tiles": T.value, "n_edges": E.value, "layer_off": list(off),
            "indeg": list(indeg)[:T.value], "dep_off": list(doff), "dep_ids": list(dids)[:E.value]}
