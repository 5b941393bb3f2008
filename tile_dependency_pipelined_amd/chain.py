"""Torch-facing wrapper of the C ABI: a plan object that takes device tensors.

PyTorch supplies device memory and streams only; every arithmetic step runs
in libcpchain.so.
"""
import torch

from . import native as nat

DTYPES = {nat.CP_F32: torch.float32, nat.CP_BF16: torch.bfloat16}
MODES = {"pipelined": nat.CP_MODE_PIPELINED, "sequential": nat.CP_MODE_SEQUENTIAL,
         "microbatch": nat.CP_MODE_MICROBATCH, "spatial": nat.CP_MODE_SPATIAL}


class Chain:
    """A planned GEMM chain Y = act_L(...act_1(X W_1)...W_L) on the current device."""

    def __init__(self, M, widths, dtype, tile_m, tile_n, acts=None, flags=0):
        self.M = int(M)
        self.widths = [int(w) for w in widths]
        self.dtype = int(dtype)
        self.tile = (int(tile_m), int(tile_n))
        self.acts = list(acts) if acts is not None else None
        self.flags = int(flags)
        self.handle = nat.cp_chain_plan(M, widths, dtype, tile_m, tile_n, acts, flags)
        g = nat.cp_chain_stats(self.handle)
        self.n_tiles = g["n_tiles"]
        self.n_workers = g["n_workers"]
        self.n_edges = g["n_edges"]

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def _check_tensor(self, t, shape, name):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a device tensor")
        if t.dtype != self.torch_dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {self.torch_dtype} tensor of shape {shape}, "
                             f"got {t.dtype} {tuple(t.shape)}")

    def run(self, X, Ws, Y, mode="pipelined", microbatch_rows=0, stream=None):
        L = len(self.widths) - 1
        if len(Ws) != L:
            raise ValueError(f"expected {L} weights")
        self._check_tensor(X, (self.M, self.widths[0]), "X")
        for l, w in enumerate(Ws):
            self._check_tensor(w, (self.widths[l], self.widths[l + 1]), f"W[{l}]")
        self._check_tensor(Y, (self.M, self.widths[-1]), "Y")
        s = stream if stream is not None else torch.cuda.current_stream()
        m = MODES[mode] if isinstance(mode, str) else int(mode)
        nat.cp_chain_run(self.handle, X.data_ptr(), [w.data_ptr() for w in Ws], Y.data_ptr(),
                         s.cuda_stream, m, microbatch_rows)
        return Y

    def stats(self, check=True):
        return nat.cp_chain_stats(self.handle, check=check)

    def trace(self):
        return nat.cp_chain_trace(self.handle, self.n_tiles)

    def intermediate(self, layer):
        """Intermediate C_layer (1 <= layer < L) of the last run as a new device tensor."""
        out = torch.empty((self.M, self.widths[layer]), dtype=self.torch_dtype, device="cuda")
        nat.cp_chain_intermediate(self.handle, layer, out.data_ptr(), out.numel() * out.element_size())
        return out

    def close(self):
        if self.handle:
            nat.cp_chain_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def to_device(a, dtype, device="cuda"):
    """Upload a numpy array (float32, or uint16 bf16 bit patterns) as a tensor."""
    import numpy as np
    if dtype == nat.CP_BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def to_host(t, dtype):
    """Download a result tensor as float32 values or uint16 bf16 bit patterns."""
    import numpy as np
    if dtype == nat.CP_BF16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy()
