"""The allocation-free entry point cp_chain_run_noalloc, called through the C
ABI, against the planned entry point (cp_chain_plan + cp_chain_run,
pipelined mode) on the same seeded inputs: the same kernels, split factors
and grid, so Y must agree bit for bit, and both must meet the oracle's bar.
Calls follow one another with shapes that shrink, repeat (the second copy of
the per-run state) and change element type, since every call on a device
shares its one scratch array."""
import sys

import numpy as np
import pytest

import oracle
from tile_dependency_pipelined_amd import inputs as gen

pytestmark = pytest.mark.gpu

TOL = {gen.F32: 1e-4, gen.BF16: 2e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def rt():
    import torch
    from tile_dependency_pipelined_amd import chain, native
    assert torch.cuda.is_available()
    return {"torch": torch, "chain": chain, "nat": native}


def values(y, dtype):
    return oracle.bf16_to_f64(y) if dtype == gen.BF16 else y.astype(np.float64)


CASES = {
    # name: (dtype, M, widths, tile, acts, seed)
    "bf16 gelu 512": (gen.BF16, 512, (1024, 2048, 512), (128, 128), (gen.ACT_GELU_TANH, gen.ACT_NONE), 11),
    "bf16 smaller 256": (gen.BF16, 256, (512, 1024, 256), (128, 128), (gen.ACT_NONE, gen.ACT_NONE), 12),
    "bf16 split-K 128": (gen.BF16, 128, (4096, 2048, 512), (128, 128), (gen.ACT_GELU_TANH, gen.ACT_NONE), 13),
    "bf16 256x256 three layers": (gen.BF16, 512, (1024, 512, 768, 256), (256, 256),
                                  (gen.ACT_NONE, gen.ACT_GELU_TANH, gen.ACT_NONE), 14),
    "fp32 128x512 chain": (gen.F32, 128, (512, 512, 512), (64, 64), (gen.ACT_NONE, gen.ACT_NONE), 15),
}


def run_both(rt, name):
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    dtype, M, widths, tile, acts, seed = CASES[name]
    L = len(widths) - 1
    stds = tuple(1 / np.sqrt(widths[l]) for l in range(L))
    X, Ws = gen.chain_inputs(M, widths, dtype, 1.0, stds, seed)
    dX, dW = ch.to_device(X, dtype), [ch.to_device(w, dtype) for w in Ws]
    td = ch.DTYPES[dtype]
    y_plan = torch.full((M, widths[-1]), float("nan"), dtype=td, device="cuda")
    with ch.Chain(M, widths, dtype, tile[0], tile[1], acts=list(acts)) as c:
        c.run(dX, dW, y_plan)
        st = c.stats()
    y_na = torch.full((M, widths[-1]), float("nan"), dtype=td, device="cuda")
    stream = torch.cuda.current_stream()
    say("noalloc", name, "M", M, "widths", widths, "tile", tile, "nsplit", st["nsplit"][:L])
    status = nat.cp_chain_run_noalloc(M, widths, dtype, tile[0], tile[1], list(acts), dX.data_ptr(),
                                      [w.data_ptr() for w in dW], y_na.data_ptr(), stream.cuda_stream)
    assert status == nat.CP_OK
    a, b = ch.to_host(y_plan, dtype), ch.to_host(y_na, dtype)
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
    err = oracle.rel_err(values(b, dtype), oracle.chain(X, Ws, dtype, acts=list(acts)))
    say("  rel err", err)
    assert err <= TOL[dtype]
    return dX, dW, y_na


def test_noalloc_matches_planned_run_on_consecutive_calls(rt):
    """Two calls in a row, the second with a smaller input, then a repeat of
    that shape (the other state copy, no setup), a split-K chain, a 256x256
    three-layer chain, an fp32 chain and the first shape again: each call's
    Y equals the planned run's bit for bit."""
    for name in ("bf16 gelu 512", "bf16 smaller 256", "bf16 smaller 256", "bf16 split-K 128",
                 "bf16 256x256 three layers", "fp32 128x512 chain", "bf16 gelu 512"):
        run_both(rt, name)


def test_noalloc_async_back_to_back(rt):
    """Without a status pointer the call only enqueues: five back-to-back
    calls on the same shape and stream (alternating state copies), then one
    synchronisation; the output equals the planned run's."""
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    dX, dW, y_ref = run_both(rt, "bf16 split-K 128")
    dtype, M, widths, tile, acts, _ = CASES["bf16 split-K 128"]
    stream = torch.cuda.current_stream()
    outs = []
    for _ in range(5):
        y = torch.full((M, widths[-1]), float("nan"), dtype=torch.bfloat16, device="cuda")
        nat.cp_chain_run_noalloc(M, widths, dtype, tile[0], tile[1], list(acts), dX.data_ptr(),
                                 [w.data_ptr() for w in dW], y.data_ptr(), stream.cuda_stream, sync=False)
        outs.append(y)
    torch.cuda.synchronize()
    ref = ch.to_host(y_ref, dtype)
    for y in outs:
        assert np.array_equal(ch.to_host(y, dtype).view(np.uint8), ref.view(np.uint8))


def test_noalloc_rejects_chains_beyond_its_scratch(rt):
    """A chain whose intermediates exceed the fixed scratch is refused with
    CP_ERR_OOM before anything is launched; bad arguments keep the plan's
    codes."""
    torch, nat = rt["torch"], rt["nat"]
    x = torch.empty(64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nat.CpError) as e:   # 4096 x 8192 bf16 intermediate = 64 MiB
        nat.cp_chain_run_noalloc(4096, [8192, 8192, 8192], nat.CP_BF16, 256, 256, None, x.data_ptr(),
                                 [x.data_ptr(), x.data_ptr()], x.data_ptr(), None)
    assert e.value.code == nat.CP_ERR_OOM
    assert "64 MiB" in nat.cp_chain_last_error() or "67108864" in nat.cp_chain_last_error()
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_run_noalloc(100, [512, 512], nat.CP_BF16, 64, 64, None, x.data_ptr(), [x.data_ptr()],
                                 x.data_ptr(), None)
    assert e.value.code == nat.CP_ERR_SHAPE
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_run_noalloc(128, [512, 512], nat.CP_BF16, 64, 64, None, 0, [x.data_ptr()],
                                 x.data_ptr(), None)
    assert e.value.code == nat.CP_ERR_INVALID_ARG
