"""GPU parity tests: the HIP path, called through the C ABI, against the CPU
oracle on the same seeded inputs; bit-exact agreement between the pipelined,
sequential and micro-batched modes; exact scoreboard/queue invariants.

Tolerances: max|err|/max|ref| <= 1e-4 for fp32 chains and <= 2e-2 for bf16
chains (fp32 accumulation, bf16 storage of every intermediate)."""
import sys

import numpy as np
import pytest

import oracle
from tile_dependency_pipelined_amd import inputs as gen
from tile_dependency_pipelined_amd import tuning

pytestmark = pytest.mark.gpu

TOL = {gen.F32: 1e-4, gen.BF16: 2e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def rt():
    import torch
    from tile_dependency_pipelined_amd import chain, native
    assert torch.cuda.is_available()
    torch.cuda.init()
    return {"torch": torch, "chain": chain, "nat": native}


def run_modes(rt, X, Ws, dtype, tile, acts=None, flags=0, modes=("pipelined", "sequential"),
              mb_rows=None, reps=1):
    """Run the chain in each mode; return {mode: host Y} and the pipelined stats."""
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    M = X.shape[0]
    widths = [X.shape[1]] + [w.shape[1] for w in Ws]
    dX = ch.to_device(X, dtype)
    dW = [ch.to_device(w, dtype) for w in Ws]
    out, stats = {}, None
    with ch.Chain(M, widths, dtype, tile[0], tile[1], acts=acts, flags=flags) as c:
        for mode in modes:
            for rep in range(reps):
                dY = torch.full((M, widths[-1]), float("nan"), dtype=ch.DTYPES[dtype], device="cuda")
                c.run(dX, dW, dY, mode=mode,
                      microbatch_rows=(mb_rows or tile[0]) if mode == "microbatch" else 0)
                st = c.stats()
                assert st["status"] == 0, st
                if mode in ("pipelined", "spatial"):
                    check_invariants(st, flags)
                if mode == "pipelined":
                    stats = st
                y = ch.to_host(dY, dtype)
                if rep == 0:
                    out[mode] = y
                else:
                    assert np.array_equal(y.view(np.uint32 if dtype == gen.F32 else np.uint16),
                                          out[mode].view(np.uint32 if dtype == gen.F32 else np.uint16)), \
                        f"{mode} rep {rep} differs"
    return out, stats


def check_invariants(st, flags):
    T = st["n_tiles"]
    assert st["nonzero_scores"] == 0, st
    assert st["queue_is_perm"] == 1, st
    assert st["tail"] == T, st
    assert st["head"] >= T, st
    assert st["queues_drained"] == 1, st
    assert st["nonzero_arrivals"] == 0, st
    if flags & rt_flags()["DEBUG"]:
        assert st["bad_dequeues"] == 0, st
    if flags & rt_flags()["TRACE"]:
        assert st["order_violations"] == 0, st


def rt_flags():
    from tile_dependency_pipelined_amd import native as nat
    return {"DEBUG": nat.CP_FLAG_DEBUG, "TRACE": nat.CP_FLAG_TRACE, "POISON": nat.CP_FLAG_POISON,
            "DELAY": nat.CP_FLAG_DELAY_INJECT}


def as_values(y, dtype):
    return oracle.bf16_to_f64(y) if dtype == gen.BF16 else y.astype(np.float64)


def same_bits(a, b):
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


def all_flags():
    f = rt_flags()
    return f["DEBUG"] | f["TRACE"] | f["POISON"]


# ----------------------------------------------------------------------------- fp32

def test_c1_fp32_parity_all_modes(rt):
    cfg = gen.CONFIGS["c1"]
    X, Ws = gen.config_inputs(cfg)
    say("c1: fp32 128x512x512x512, tile", cfg.tile)
    out, st = run_modes(rt, X, Ws, cfg.dtype, cfg.tile, flags=all_flags(),
                        modes=("pipelined", "sequential", "microbatch", "spatial"), mb_rows=64, reps=3)
    ref = oracle.chain(X, Ws, cfg.dtype)
    err = oracle.rel_err(as_values(out["pipelined"], cfg.dtype), ref)
    say("c1 rel err", err, "stats", st)
    assert err <= TOL[gen.F32]
    assert same_bits(out["pipelined"], out["sequential"])
    assert same_bits(out["pipelined"], out["microbatch"])
    assert same_bits(out["pipelined"], out["spatial"])
    # 16 tiles per layer leave most compute units idle, so the plan splits
    # both fp32 layers along k (items of at least 128 k, k-range dependencies)
    assert st["nsplit"][0] > 1 and st["nsplit"][1] > 1, st["nsplit"]
    assert st["nonzero_arrivals"] == 0
    # unsplit, the plan uses exactly the hand-derived C1 tile graph
    nat = rt["nat"]
    out1, st1 = run_modes(rt, X, Ws, cfg.dtype, cfg.tile, flags=all_flags() | nat.CP_FLAG_NO_SPLIT,
                          modes=("pipelined", "sequential"), reps=2)
    assert st1["n_tiles"] == 32 and st1["n_edges"] == 128
    assert oracle.rel_err(as_values(out1["pipelined"], cfg.dtype), ref) <= TOL[gen.F32]
    assert same_bits(out1["pipelined"], out1["sequential"])


def test_fp32_split_many_partials(rt):
    """An fp32 layer with two tiles and k = 4096 is split into 32 items of
    128 k each, so the last item to arrive sums its partials in several
    groups of loads, in split order: every mode gives the same bits, the
    result matches the oracle, and the arrival counters end at 0."""
    M, widths = 128, (4096, 64, 64)
    X, Ws = gen.chain_inputs(M, widths, gen.F32, 1.0, (1 / 64, 1 / 8), 93)
    say("fp32 split-K chain with many partials", M, widths)
    out, st = run_modes(rt, X, Ws, gen.F32, (64, 64), flags=all_flags(),
                        modes=("pipelined", "sequential", "microbatch"), mb_rows=64, reps=2)
    say("nsplit", st["nsplit"], "items", st["n_tiles"])
    assert st["nsplit"][0] > 4, st["nsplit"]
    ref = oracle.chain(X, Ws, gen.F32)
    assert oracle.rel_err(as_values(out["pipelined"], gen.F32), ref) <= TOL[gen.F32]
    for m in ("sequential", "microbatch"):
        assert same_bits(out["pipelined"], out[m]), m


# ----------------------------------------------------------------------------- bf16 small

BF16_TILES = [(256, 256), (256, 128), (128, 256), (128, 128), (256, 64), (64, 256), (128, 64),
              (64, 128), (64, 64)]


@pytest.mark.parametrize("tile", BF16_TILES, ids=[f"{a}x{b}" for a, b in BF16_TILES])
def test_bf16_small_parity(rt, tile):
    bm, bn = tile
    M = 3 * bm
    # an odd number of 64-k slabs exercises the k loop's remainder step; the
    # 256x256 body takes k in steps of 128 (two slabs) and has none
    k0 = 384 if tile == (256, 256) else 320
    widths = (k0, 3 * bn, 2 * bn)
    say("bf16 small", tile, M, widths)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / np.sqrt(k0), 1 / np.sqrt(3 * bn)), 50)
    out, st = run_modes(rt, X, Ws, gen.BF16, tile, flags=all_flags(),
                        modes=("pipelined", "sequential", "microbatch", "spatial"), mb_rows=bm)
    ref = oracle.chain(X, Ws, gen.BF16)
    err = oracle.rel_err(as_values(out["pipelined"], gen.BF16), ref)
    say("rel err", err)
    assert err <= TOL[gen.BF16]
    assert same_bits(out["pipelined"], out["sequential"])
    assert same_bits(out["pipelined"], out["microbatch"])
    assert same_bits(out["pipelined"], out["spatial"])


@pytest.mark.parametrize("release", ["write-through", "fence"])
@pytest.mark.parametrize("dtype", [gen.F32, gen.BF16], ids=["f32", "bf16"])
def test_signed_permutation_chain_exact_with_poison(rt, dtype, release):
    """X . P1 D1 . P2 D2 . P3 D3 is exact in every element type, so the GPU
    result must equal the oracle bit for bit; intermediates are NaN-poisoned
    before every run and a quarter of producers are delayed, so a consumer
    that read an intermediate before its producers published would show.
    Both release protocols (write-through stores, or a fence per tile)."""
    f = rt_flags()
    nat = rt["nat"]
    extra = nat.CP_FLAG_FENCE_RELEASE if release == "fence" else 0
    tile = (64, 64) if dtype == gen.F32 else (128, 128)
    n = 512 if dtype == gen.F32 else 1024
    M = 4 * tile[0]
    X = gen.normal_matrix((M, n), 1.0, 60, dtype)
    Ws = [gen.signed_permutation(n, 61 + l, dtype, scale_pow2=s) for l, s in enumerate((1, -2, 0))]
    say("perm chain", dtype, tile, M, n, release)
    out, st = run_modes(rt, X, Ws, dtype, tile, flags=all_flags() | f["DELAY"] | extra,
                        modes=("pipelined", "sequential", "spatial"), reps=3)
    assert st["fenced"] == (1 if release == "fence" else 0), st
    ref = oracle.chain(X, Ws, dtype)
    assert np.array_equal(as_values(out["pipelined"], dtype), ref)
    assert np.array_equal(as_values(out["sequential"], dtype), ref)
    assert np.array_equal(as_values(out["spatial"], dtype), ref)


def lamport_flags(nat, early):
    return nat.CP_FLAG_LAMPORT | (nat.CP_FLAG_EARLY_DISPATCH if early else 0)


EARLY = pytest.mark.parametrize("early", [False, True], ids=["released", "early"])


@EARLY
@pytest.mark.parametrize("dtype", [gen.F32, gen.BF16], ids=["f32", "bf16"])
def test_lamport_release_before_store_exact(rt, dtype, early):
    """Lamport-sentinel release with a quarter of producers releasing their
    tile before storing it (stored ~20 us later): consumers do read the
    sentinel and must re-read until the data lands.  With early dispatch
    every consumer is queued once its producers have started, so it waits
    inside its k loop for their stores.  The signed-permutation chain is
    exact, so the result must equal the oracle bit for bit, in three
    consecutive runs (alternating intermediate copies, each refilled by the
    previous run's workers), and equal the sequential mode's."""
    f = rt_flags()
    nat = rt["nat"]
    tile = (64, 64) if dtype == gen.F32 else (128, 128)
    n = 512 if dtype == gen.F32 else 1024
    M = 4 * tile[0]
    X = gen.normal_matrix((M, n), 1.0, 160, dtype)
    Ws = [gen.signed_permutation(n, 161 + l, dtype, scale_pow2=s) for l, s in enumerate((1, -2, 0))]
    say("lamport perm chain", dtype, tile, M, n, "early" if early else "released")
    out, st = run_modes(rt, X, Ws, dtype, tile, flags=all_flags() | f["DELAY"] | lamport_flags(nat, early),
                        modes=("pipelined", "sequential"), reps=3)
    assert st["lamport"] == 1 and st["fenced"] == 0, st
    say("  waves that re-read a sentinel fragment in the last run:", st["lamport_rereads"])
    assert st["lamport_rereads"] > 0, st   # consumers did see the sentinel
    ref = oracle.chain(X, Ws, dtype)
    assert np.array_equal(as_values(out["pipelined"], dtype), ref)
    assert np.array_equal(as_values(out["sequential"], dtype), ref)


@pytest.mark.parametrize("case", [
    ("bf16 256x256, gelu", gen.BF16, 512, (1024, 768, 512), (256, 256), (1, 0)),
    ("bf16 128x128 split-K both layers", gen.BF16, 128, (4096, 2048, 512), (128, 128), (1, 0)),
    ("bf16 64x128 four layers", gen.BF16, 256, (256, 512, 384, 640, 256), (64, 128), (0, 1, 0, 0)),
    ("fp32 64x64 split", gen.F32, 128, (512, 512, 512), (64, 64), (0, 0)),
], ids=lambda c: c[0])
@EARLY
def test_lamport_parity(rt, case, early):
    """Lamport mode against the oracle on several bodies, split-K layers and
    GeLU, with delayed (release-before-store) producers, with and without
    early dispatch (whose split producer tiles count their items' starts on
    the arrival counter): within the bar, bit-identical to the sequential
    mode, invariants exact, in repeated runs."""
    f = rt_flags()
    nat = rt["nat"]
    name, dtype, M, widths, tile, acts = case
    L = len(widths) - 1
    X, Ws = gen.chain_inputs(M, widths, dtype, 1.0, tuple(1 / np.sqrt(w) for w in widths[:-1]), 170)
    say("lamport parity", name, "early" if early else "released")
    out, st = run_modes(rt, X, Ws, dtype, tile, acts=list(acts),
                        flags=all_flags() | f["DELAY"] | lamport_flags(nat, early),
                        modes=("pipelined", "sequential", "microbatch"), mb_rows=tile[0], reps=2)
    ref = oracle.chain(X, Ws, dtype, acts=list(acts))
    err = oracle.rel_err(as_values(out["pipelined"], dtype), ref)
    say("  rel err", err, "nsplit", st["nsplit"][:L])
    assert err <= TOL[dtype]
    assert same_bits(out["pipelined"], out["sequential"])
    assert same_bits(out["pipelined"], out["microbatch"])


@EARLY
@pytest.mark.parametrize("dtype", [gen.F32, gen.BF16], ids=["f32", "bf16"])
def test_lamport_input_negative_zero_is_data(rt, dtype, early):
    """The caller's X may hold -0.0 (the sentinel's bit pattern): only
    intermediates are checked, so a Lamport run with a third of X set to
    -0.0 completes (no watchdog) with the sequential mode's bits, with and
    without early dispatch."""
    nat = rt["nat"]
    M, widths = 256, (512, 512, 256)
    X, Ws = gen.chain_inputs(M, widths, dtype, 1.0, (1 / np.sqrt(512), 1 / np.sqrt(512)), 172)
    X = X.copy()
    neg0 = np.uint16(0x8000) if dtype == gen.BF16 else np.float32(-0.0)
    X.reshape(-1)[::3] = neg0
    tile = (64, 64) if dtype == gen.F32 else (128, 128)
    out, st = run_modes(rt, X, Ws, dtype, tile, flags=all_flags() | lamport_flags(nat, early),
                        modes=("pipelined", "sequential"), reps=2)
    assert st["status"] == 0, st
    # released only when stored, no consumer meets a sentinel, so a re-read
    # here would be X's -0.0 taken for one; with early dispatch consumers do
    # re-read intermediates still being computed, and finishing without the
    # watchdog with the sequential bits is what shows that X is not checked
    if not early:
        assert st["lamport_rereads"] == 0, st
    assert same_bits(out["pipelined"], out["sequential"])
    assert oracle.rel_err(as_values(out["pipelined"], dtype), oracle.chain(X, Ws, dtype)) <= TOL[dtype]


def test_lamport_plan_refuses_spatial_and_reads_back_its_copy(rt):
    """A Lamport plan's spatial runs are refused; cp_chain_intermediate
    returns the intermediate of the pipelined run's own copy, which equals
    the sequential run's C_1 with -0.0 stored as +0.0."""
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    M, widths = 256, (512, 1024, 256)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / np.sqrt(512), 1 / 32), 171)
    dX, dW = ch.to_device(X, gen.BF16), [ch.to_device(w, gen.BF16) for w in Ws]
    dY = torch.empty((M, widths[-1]), dtype=torch.bfloat16, device="cuda")
    acts = [gen.ACT_GELU_TANH, gen.ACT_NONE]   # GeLU makes -0.0 for large negative inputs
    with ch.Chain(M, widths, gen.BF16, 64, 128, acts=acts, flags=nat.CP_FLAG_LAMPORT) as c:
        with pytest.raises(nat.CpError) as e:
            c.run(dX, dW, dY, mode="spatial")
        assert e.value.code == nat.CP_ERR_UNSUPPORTED
        c.run(dX, dW, dY, mode="sequential")
        seq = ch.to_host(c.intermediate(1), gen.BF16)
        for _ in range(2):
            c.run(dX, dW, dY, mode="pipelined")
            lam = ch.to_host(c.intermediate(1), gen.BF16)
            assert not np.any(lam == 0x8000)
            assert np.array_equal(lam, np.where(seq == 0x8000, 0, seq))


def test_gelu_chain_small(rt):
    M, widths = 128, (256, 512, 256)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / 16, 1 / np.sqrt(512)), 70)
    acts = [gen.ACT_GELU_TANH, gen.ACT_NONE]
    out, _ = run_modes(rt, X, Ws, gen.BF16, (64, 128), acts=acts, flags=all_flags())
    ref = oracle.chain(X, Ws, gen.BF16, acts=acts)
    err = oracle.rel_err(as_values(out["pipelined"], gen.BF16), ref)
    say("gelu rel err", err)
    assert err <= TOL[gen.BF16]
    assert same_bits(out["pipelined"], out["sequential"])


# ----------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("case", [
    ("one tile, one layer", 64, (64, 64), (64, 64)),
    ("one layer", 256, (512, 1024), (128, 128)),
    ("single row-block", 128, (256, 512, 256), (128, 128)),
    ("eight layers", 256, (128, 256, 128, 256, 128, 256, 128, 256, 128), (64, 128)),
    ("widening and narrowing", 192, (64, 448, 64, 192), (64, 64)),
    ("fewer tiles than CUs", 128, (128, 128, 128), (128, 128)),
], ids=lambda c: c[0])
def test_edge_shapes(rt, case):
    name, M, widths, tile = case
    L = len(widths) - 1
    stds = tuple(1 / np.sqrt(widths[l]) for l in range(L))
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, stds, 80)
    say("edge", name)
    out, st = run_modes(rt, X, Ws, gen.BF16, tile, flags=all_flags(),
                        modes=("pipelined", "sequential", "spatial"))
    ref = oracle.chain(X, Ws, gen.BF16)
    err = oracle.rel_err(as_values(out["pipelined"], gen.BF16), ref)
    assert err <= TOL[gen.BF16], err
    assert same_bits(out["pipelined"], out["sequential"])
    assert same_bits(out["pipelined"], out["spatial"])


def test_many_tiles_many_waves(rt):
    """More tiles than persistent workers, so workers loop over several
    tiles and the last wave is ragged."""
    M, widths = 4096, (256, 1024, 320)   # 64 row-blocks of 64: 1024 + 320 tiles
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / 16, 1 / 32), 81)
    out, st = run_modes(rt, X, Ws, gen.BF16, (64, 64), flags=all_flags(), reps=2)
    say("workers", st["n_workers"], "tiles", st["n_tiles"], "fenced", st["fenced"])
    assert st["n_tiles"] > st["n_workers"]
    assert st["fenced"] == 0
    ref = oracle.chain(X, Ws, gen.BF16)
    assert oracle.rel_err(as_values(out["pipelined"], gen.BF16), ref) <= TOL[gen.BF16]
    assert same_bits(out["pipelined"], out["sequential"])


@pytest.mark.parametrize("dtype", [gen.F32, gen.BF16], ids=["f32", "bf16"])
def test_deferred_release_exact(rt, dtype):
    """More first-layer tiles than workers: a worker whose next slot is
    already filled when its tile ends releases that tile only after the next
    one has requested its first slabs (the trace marks those).  Deferred
    releases must occur, no consumer may start before any of its producers
    released (the trace order check), and the signed-permutation chain stays
    exact with NaN-poisoned intermediates and delayed producers."""
    f = rt_flags()
    M, n = 8192, 512
    tile = (64, 64)
    X = gen.normal_matrix((M, n), 1.0, 180, dtype)
    Ws = [gen.signed_permutation(n, 181 + l, dtype, scale_pow2=s) for l, s in enumerate((1, 0, -1))]
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    dX, dW = ch.to_device(X, dtype), [ch.to_device(w, dtype) for w in Ws]
    ref = oracle.chain(X, Ws, dtype)
    with ch.Chain(M, [n] * 4, dtype, tile[0], tile[1], flags=all_flags() | f["DELAY"]) as c:
        for rep in range(2):
            dY = torch.full((M, n), float("nan"), dtype=ch.DTYPES[dtype], device="cuda")
            c.run(dX, dW, dY)
            st = c.stats()
            check_invariants(st, all_flags())
            tr = np.array(c.trace(), dtype=np.uint64).reshape(-1, nat.CP_TRACE_WORDS).astype(np.int64)
            deferred = int(tr[:, 7].sum())
            say("deferred releases", deferred, "of", st["n_tiles"], "tiles;", st["n_workers"], "workers")
            assert deferred > 0
            assert np.array_equal(as_values(ch.to_host(dY, dtype), dtype), ref)


def test_trace_stamps(rt):
    """The trace holds, per tile, wall-clock stamps in protocol order (ticket
    taken <= dequeued <= body done <= released) and shader-clock stamps
    whose ratio to the wall clock is a plausible clock frequency."""
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    M, widths = 512, (512, 1024, 512)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / np.sqrt(512), 1 / 32), 85)
    dX = ch.to_device(X, gen.BF16)
    dW = [ch.to_device(w, gen.BF16) for w in Ws]
    dY = torch.empty((M, widths[-1]), dtype=torch.bfloat16, device="cuda")
    with ch.Chain(M, widths, gen.BF16, 128, 128, flags=nat.CP_FLAG_TRACE) as c:
        c.run(dX, dW, dY)
        st = c.stats()
        check_invariants(st, nat.CP_FLAG_TRACE)
        tr = np.array(c.trace(), dtype=np.uint64).reshape(-1, nat.CP_TRACE_WORDS).astype(np.int64)
    T = st["n_tiles"]
    first_layer = (M // 128) * (widths[1] // 128)
    assert tr.shape == (T, 8)
    assert tr[:, 6].max() < st["n_workers"] and set(np.unique(tr[:, 7])) <= {0, 1}
    assert (tr[:, 0] <= tr[:, 1]).all() and (tr[:, 1] < tr[:, 2]).all()
    assert (tr[:first_layer, 3] >= tr[:first_layer, 2]).all()   # producers released after their body
    assert (tr[first_layer:, 3] == 0).all()                       # last layer releases nothing
    cycles = tr[:, 5] - tr[:, 4]
    ghz = cycles / (tr[:, 2] - tr[:, 1]) * 0.1
    say("trace: shader clock GHz min %.2f median %.2f max %.2f" % (ghz.min(), np.median(ghz), ghz.max()))
    assert (cycles > 0).all() and 0.3 < np.median(ghz) < 3.0


@pytest.mark.parametrize("coop", [False, True], ids=["plain", "cooperative"])
def test_pipelined_repeats_alternate_state(rt, coop):
    """Back-to-back pipelined runs alternate between the plan's two copies of
    the scoreboard/queue state, each reset by the previous run's workers:
    every run must meet the invariants and give the same bits."""
    nat = rt["nat"]
    M, widths = 512, (256, 512, 256)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / 16, 1 / np.sqrt(512)), 83)
    flags = all_flags() | (nat.CP_FLAG_COOPERATIVE if coop else 0)
    say("alternating state copies, cooperative" if coop else "alternating state copies, plain launch")
    out, st = run_modes(rt, X, Ws, gen.BF16, (64, 64), flags=flags, modes=("pipelined",), reps=5)
    ref = oracle.chain(X, Ws, gen.BF16)
    assert oracle.rel_err(as_values(out["pipelined"], gen.BF16), ref) <= TOL[gen.BF16]


def test_pipelined_and_spatial_alternate(rt):
    """The two protocol modes use different queue layouts; switching between
    them resets the state copy for the new layout first.  Every run in an
    alternating sequence meets the invariants and gives the same bits."""
    torch, ch = rt["torch"], rt["chain"]
    M, widths = 512, (256, 512, 384, 256)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / 16, 1 / np.sqrt(512), 1 / np.sqrt(384)), 84)
    dX, dW = ch.to_device(X, gen.BF16), [ch.to_device(w, gen.BF16) for w in Ws]
    say("alternating pipelined / spatial")
    ref = None
    with ch.Chain(M, widths, gen.BF16, 64, 128, flags=all_flags()) as c:
        for mode in ("pipelined", "spatial", "spatial", "pipelined", "pipelined", "spatial", "pipelined"):
            dY = torch.full((M, widths[-1]), float("nan"), dtype=torch.bfloat16, device="cuda")
            c.run(dX, dW, dY, mode=mode)
            st = c.stats()
            check_invariants(st, all_flags())
            y = ch.to_host(dY, gen.BF16)
            if ref is None:
                ref = y
            assert same_bits(y, ref), mode
    err = oracle.rel_err(as_values(ref, gen.BF16), oracle.chain(X, Ws, gen.BF16))
    assert err <= TOL[gen.BF16]


@pytest.mark.parametrize("acts", [(gen.ACT_NONE, gen.ACT_NONE), (gen.ACT_GELU_TANH, gen.ACT_NONE)],
                         ids=["plain", "gelu"])
def test_split_k_layers(rt, acts):
    """Layers with fewer tiles than the worker grid holds are split along k:
    every item stores an fp32 partial and the last to arrive sums them in
    split order and runs the epilogue (GeLU included).  All four modes give
    the same bits, the arrival counters end at 0, and the result matches the
    oracle; with CP_FLAG_NO_SPLIT it matches the oracle too."""
    nat = rt["nat"]
    M, widths = 128, (4096, 2048, 512)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / 64, 1 / np.sqrt(2048)), 85)
    say("split-K chain", M, widths, acts)
    out, st = run_modes(rt, X, Ws, gen.BF16, (128, 128), acts=list(acts), flags=all_flags(),
                        modes=("pipelined", "sequential", "microbatch", "spatial"), mb_rows=128, reps=2)
    say("nsplit", st["nsplit"], "items", st["n_tiles"])
    assert st["nsplit"][0] > 1 and st["nsplit"][1] > 1, st["nsplit"]
    ref = oracle.chain(X, Ws, gen.BF16, acts=list(acts))
    err = oracle.rel_err(as_values(out["pipelined"], gen.BF16), ref)
    say("split rel err", err)
    assert err <= TOL[gen.BF16]
    for m in ("sequential", "microbatch", "spatial"):
        assert same_bits(out["pipelined"], out[m]), m
    out2, st2 = run_modes(rt, X, Ws, gen.BF16, (128, 128), acts=list(acts),
                          flags=all_flags() | nat.CP_FLAG_NO_SPLIT, modes=("pipelined",))
    assert st2["nsplit"][:2] == [1, 1]
    assert oracle.rel_err(as_values(out2["pipelined"], gen.BF16), ref) <= TOL[gen.BF16]


def test_split_k_256_tiles(rt):
    """Split-K with the 256x256 body (16x16x32 blocks, k step 128): a
    two-tile first layer with k = 8192 is split four ways; every mode gives
    the same bits and the result matches the oracle."""
    M, widths = 256, (8192, 512, 256)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / np.sqrt(8192), 1 / np.sqrt(512)), 89)
    say("split-K chain, 256x256 tiles", M, widths)
    out, st = run_modes(rt, X, Ws, gen.BF16, (256, 256), acts=[gen.ACT_GELU_TANH, gen.ACT_NONE],
                        flags=all_flags(), modes=("pipelined", "sequential", "spatial"), reps=2)
    say("nsplit", st["nsplit"], "items", st["n_tiles"])
    assert st["nsplit"][0] > 1, st["nsplit"]
    ref = oracle.chain(X, Ws, gen.BF16, acts=[gen.ACT_GELU_TANH, gen.ACT_NONE])
    assert oracle.rel_err(as_values(out["pipelined"], gen.BF16), ref) <= TOL[gen.BF16]
    for m in ("sequential", "spatial"):
        assert same_bits(out["pipelined"], out[m]), m


@pytest.mark.parametrize("nsplit", [2, 4])
@pytest.mark.parametrize("tile", BF16_TILES, ids=[f"{a}x{b}" for a, b in BF16_TILES])
def test_split_k_two_and_four_partials(rt, tile, nsplit):
    """Two or four partials per split tile take the software-pipelined sum,
    whose unit size depends on the tile's wave sub-tile and MFMA block: on
    every bf16 tile shape, a one-row-block chain whose first layer has two
    tiles and 16 k steps per item (k = 16 k-step x nsplit) is split exactly
    nsplit ways.  Pipelined and sequential runs give the same bits, the
    result matches the oracle, and the arrival counters end at 0."""
    bm, bn = tile
    k_step = 128 if tile == (256, 256) else 64
    K0 = 16 * k_step * nsplit
    M, widths = bm, (K0, 2 * bn, bn)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / np.sqrt(K0), 1 / np.sqrt(2 * bn)), 97 + nsplit)
    say("split-K sum", tile, "nsplit", nsplit, M, widths)
    out, st = run_modes(rt, X, Ws, gen.BF16, tile, acts=[gen.ACT_GELU_TANH, gen.ACT_NONE], flags=all_flags(),
                        modes=("pipelined", "sequential"), reps=2)
    assert st["nsplit"][0] == nsplit and st["nsplit"][1] == 1, st["nsplit"]
    ref = oracle.chain(X, Ws, gen.BF16, acts=[gen.ACT_GELU_TANH, gen.ACT_NONE])
    assert oracle.rel_err(as_values(out["pipelined"], gen.BF16), ref) <= TOL[gen.BF16]
    assert same_bits(out["pipelined"], out["sequential"])


def test_split_k_many_partials(rt):
    """A long-k layer with two tiles is split into 16 items per tile, so the
    last item to arrive sums its partials in several groups of loads; the
    sum keeps split order, so every mode gives the same bits."""
    M, widths = 128, (16384, 256, 256)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / 128, 1 / 16), 87)
    say("split-K chain with many partials", M, widths)
    out, st = run_modes(rt, X, Ws, gen.BF16, (128, 128), acts=[gen.ACT_GELU_TANH, gen.ACT_NONE],
                        flags=all_flags(), modes=("pipelined", "sequential", "microbatch"), mb_rows=128, reps=2)
    say("nsplit", st["nsplit"], "items", st["n_tiles"])
    assert st["nsplit"][0] >= 8, st["nsplit"]
    ref = oracle.chain(X, Ws, gen.BF16, acts=[gen.ACT_GELU_TANH, gen.ACT_NONE])
    assert oracle.rel_err(as_values(out["pipelined"], gen.BF16), ref) <= TOL[gen.BF16]
    for m in ("sequential", "microbatch"):
        assert same_bits(out["pipelined"], out[m]), m


def test_rejects_bad_shapes_on_device(rt):
    nat = rt["nat"]
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(100, [256, 256], nat.CP_BF16, 64, 64)
    assert e.value.code == nat.CP_ERR_SHAPE


def test_watchdog_timeout_is_reported(rt):
    """A consumer that never becomes ready ends the run through the worker's
    own bounded wait (50 ms with this test flag) with CP_ERR_TIMEOUT."""
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    M, widths = 128, (128, 128, 128)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (0.1, 0.1), 90)
    dX, dW = ch.to_device(X, gen.BF16), [ch.to_device(w, gen.BF16) for w in Ws]
    dY = torch.empty((M, 128), dtype=torch.bfloat16, device="cuda")
    with ch.Chain(M, widths, gen.BF16, 64, 64, flags=nat.CP_FLAG_STARVE_LAST | nat.CP_FLAG_DEBUG) as c:
        c.run(dX, dW, dY)
        st = c.stats(check=False)
        say("watchdog stats", st)
        assert st["rc"] == nat.CP_ERR_TIMEOUT and st["status"] == nat.CP_ERR_TIMEOUT
        assert st["tail"] == st["n_tiles"] - 1 and st["queues_drained"] == 0
        # the failed run still reset the other state copy: a second run fails
        # the same way, not earlier or later
        c.run(dX, dW, dY)
        st = c.stats(check=False)
        assert st["status"] == nat.CP_ERR_TIMEOUT and st["tail"] == st["n_tiles"] - 1, st
        assert st["bad_dequeues"] == 1, st   # only the starved tile is never dequeued
        # spatial mode waits on the same never-ready tile and times out too
        c.run(dX, dW, dY, mode="spatial")
        st = c.stats(check=False)
        assert st["status"] == nat.CP_ERR_TIMEOUT and st["tail"] == st["n_tiles"] - 1, st
        # the plan is reusable afterwards in the other modes
        c.run(dX, dW, dY, mode="sequential")
        assert c.stats()["status"] == 0


# ----------------------------------------------------------------------------- workloads

def test_c2_full_parity(rt):
    cfg = gen.CONFIGS["c2"]
    tile = tuning.TILES["c2"]
    X, Ws = gen.config_inputs(cfg)
    say("c2 full, tile", tile)
    out, st = run_modes(rt, X, Ws, cfg.dtype, tile, flags=all_flags(),
                        modes=("pipelined", "sequential", "microbatch"), mb_rows=256)
    ref = oracle.chain(X, Ws, cfg.dtype)
    err = oracle.rel_err(as_values(out["pipelined"], cfg.dtype), ref)
    say("c2 rel err", err)
    assert err <= TOL[gen.BF16]
    assert same_bits(out["pipelined"], out["sequential"])
    assert same_bits(out["pipelined"], out["microbatch"])


@pytest.mark.parametrize("key", ["c3", "c4", "c5"])
def test_full_size_parity(rt, key):
    """Full-size run in the benchmark's launch configuration (its tile, the
    planner's split factors), every element of Y compared with the oracle
    over all M rows, against both readings of the intermediates' storage:
    rounded to bf16 after every layer (what the chain computes) and kept in
    fp64 (no intermediate rounding); both must meet the bf16 bar.  Each
    intermediate C_l the pipelined run stored is compared with the oracle's
    H_l as a diagnostic (and held to the same bar).  All four modes give the
    same bits, and every scoreboard/queue invariant holds."""
    torch, ch = rt["torch"], rt["chain"]
    cfg = gen.CONFIGS[key]
    tile = tuning.TILES[key]
    say(key, "generating inputs")
    X, Ws = gen.config_inputs(cfg)
    L = cfg.n_layers
    chunks = tuning.chunk_sweep(cfg.M, tile[0])
    mb = chunks[len(chunks) // 2] if chunks else tile[0]
    dX = ch.to_device(X, cfg.dtype)
    dW = [ch.to_device(w, cfg.dtype) for w in Ws]
    out, inter = {}, []
    with ch.Chain(cfg.M, cfg.widths, cfg.dtype, tile[0], tile[1], acts=list(cfg.acts),
                  flags=rt_flags()["DEBUG"]) as c:
        for mode in ("pipelined", "sequential", "spatial", "microbatch"):
            say(key, "running", mode, "tile", tile)
            dY = torch.full((cfg.M, cfg.widths[-1]), float("nan"), dtype=ch.DTYPES[cfg.dtype], device="cuda")
            c.run(dX, dW, dY, mode=mode, microbatch_rows=mb if mode == "microbatch" else 0)
            st = c.stats()
            assert st["status"] == 0, st
            if mode in ("pipelined", "spatial"):
                check_invariants(st, rt_flags()["DEBUG"])
            out[mode] = ch.to_host(dY, cfg.dtype)
            if mode == "pipelined":
                inter = [ch.to_host(c.intermediate(l), cfg.dtype) for l in range(1, L)]
    for mode in ("sequential", "spatial", "microbatch"):
        assert same_bits(out["pipelined"], out[mode]), mode
    y = as_values(out["pipelined"], cfg.dtype)
    assert np.all(np.isfinite(y))
    say(key, "oracle over all", cfg.M, "rows")
    ref, hs = oracle.chain(X, Ws, cfg.dtype, acts=list(cfg.acts), return_intermediates=True)
    err = oracle.rel_err(y, ref)
    errs_c = [oracle.rel_err(as_values(inter[l], cfg.dtype), hs[l]) for l in range(L - 1)]
    say(key, "rel err Y", err, "intermediates", errs_c)
    assert err <= TOL[gen.BF16]
    for l, e in enumerate(errs_c):
        assert e <= TOL[gen.BF16], (l + 1, e)
    del hs
    ref2 = oracle.chain(X, Ws, cfg.dtype, acts=list(cfg.acts), round_intermediates=False)
    err2 = oracle.rel_err(y, ref2)
    say(key, "rel err Y vs the unrounded-intermediate chain", err2)
    assert err2 <= TOL[gen.BF16]


def test_intermediate_readback_matches_prefix_chain(rt):
    """cp_chain_intermediate returns exactly what the chain stored as C_l:
    for a chain without split layers, C_1 equals bit for bit the output of
    the one-layer chain X . W1 (same body, same tile); layers out of range
    and short buffers are refused."""
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    M, widths = 512, (512, 1024, 512)
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, (1 / np.sqrt(512), 1 / 32), 86)
    dX, dW = ch.to_device(X, gen.BF16), [ch.to_device(w, gen.BF16) for w in Ws]
    dY = torch.empty((M, widths[-1]), dtype=torch.bfloat16, device="cuda")
    d1 = torch.empty((M, widths[1]), dtype=torch.bfloat16, device="cuda")
    flags = nat.CP_FLAG_NO_SPLIT
    with ch.Chain(M, widths, gen.BF16, 128, 128, acts=[gen.ACT_GELU_TANH, gen.ACT_NONE], flags=flags) as c:
        c.run(dX, dW, dY)
        c1 = ch.to_host(c.intermediate(1), gen.BF16)
        with pytest.raises(nat.CpError) as e:
            nat.cp_chain_intermediate(c.handle, 2, d1.data_ptr(), d1.numel() * 2)
        assert e.value.code == nat.CP_ERR_INVALID_ARG
        with pytest.raises(nat.CpError) as e:
            nat.cp_chain_intermediate(c.handle, 1, d1.data_ptr(), d1.numel() * 2 - 2)
        assert e.value.code == nat.CP_ERR_INVALID_ARG
    with ch.Chain(M, widths[:2], gen.BF16, 128, 128, acts=[gen.ACT_GELU_TANH], flags=flags) as c:
        c.run(dX, dW[:1], d1)
        c.stats()
    assert same_bits(c1, ch.to_host(d1, gen.BF16))
    ref, hs = oracle.chain(X, Ws, gen.BF16, acts=[gen.ACT_GELU_TANH, gen.ACT_NONE], return_intermediates=True)
    assert oracle.rel_err(as_values(c1, gen.BF16), hs[0]) <= TOL[gen.BF16]


@pytest.mark.parametrize("case", [
    ("split-K fp32, 64x64", 128, (512, 512, 512), gen.F32, (64, 64), [0, 0]),
    ("four layers with GeLU, 128x128", 256, (1024, 2048, 1024, 2048, 512), gen.BF16, (128, 128), [0, 1, 0, 0]),
    ("first-layer backlog, deferred releases, 64x64", 8192, (512, 512, 512, 512), gen.BF16, (64, 64), [0, 0, 0]),
], ids=lambda c: c[0])
def test_repeated_runs_exact_every_protocol(rt, case):
    """One plan per release protocol (write-through, fence, Lamport,
    Lamport with early dispatch) runs the pipelined chain 100 times: every
    run keeps every invariant (counters 0, one dequeue per tile, queues a
    permutation and drained, no consumer dequeued before a producer
    released) and gives the sequential run's output bit for bit, so a race
    that shows only now and then in the protocol fails here."""
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    name, M, widths, dtype, tile, acts = case
    say(name, "M", M, "widths", widths, "tile", tile)
    stds = tuple(1 / np.sqrt(w) for w in widths[:-1])
    X, Ws = gen.chain_inputs(M, widths, dtype, 1.0, stds, 88)
    dX, dW = ch.to_device(X, dtype), [ch.to_device(w, dtype) for w in Ws]
    dY = torch.empty((M, widths[-1]), dtype=ch.DTYPES[dtype], device="cuda")
    with ch.Chain(M, widths, dtype, tile[0], tile[1], acts=acts) as c:
        c.run(dX, dW, dY, mode="sequential")
        c.stats()
        ref = ch.to_host(dY, dtype)
    dbg = rt_flags()["DEBUG"] | rt_flags()["TRACE"]
    for pname, pf in (("write-through", 0), ("fence", nat.CP_FLAG_FENCE_RELEASE),
                      ("lamport", lamport_flags(nat, False)), ("lamport, early", lamport_flags(nat, True))):
        say(name, pname)
        with ch.Chain(M, widths, dtype, tile[0], tile[1], acts=acts, flags=dbg | pf) as c:
            for r in range(100):
                dY.fill_(float("nan"))
                c.run(dX, dW, dY)
                st = c.stats()
                assert st["status"] == 0, (pname, r, st)
                check_invariants(st, dbg)
                assert same_bits(ch.to_host(dY, dtype), ref), (pname, r)


@pytest.mark.parametrize("case", [
    ("output row of 2^22 elements", 64, (64, 1 << 22), (64, 128)),
    ("contraction of 2^22 elements, split-K", 64, (1 << 22, 128, 128), (64, 128)),
], ids=lambda c: c[0])
def test_maximum_widths(rt, case):
    """Widths at the plan's limit (2^22 elements per row): the per-lane
    32-bit offsets of the direct loads (row x width x 2 bytes) and the
    buffer ranges are at their largest.  Pipelined and sequential give the
    same bits, and the oracle agrees: on 2048 sampled columns and the last
    tile's columns of the wide output (one layer, columns independent), on
    every element of the long-contraction chain."""
    torch, ch, nat = rt["torch"], rt["chain"], rt["nat"]
    name, M, widths, tile = case
    say(name, "M", M, "widths", widths, "tile", tile, "generating inputs")
    stds = tuple(1 / np.sqrt(w) for w in widths[:-1])
    X, Ws = gen.chain_inputs(M, widths, gen.BF16, 1.0, stds, 89)
    dX, dW = ch.to_device(X, gen.BF16), [ch.to_device(w, gen.BF16) for w in Ws]
    out = {}
    with ch.Chain(M, widths, gen.BF16, tile[0], tile[1], flags=rt_flags()["DEBUG"]) as c:
        for mode in ("pipelined", "sequential"):
            say(name, "running", mode)
            dY = torch.full((M, widths[-1]), float("nan"), dtype=torch.bfloat16, device="cuda")
            c.run(dX, dW, dY, mode=mode)
            st = c.stats()
            assert st["status"] == 0, st
            if mode == "pipelined":
                check_invariants(st, rt_flags()["DEBUG"])
            out[mode] = dY
    assert torch.equal(out["pipelined"].view(torch.int16), out["sequential"].view(torch.int16))
    Y = out["pipelined"]
    if len(widths) == 2:
        rng = np.random.default_rng(5)
        cols = np.concatenate([np.sort(rng.choice(widths[1] - tile[1], 2048, replace=False)),
                               np.arange(widths[1] - tile[1], widths[1])])
        got = ch.to_host(Y[:, torch.as_tensor(cols, device="cuda")].contiguous(), gen.BF16)
        ref = oracle.chain(X, [np.ascontiguousarray(Ws[0][:, cols])], gen.BF16)
    else:
        say(name, "oracle over all", M, "rows")
        got = ch.to_host(Y, gen.BF16)
        ref = oracle.chain(X, Ws, gen.BF16)
    err = oracle.rel_err(as_values(got, gen.BF16), ref)
    say(name, "rel err", err)
    assert err <= TOL[gen.BF16]
