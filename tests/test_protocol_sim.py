"""CPU model of the pipelined chain's queue protocol under ThreadSanitizer
(no GPU): tests/sim/cp_protocol_sim.cpp runs the worker kernel's steps on
std::thread workers with seeded delays -- per-XCD queues with static first
slots, tickets, the scoreboard, batched pushes, split-K arrivals, the
exit-time reset of the other state copy over consecutive runs, the spatial
one-queue-per-layer layout, and the watchdog -- on dependency tables made by
the library's own host builder (cp_chain_tile_graph_split).  Each run must
terminate with every invariant exact and the same output as a sequential
evaluation, and TSan must report no data race on the tile data.  Planted
protocol mistakes (weakened memory orders, a skipped reset, a wrong first
slot) must each be caught.  --early runs the same protocol with early
dispatch (Lamport plans' CP_FLAG_EARLY_DISPATCH)."""
import os
import subprocess

import pytest

nat = pytest.importorskip("tile_dependency_pipelined_amd.native",
                          reason="libcpchain.so not built (python -m tile_dependency_pipelined_amd.build)")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "sim", "cp_protocol_sim.cpp")
TSAN = {"TSAN_OPTIONS": "halt_on_error=1 exitcode=66 second_deadlock_stack=1"}

# (name, M, widths, tile_m, tile_n, nsplit)
GRAPHS = {
    "fp32 128x512x512x512, split 4": (128, [512, 512, 512], 64, 64, [4, 4]),
    "2048x8192 two layers, 256x256 tiles": (2048, [8192] * 3, 256, 256, [1, 1]),
    "256x8192x28672x8192, layer 2 split 4": (256, [8192, 28672, 8192], 128, 128, [1, 4]),
    "eight layers, mixed splits": (256, [128, 256, 128, 256, 128, 256, 128, 256, 128], 64, 64,
                                   [1, 2, 1, 2, 1, 2, 1, 2]),
    "three layers, every layer split": (128, [1024, 512, 1024, 256], 64, 64, [4, 2, 4]),
}


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    d = tmp_path_factory.mktemp("sim")
    exe = str(d / "cp_protocol_sim")
    # host-only build with ThreadSanitizer (g++; no GPU code in it)
    cmd = ["g++", "-O1", "-g", "-fsanitize=thread", "-std=c++17", "-pthread", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "tile_dependency_pipelined_amd", "csrc"), SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("simulator build failed:\n" + r.stderr[-3000:])
    return {"exe": exe, "dir": d}


def graph_file(sim, name):
    M, widths, bm, bn, ns = GRAPHS[name]
    path = sim["dir"] / ("g_" + "".join(c if c.isalnum() else "_" for c in name) + ".txt")
    if not path.exists():
        g = nat.cp_chain_tile_graph(M, widths, bm, bn, nsplit=ns)
        L = len(widths) - 1
        lines = [f"{L} {M // bm}", " ".join(str(w // bn) for w in widths[1:]), " ".join(map(str, ns)),
                 " ".join(map(str, g["layer_off"])), f"{g['n_tiles']} {g['n_edges']}",
                 " ".join(map(str, g["indeg"])), " ".join(map(str, g["dep_off"])),
                 " ".join(map(str, g["dep_ids"]))]
        path.write_text("\n".join(lines) + "\n")
    return str(path)


def run_sim(sim, name, *args, timeout=300):
    env = dict(os.environ, **TSAN)
    r = subprocess.run([sim["exe"], graph_file(sim, name)] + [str(a) for a in args], capture_output=True,
                       text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout, r.stderr


@pytest.mark.parametrize("name", list(GRAPHS))
@pytest.mark.parametrize("seed", [1, 2])
def test_protocol_exact_under_tsan(sim, name, seed):
    """Per-XCD queues (eight), more items than workers, four consecutive runs
    over the two alternating state copies: every invariant exact, output
    equal to the sequential chain, no data race."""
    rc, out, err = run_sim(sim, name, "--workers", 24, "--queues", 8, "--runs", 4, "--seed", seed,
                           "--delay-us", 30, "--delay-pct", 30)
    assert rc == 0, err[-4000:]
    assert out.count(": ok,") == 4, out


@pytest.mark.parametrize("workers", [1, 3, 8])
def test_protocol_few_workers(sim, workers):
    """Fewer workers than queues (the plan then uses one queue per worker)
    and a single worker: still exact and terminating."""
    rc, out, err = run_sim(sim, "three layers, every layer split", "--workers", workers, "--runs", 3,
                           "--seed", 7)
    assert rc == 0, err[-4000:]
    assert out.count(": ok,") == 3 and f"{min(workers, 8)} queues" in out, out


@pytest.mark.parametrize("name", ["fp32 128x512x512x512, split 4", "eight layers, mixed splits"])
def test_spatial_layout(sim, name):
    """One queue per layer, each served by its own group of workers (the
    spatial mode's layout): exact, terminating, race-free."""
    rc, out, err = run_sim(sim, name, "--spatial", "--workers", 16, "--runs", 3, "--seed", 5)
    assert rc == 0, err[-4000:]
    assert out.count(": ok,") == 3, out


@pytest.mark.parametrize("spatial", [False, True], ids=["xcd queues", "spatial"])
def test_watchdog_ends_a_starved_run(sim, spatial):
    """The last item's in-degree raised by one never becomes ready: the
    worker waiting for it times out, every worker exits, only that item is
    never dequeued, and the next run (on the reset other copy) does the same."""
    extra = ["--spatial"] if spatial else []
    rc, out, err = run_sim(sim, "fp32 128x512x512x512, split 4", "--starve", "--timeout-ms", 150,
                           "--workers", 16, "--runs", 2, *extra)
    assert rc == 0, err[-4000:]
    assert out.count("timed out, all 16 workers exited") == 2, out


@pytest.mark.parametrize("name", ["fp32 128x512x512x512, split 4", "256x8192x28672x8192, layer 2 split 4",
                                  "eight layers, mixed splits", "three layers, every layer split"])
def test_early_dispatch_exact_under_tsan(sim, name):
    """Early dispatch (Lamport plans): consumers queued once every item of
    each producer tile has started, then waiting per producer tile for its
    store: every invariant exact, output equal to the sequential chain, no
    data race on the tile data, every consumer started after all items of
    its producer tiles."""
    rc, out, err = run_sim(sim, name, "--early", "--workers", 24, "--queues", 8, "--runs", 4, "--seed", 11,
                           "--delay-us", 30, "--delay-pct", 30)
    assert rc == 0, err[-4000:]
    assert out.count(": ok,") == 4, out


@pytest.mark.parametrize("workers", [1, 2, 3, 8])
def test_early_dispatch_few_workers(sim, workers):
    """Deadlock freedom of early dispatch with fewer workers than items (down
    to one): an item is queued only when all its producers are on workers,
    so a waiting consumer never holds the worker a producer needs."""
    rc, out, err = run_sim(sim, "three layers, every layer split", "--early", "--workers", workers, "--runs", 3,
                           "--seed", 13, "--delay-us", 20, "--delay-pct", 30)
    assert rc == 0, err[-4000:]
    assert out.count(": ok,") == 3, out


def test_planted_early_dispatch_mistake_is_caught(sim):
    """Early dispatch that queues a split tile's consumers when its first
    item starts (not its last): a consumer may start before a producer item
    does, and with few workers wait for a tile whose remaining items sit
    behind it in the queue; the order check or the watchdog must catch it."""
    for workers, seed in ((2, 3), (4, 5), (8, 7)):
        rc, out, err = run_sim(sim, "three layers, every layer split", "--early", "--plant", 6, "--workers", workers,
                               "--runs", 3, "--seed", seed, "--timeout-ms", 300)
        if rc != 0:
            assert "FAIL:" in err or "ThreadSanitizer" in err, err[-2000:]
            return
    pytest.fail("planted early-dispatch mistake not caught\n" + out)


@pytest.mark.parametrize("plant, what", [
    (1, "consumer loads its counter relaxed instead of acquiring it"),
    (2, "producer decrements are relaxed (no release)"),
    (3, "split-K arrival count is relaxed"),
    (4, "the exit-time reset of the other copy is skipped"),
    (5, "first slots are computed one item off"),
])
def test_planted_protocol_mistake_is_caught(sim, plant, what):
    rc, out, err = run_sim(sim, "fp32 128x512x512x512, split 4", "--workers", 16, "--runs", 3, "--seed", 3,
                           "--plant", plant, "--timeout-ms", 300)
    assert rc != 0, f"planted mistake not caught: {what}\n{out}"
    assert "ThreadSanitizer: data race" in err or "FAIL:" in err, err[-2000:]
