"""Host-side tests of the C-ABI library (no GPU needed): the library loads
and exports every symbol include/cp_chain.h declares, the dependency-table
builder matches the hand-derived golden graph and the structural rule of the
chain, and argument errors map to the documented codes."""
import os
import re

import pytest

from tile_dependency_pipelined_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cp_chain.h")

nat = pytest.importorskip("tile_dependency_pipelined_amd.native",
                          reason="libcpchain.so not built (python -m tile_dependency_pipelined_amd.build)")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(cp_\w+)\s*\(", src, flags=re.M)))


def test_header_symbols_exported():
    names = header_functions()
    assert set(names) == set(nat.EXPORTS), names
    for n in names:
        assert hasattr(nat.lib(), n), n  # resolves through dlsym


def test_header_constants_match_binding():
    src = open(HEADER).read()
    for name in ("CP_F32", "CP_BF16", "CP_ACT_NONE", "CP_ACT_GELU_TANH", "CP_MODE_PIPELINED",
                 "CP_MODE_SEQUENTIAL", "CP_MODE_MICROBATCH", "CP_OK", "CP_ERR_INVALID_ARG",
                 "CP_ERR_SHAPE", "CP_ERR_UNSUPPORTED", "CP_ERR_OOM", "CP_ERR_HIP", "CP_ERR_TIMEOUT",
                 "CP_ERR_NO_DEVICE", "CP_ERR_INVARIANT", "CP_MAX_LAYERS", "CP_MODE_SPATIAL",
                 "CP_TRACE_WORDS"):
        m = re.search(rf"#define\s+{name}\s+\(?(-?\d+)\)?", src)
        assert m, name
        assert int(m.group(1)) == getattr(nat, name), name
    for name in ("CP_FLAG_DEBUG", "CP_FLAG_TRACE", "CP_FLAG_POISON", "CP_FLAG_DELAY_INJECT",
                 "CP_FLAG_STARVE_LAST", "CP_FLAG_EAGER", "CP_FLAG_COOPERATIVE", "CP_FLAG_FENCE_RELEASE",
                 "CP_FLAG_TIMING", "CP_FLAG_NO_SPLIT", "CP_FLAG_LAMPORT", "CP_FLAG_EARLY_DISPATCH"):
        m = re.search(rf"#define\s+{name}\s+(\d+)u", src)
        assert m and int(m.group(1)) == getattr(nat, name), name


def read_golden(path):
    out = {"edges": {}}
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] in ("n_tiles", "n_first", "n_edges"):
            out[parts[0]] = int(parts[1])
        elif parts[0] in ("layer_off", "nsplit", "indeg"):
            out[parts[0]] = [int(x) for x in parts[1:]]
        else:
            out["edges"][int(parts[0])] = [int(x) for x in parts[1:]]
    return out


def test_tile_graph_matches_hand_derived_golden():
    gold = read_golden(os.path.join(ROOT, "tests", "golden", "c1_tile_graph.txt"))
    g = nat.cp_chain_tile_graph(128, [512, 512, 512], 64, 64)
    assert g["n_tiles"] == gold["n_tiles"]
    assert g["n_edges"] == gold["n_edges"]
    assert g["layer_off"] == gold["layer_off"]
    assert g["layer_off"][1] == gold["n_first"]
    for p, cons in gold["edges"].items():
        assert g["dep_ids"][g["dep_off"][p]:g["dep_off"][p + 1]] == cons
    assert g["indeg"] == [0] * 16 + [8] * 16


@pytest.mark.parametrize("name, M, widths", [
    ("split_consumer_tile_graph.txt", 128, [256, 256, 128]),
    ("split_producer_tile_graph.txt", 64, [256, 128, 64]),
])
def test_split_tile_graph_matches_hand_derived_golden(name, M, widths):
    gold = read_golden(os.path.join(ROOT, "tests", "golden", name))
    g = nat.cp_chain_tile_graph(M, widths, 64, 64, nsplit=gold["nsplit"])
    assert g["n_tiles"] == gold["n_tiles"]
    assert g["n_edges"] == gold["n_edges"]
    assert g["layer_off"] == gold["layer_off"]
    assert g["indeg"] == gold["indeg"]
    for p, cons in gold["edges"].items():
        assert g["dep_ids"][g["dep_off"][p]:g["dep_off"][p + 1]] == cons, p


@pytest.mark.parametrize("M, widths, bn, ns", [
    (256, [512, 1024, 512, 256], 64, [1, 4, 2]),
    (128, [1024, 512, 2048], 128, [2, 4]),
    (384, [256, 768, 384, 768], 64, [4, 2, 3]),
])
def test_split_tile_graph_rule(M, widths, bn, ns):
    """Any split: item s of consumer tile (l+1, i, j) depends on exactly the
    producer tiles (l, i, k) of its k range, through their first items, and
    the in-degree equals the number of those tiles."""
    g = nat.cp_chain_tile_graph(M, widths, 64, bn, nsplit=ns)
    L, nrb = len(widths) - 1, M // 64
    nbn = [w // bn for w in widths[1:]]
    off = [0]
    for l in range(L):
        off.append(off[-1] + nrb * nbn[l] * ns[l])
    assert g["layer_off"] == off
    item = lambda l, i, j, s: off[l] + (i * nbn[l] + j) * ns[l] + s
    want = set()
    for l in range(L - 1):
        per = nbn[l] // ns[l + 1]
        for i in range(nrb):
            for k in range(nbn[l]):
                for j in range(nbn[l + 1]):
                    want.add((item(l, i, k, 0), item(l + 1, i, j, k // per)))
    got = set()
    for p in range(g["n_tiles"]):
        for c in g["dep_ids"][g["dep_off"][p]:g["dep_off"][p + 1]]:
            assert (p, c) not in got
            got.add((p, c))
    assert got == want and g["n_edges"] == len(want)
    indeg = [0] * g["n_tiles"]
    for _, c in want:
        indeg[c] += 1
    assert g["indeg"] == indeg


def test_split_tile_graph_rejects_bad_splits():
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_tile_graph(128, [256, 256, 128], 64, 64, nsplit=[1, 3])   # 3 does not divide 4
    assert e.value.code == nat.CP_ERR_SHAPE
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_tile_graph(128, [256, 256, 128], 64, 64, nsplit=[0, 1])
    assert e.value.code == nat.CP_ERR_SHAPE


def check_graph_rule(M, widths, bm, bn):
    g = nat.cp_chain_tile_graph(M, widths, bm, bn)
    L = len(widths) - 1
    nrb = M // bm
    nbn = [w // bn for w in widths[1:]]
    off = [0]
    for l in range(L):
        off.append(off[-1] + nrb * nbn[l])
    assert g["layer_off"] == off
    T = off[-1]
    assert g["n_tiles"] == T
    edges = set()
    for p in range(T):
        for c in g["dep_ids"][g["dep_off"][p]:g["dep_off"][p + 1]]:
            assert (p, c) not in edges
            edges.add((p, c))
    # expected edge set from the rule: (l, i, k) -> (l+1, i, j) for all k, j
    want = set()
    for l in range(L - 1):
        for i in range(nrb):
            for k in range(nbn[l]):
                for j in range(nbn[l + 1]):
                    want.add((off[l] + i * nbn[l] + k, off[l + 1] + i * nbn[l + 1] + j))
    assert edges == want
    assert g["n_edges"] == len(want)
    indeg = [0] * T
    for _, c in edges:
        indeg[c] += 1
    assert g["indeg"] == indeg
    return g


@pytest.mark.parametrize("M,widths,bm,bn", [
    (128, [512, 512, 512], 64, 64),
    (512, [4096, 4096, 4096], 128, 128),
    (256, [64, 192, 128, 320], 64, 64),
    (64, [64, 64], 64, 64),
    (256, [128] * 9, 128, 64),
])
def test_tile_graph_rule(M, widths, bm, bn):
    check_graph_rule(M, widths, bm, bn)


@pytest.mark.parametrize("key,bm,bn,T,E,indeg", [
    ("c2", 256, 256, 64, 512, 16), ("c2", 128, 128, 256, 4096, 32),
    ("c3", 256, 256, 512, 8192, 32), ("c3", 128, 128, 2048, 65536, 64),
    ("c4", 256, 256, 512, 12288, 32), ("c4", 128, 128, 2048, 98304, 64),
    ("c5", 256, 256, 144, 3584, 112), ("c5", 64, 256, 576, 14336, 112),
])
def test_tile_graph_counts_for_workloads(key, bm, bn, T, E, indeg):
    cfg = gen.CONFIGS[key]
    g = nat.cp_chain_tile_graph(cfg.M, list(cfg.widths), bm, bn)
    assert (g["n_tiles"], g["n_edges"]) == (T, E)
    assert max(g["indeg"]) == indeg


def test_error_codes_without_device():
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_tile_graph(100, [512, 512], 64, 64)
    assert e.value.code == nat.CP_ERR_SHAPE
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_tile_graph(128, [512, 500], 64, 64)
    assert e.value.code == nat.CP_ERR_SHAPE
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_tile_graph(128, [512] * 10, 64, 64)
    assert e.value.code == nat.CP_ERR_INVALID_ARG
    # unsupported tile is rejected before any device work
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(128, [512, 512], nat.CP_BF16, 96, 64)
    assert e.value.code == nat.CP_ERR_UNSUPPORTED
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(128, [512, 512], nat.CP_F32, 128, 128)
    assert e.value.code == nat.CP_ERR_UNSUPPORTED
    # k not a multiple of the k step (64 for bf16; 128 for 256x256 tiles)
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(128, [96, 512], nat.CP_BF16, 64, 64)
    assert e.value.code == nat.CP_ERR_SHAPE
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(256, [320, 256], nat.CP_BF16, 256, 256)
    assert e.value.code == nat.CP_ERR_SHAPE
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(128, [512, 512], 7, 64, 64)
    assert e.value.code == nat.CP_ERR_INVALID_ARG
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(128, [512, 512], nat.CP_BF16, 64, 64, flags=1 << 12)
    assert e.value.code == nat.CP_ERR_INVALID_ARG
    # two release protocols at once
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(128, [512, 512], nat.CP_BF16, 64, 64,
                          flags=nat.CP_FLAG_LAMPORT | nat.CP_FLAG_FENCE_RELEASE)
    assert e.value.code == nat.CP_ERR_INVALID_ARG
    # early dispatch without the sentinel: consumers would read unstored data
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(128, [512, 512, 512], nat.CP_BF16, 64, 64, flags=nat.CP_FLAG_EARLY_DISPATCH)
    assert e.value.code == nat.CP_ERR_INVALID_ARG and "LAMPORT" in str(e.value)
    assert nat.error_string(nat.CP_ERR_TIMEOUT)
    assert nat.error_string(12345) == "unknown status"


def test_plan_without_device_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is visible")
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(128, [512, 512, 512], nat.CP_F32, 64, 64)
    assert e.value.code == nat.CP_ERR_NO_DEVICE


def test_destroy_null_is_noop():
    assert nat.lib().cp_chain_destroy(None) == 0
    assert nat.lib().cp_chain_run(None, None, None, None, None, 0, 0) == nat.CP_ERR_INVALID_ARG


@pytest.mark.parametrize("key,bound", [("c1", "mfma"), ("c2", "mfma"), ("c3", "mfma"), ("c4", "mfma"),
                                       ("c5", "hbm")])
def test_bench_roofline_bound(key, bound):
    """The benchmark reports the roofline that bounds each workload: its
    arithmetic intensity (algorithmic flops over X + sum W + Y bytes) against
    the ridge point of the element type's peak and 8 TB/s.  C5 (254 flop/B)
    sits below the bf16 ridge (312.5 flop/B); the others above theirs."""
    import bench
    cfg = gen.CONFIGS[key]
    peak = bench.PEAK_BF16_TFLOPS if cfg.dtype == gen.BF16 else bench.PEAK_FP32_TFLOPS
    b, achieved, peak_b, unit, intensity = bench.roofline(cfg.flops, cfg.min_bytes(), 1.0, peak)
    assert b == bound
    if b == "hbm":
        assert unit == "GB/s" and peak_b == bench.PEAK_HBM_GBS
        assert achieved == pytest.approx(cfg.min_bytes() / 1e-3 / 1e9)
    else:
        assert unit == "TFLOP/s" and peak_b == peak
        assert achieved == pytest.approx(cfg.flops / 1e-3 / 1e12)
    if key == "c5":
        assert intensity == pytest.approx(253.7, abs=0.5)


@pytest.mark.parametrize("case,code", [
    ("empty M", nat.CP_ERR_SHAPE), ("negative M", nat.CP_ERR_SHAPE), ("zero layers", nat.CP_ERR_INVALID_ARG),
    ("zero width", nat.CP_ERR_SHAPE), ("row longer than 2^22", nat.CP_ERR_SHAPE)])
def test_degenerate_shapes_rejected(case, code):
    """Empty and degenerate chains are refused with the documented codes,
    by the host-only graph builder and by the planner before any device
    work; nothing is launched for them."""
    M, widths = {"empty M": (0, [512, 512]), "negative M": (-64, [512, 512]),
                 "zero layers": (128, [512]), "zero width": (128, [512, 0]),
                 "row longer than 2^22": (128, [1 << 23, 512])}[case]
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_tile_graph(M, widths, 64, 64)
    assert e.value.code == code
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_plan(M, widths, nat.CP_BF16, 64, 64)
    assert e.value.code == code


def test_null_handles_rejected():
    """Calls on a NULL plan return CP_ERR_INVALID_ARG (destroy is a no-op)."""
    for call in (lambda: nat.cp_chain_run(None, 0, [0], 0, None, nat.CP_MODE_PIPELINED),
                 lambda: nat.cp_chain_stats(None), lambda: nat.cp_chain_trace(None, 4),
                 lambda: nat.cp_chain_intermediate(None, 1, 0, 0)):
        with pytest.raises(nat.CpError) as e:
            call()
        assert e.value.code == nat.CP_ERR_INVALID_ARG


@pytest.mark.parametrize("M, widths, nsplit", [
    (64, [64, 1 << 22, 1 << 22], None),          # 2^16 tiles per layer, 2^32 edges
    (1 << 14, [64, 1 << 20, 1 << 20], None),     # 2^28 tiles per layer, 2^40 edges
    (1 << 16, [1 << 22, 1 << 16], [1 << 12]),    # 2^20 tiles x 2^12 items each = 2^32 items
])
def test_graph_size_overflow_rejected(M, widths, nsplit):
    """Shapes inside the per-dimension limits whose tile graph would not fit
    32-bit indices (edges or work items beyond 2^31) are refused with
    CP_ERR_SHAPE before anything is built, by the host-only builder and by
    the planner, instead of overflowing the edge offsets."""
    with pytest.raises(nat.CpError) as e:
        nat.cp_chain_tile_graph(M, widths, 64, 64, nsplit=nsplit)
    assert e.value.code == nat.CP_ERR_SHAPE
    assert "too large" in nat.cp_chain_last_error()
    if nsplit is None:
        with pytest.raises(nat.CpError) as e:
            nat.cp_chain_plan(M, widths, nat.CP_BF16, 64, 64)
        assert e.value.code == nat.CP_ERR_SHAPE


def test_microbatch_chunks_and_tile():
    """The micro-batched baseline needs at least two row chunks, each a
    multiple of the tile height that divides M; where the timed tile spans
    the batch (256-row tiles on a 256-row batch) its plan takes tiles of half
    the height."""
    from tile_dependency_pipelined_amd import inputs as gen, tuning
    assert tuning.chunk_sweep(2048, 256) == [256, 512, 1024]
    assert tuning.chunk_sweep(256, 256) == []
    assert tuning.microbatch_tile(256, (256, 128)) == (128, 128)
    assert tuning.microbatch_tile(2048, (256, 256)) == (256, 256)
    for key, tile in tuning.TILES.items():
        cfg = gen.CONFIGS[key]
        mb = tuning.microbatch_tile(cfg.M, tile)
        chunks = tuning.chunk_sweep(cfg.M, mb[0])
        assert chunks and all(cfg.M % c == 0 and c % mb[0] == 0 and c < cfg.M for c in chunks), (key, mb, chunks)
