"""Host tests of the rocprofv3 summary helpers: on counter files with known
values, the traffic a launch moves is scaled by the 1 GiB copy, the derived
read-path figures follow their definitions, and a summary taken on other
kernel sources is not used."""
import csv
import os

from tile_dependency_pipelined_amd import profiling as pf

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
WORKER = "void cp::worker_kernel<cp::Bf16Body<256, 256, 2, 2, 4, 64, 16>, false, false>(cp::ChainArgs)"
COPY = "void at::native::elementwise_kernel<copy>"


def write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, counter, value in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def summarize(tmp_path, files, **kw):
    out = tmp_path / "s.md"
    argv = ["summarize", "--workload", "c3", "--tile", "256x256", "--out", str(out)]
    for k, v in kw.items():
        argv += [f"--{k}", str(v)]
    for flag, path in files:
        argv += [flag, str(path)]
    pf.main(argv)
    return out, pf.parse_kv(str(out))


def test_traffic_is_scaled_by_the_copy(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the copy reads 1 GiB; its FETCH_SIZE reads half of that in KiB: scale 2
    write_counters(fetch, [(1, COPY, "FETCH_SIZE", (1 << 20) / 2), (2, WORKER, "FETCH_SIZE", 1000.0),
                           (3, WORKER, "FETCH_SIZE", 1000.0)])
    write_counters(write, [(1, COPY, "WRITE_SIZE", 1 << 20), (2, WORKER, "WRITE_SIZE", 300.0)])
    out, kv = summarize(tmp_path, [("--fetch", fetch), ("--write", write)])
    assert float(kv["fetch_scale"]) == 2.0 and float(kv["write_scale"]) == 1.0
    assert int(kv["hbm_bytes_per_launch"]) == 1000 * 1024 * 2 + 300 * 1024
    # the summary carries the current sources' hash, so the bench can use it
    os.rename(out, tmp_path / "worker_c3_256x256.md")
    assert pf.load_traffic(str(tmp_path), "c3", (256, 256)) == 1000 * 1024 * 2 + 300 * 1024
    figs = pf.load_figures(str(tmp_path), "c3", (256, 256), ("fetch_scale", "write_scale", "absent"))
    assert figs == {"fetch_scale": 2.0, "write_scale": 1.0}


def test_summary_of_other_sources_is_ignored(tmp_path):
    p = tmp_path / "worker_c3_256x256.md"
    p.write_text("- kernel_source_sha256: 0000\n- hbm_bytes_per_launch: 123\n")
    assert pf.load_traffic(str(tmp_path), "c3", (256, 256)) is None
    assert pf.load_figures(str(tmp_path), "c3", (256, 256), ("hbm_bytes_per_launch",)) is None
    assert pf.load_traffic(str(tmp_path), "c5", (256, 128)) is None  # absent


def test_read_path_figures(tmp_path):
    cus, xcds = 4, 2
    cycles = 1000.0                      # launch cycles; GRBM_GUI_ACTIVE sums them over the XCDs
    reads, latency = 8000.0, 400.0       # CU -> L2 reads over all CUs, mean latency in cycles
    mreads, mlat = 500.0, 700.0          # L2 -> memory reads, mean latency
    c = tmp_path / "c.csv"
    write_counters(c, [
        (7, WORKER, "GRBM_GUI_ACTIVE", cycles * xcds),
        (7, WORKER, "TCP_TCC_READ_REQ_sum", reads),
        (7, WORKER, "TCP_TCC_READ_REQ_LATENCY_sum", reads * latency),
        (7, WORKER, "TCP_PENDING_STALL_CYCLES_sum", 0.25 * cus * cycles),
        (7, WORKER, "TCC_EA0_RDREQ_sum", mreads),
        (7, WORKER, "TCC_EA0_RDREQ_LEVEL_sum", mreads * mlat),
        (7, COPY, "TCP_TCC_READ_REQ_sum", 1e9),   # other kernels do not count
    ])
    _, kv = summarize(tmp_path, [("--pmc", c)], cus=cus, xcds=xcds)
    assert float(kv["derived_cu_l2_read_latency_cycles"]) == latency
    # Little's law: reads in flight per CU = latency sum / (CUs x cycles)
    assert float(kv["derived_cu_l2_reads_in_flight_per_cu"]) == reads * latency / (cus * cycles)
    assert float(kv["derived_cu_l2_read_bytes_per_cycle_per_cu"]) == reads * 128 / (cus * cycles)
    assert float(kv["derived_cu_l1_pending_stall_frac"]) == 0.25
    assert float(kv["derived_l2_mem_read_latency_cycles"]) == mlat
    assert float(kv["derived_l2_mem_reads_in_flight_per_xcd"]) == round(mreads * mlat / cycles / xcds)
