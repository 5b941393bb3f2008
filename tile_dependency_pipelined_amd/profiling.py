"""Helpers for rocprofv3 evidence: summarise kernel-trace statistics and PMC
counter dumps into the short text summaries kept under profiles/, and read
back the HBM traffic figure the benchmark reports.

    python -m tile_dependency_pipelined_amd.profiling summarize \
        --workload c3 --tile 256x256 --stats <kernel_stats.csv> \
        --fetch <counter_collection.csv> --write <counter_collection.csv> \
        [--pmc <counter_collection.csv> ...] \
        --cmd "<the commands that made the inputs>" --out profiles/<name>.md

Traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, from two separate
--pmc runs) of the persistent worker kernel, each scaled by the factor that
maps the same counter of a plain 1 GiB device copy (torch's copy kernel,
reading 1 GiB and writing 1 GiB) onto its known size.  A summary records the
SHA-256 of the kernel and planner sources it was taken on; a summary taken
on other sources is ignored (traffic null).
"""
import argparse
import csv
import hashlib
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
# The kernels and the host planner: the planner picks the split-K factors,
# which change the traffic a launch moves, so a summary taken before a change
# to either no longer describes the current launch.
KERNEL_SOURCES = [os.path.join(PKG, "csrc", n) for n in ("cp_kernels.hip", "cp_device.h", "cp_chain.cpp")]
COPY_BYTES = 1 << 30
WORKER = "worker_kernel"


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse_kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip().lstrip("-* ")
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip().strip("`")] = v.strip().strip("`")
    return out


def traffic_path(profiles_dir, workload, tile):
    return os.path.join(profiles_dir, f"worker_{workload}_{tile[0]}x{tile[1]}.md")


def load_traffic(profiles_dir, workload, tile):
    path = traffic_path(profiles_dir, workload, tile)
    if not os.path.exists(path):
        return None
    kv = parse_kv(path)
    if kv.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def load_figures(profiles_dir, workload, tile, keys):
    """{key: float} of the named figures of a summary taken on the current
    sources (keys absent from it are left out), or None."""
    path = traffic_path(profiles_dir, workload, tile)
    if not os.path.exists(path):
        return None
    kv = parse_kv(path)
    if kv.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    out = {}
    for k in keys:
        try:
            out[k] = float(kv[k])
        except (KeyError, ValueError):
            pass
    return out


def read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _get(r, *names):
    for n in names:
        if n in r and r[n] != "":
            return r[n]
    return None


def counter_per_dispatch(rows, match, counter):
    """{dispatch_id: value} of `counter` for dispatches whose kernel name
    satisfies match(name)."""
    acc = {}
    for r in rows:
        name = _get(r, "Kernel_Name", "Kernel-Name") or ""
        if not match(name):
            continue
        if _get(r, "Counter_Name", "Counter-Name") != counter:
            continue
        d = _get(r, "Dispatch_Id", "Dispatch-Id")
        acc[d] = acc.get(d, 0.0) + float(_get(r, "Counter_Value", "Counter-Value") or 0)
    return acc


def is_copy(name):
    return "copy" in name.lower() and WORKER not in name


def kernel_stats(path):
    """Rows of a rocprofv3 kernel_stats.csv: name, calls, average ns."""
    out = []
    for r in read_csv(path):
        name = _get(r, "Name", "KernelName", "Kernel_Name")
        calls = _get(r, "Calls")
        avg = _get(r, "AverageNs", "Average_ns", "AverageNs(ns)")
        if name is None or avg is None:
            continue
        out.append((name, int(float(calls or 0)), float(avg)))
    return out


def summarize(args):
    lines = [f"# rocprofv3 summary: persistent worker kernel, workload {args.workload}, "
             f"tile {args.tile}", ""]
    lines.append("Commands (run from the repository root on the GPU box):")
    lines.append("")
    for c in args.cmd:
        lines.append(f"    {c}")
    lines.append("")
    kv = {"workload": args.workload, "tile": args.tile,
          "kernel_source_sha256": kernel_source_sha256()}
    if args.stats:
        st = kernel_stats(args.stats)
        lines.append("Kernel statistics (rocprofv3 --kernel-trace --stats):")
        lines.append("")
        lines.append("| kernel | calls | average us |")
        lines.append("|---|---|---|")
        for name, calls, avg in sorted(st, key=lambda x: -x[1] * x[2])[:8]:
            short = name if len(name) < 90 else name[:87] + "..."
            lines.append(f"| `{short}` | {calls} | {avg / 1e3:.1f} |")
        lines.append("")
        w = [s for s in st if WORKER in s[0]]
        if w:
            kv["worker_average_us"] = f"{w[0][2] / 1e3:.1f}"
    for tag, path, counter in (("fetch", args.fetch, "FETCH_SIZE"), ("write", args.write, "WRITE_SIZE")):
        if not path:
            continue
        rows = read_csv(path)
        wk = counter_per_dispatch(rows, lambda n: WORKER in n, counter)
        cp = counter_per_dispatch(rows, is_copy, counter)
        if not wk or not cp:
            lines.append(f"{counter}: worker or copy dispatches missing in {os.path.basename(path)}")
            continue
        w_kib = statistics.median(wk.values())
        # the 1 GiB calibration copies are the largest copy dispatches
        c_kib = statistics.median(sorted(cp.values())[-3:])
        scale = (COPY_BYTES / 1024.0) / c_kib if c_kib > 0 else float("nan")
        kv[f"{tag}_kib_per_launch_raw"] = f"{w_kib:.0f}"
        kv[f"{tag}_copy_kib_raw"] = f"{c_kib:.0f}"
        kv[f"{tag}_scale"] = f"{scale:.4f}"
        kv[f"{tag}_bytes_per_launch"] = f"{w_kib * 1024 * scale:.0f}"
    for path in args.pmc:
        rows = read_csv(path)
        names = sorted({_get(r, "Counter_Name", "Counter-Name") for r in rows} - {None})
        for counter in names:
            wk = counter_per_dispatch(rows, lambda n: WORKER in n, counter)
            if wk:
                kv[f"pmc_{counter}_per_launch"] = f"{statistics.median(wk.values()):.6g}"
    # derived figures (each counter is the worker kernel's median per dispatch;
    # SQ cycle counters of a wave count 4-cycle units, the CU ones cycles)
    def pmc(name):
        v = kv.get(f"pmc_{name}_per_launch")
        return float(v) if v is not None else None
    hit, miss = pmc("TCC_HIT_sum"), pmc("TCC_MISS_sum")
    if hit is not None and miss is not None and hit + miss > 0:
        kv["derived_l2_hit_rate"] = f"{hit / (hit + miss):.3f}"
    busy, cu = pmc("SQ_VALU_MFMA_BUSY_CYCLES"), pmc("SQ_BUSY_CU_CYCLES")
    if busy is not None and cu:
        kv["derived_mfma_busy_frac_per_simd"] = f"{busy / (4 * cu):.3f}"
    wait, wave = pmc("SQ_WAIT_ANY"), pmc("SQ_WAVE_CYCLES")
    if wait is not None and wave:
        kv["derived_wave_wait_frac"] = f"{wait / wave:.3f}"
    lds_wait = pmc("SQ_WAIT_INST_LDS")
    if lds_wait is not None and wave:
        kv["derived_wave_lds_issue_wait_frac"] = f"{lds_wait / wave:.3f}"
    # each CU's vector L1 -> L2 reads (TCP counters summed over the CUs;
    # GRBM_GUI_ACTIVE summed over the XCDs, so GUI / XCDS is the launch's
    # cycles): mean latency, reads in flight per CU (Little's law: latency
    # sum over cycles), bytes per cycle per CU (128-byte reads), and the
    # fraction of cycles a CU's L1 waited for data from the L2
    gui = pmc("GRBM_GUI_ACTIVE")
    rq, lat = pmc("TCP_TCC_READ_REQ_sum"), pmc("TCP_TCC_READ_REQ_LATENCY_sum")
    cyc = gui / args.xcds if gui else None
    if rq and lat is not None:
        kv["derived_cu_l2_read_latency_cycles"] = f"{lat / rq:.0f}"
        if cyc:
            kv["derived_cu_l2_reads_in_flight_per_cu"] = f"{lat / (args.cus * cyc):.1f}"
            kv["derived_cu_l2_read_bytes_per_cycle_per_cu"] = f"{rq * 128 / (args.cus * cyc):.1f}"
    pend = pmc("TCP_PENDING_STALL_CYCLES_sum")
    if pend is not None and cyc:
        kv["derived_cu_l1_pending_stall_frac"] = f"{pend / (args.cus * cyc):.3f}"
    # the L2's reads from memory (TCC counters summed over the channels)
    erq, elev = pmc("TCC_EA0_RDREQ_sum"), pmc("TCC_EA0_RDREQ_LEVEL_sum")
    if erq and elev is not None:
        kv["derived_l2_mem_read_latency_cycles"] = f"{elev / erq:.0f}"
        if cyc:
            kv["derived_l2_mem_reads_in_flight_per_xcd"] = f"{elev / cyc / args.xcds:.0f}"
    if "fetch_bytes_per_launch" in kv and "write_bytes_per_launch" in kv:
        kv["hbm_bytes_per_launch"] = str(int(float(kv["fetch_bytes_per_launch"]) +
                                             float(kv["write_bytes_per_launch"])))
    lines.append("Figures (key: value):")
    lines.append("")
    for k, v in kv.items():
        lines.append(f"- {k}: {v}")
    lines.append("")
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmdname", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--workload", required=True)
    s.add_argument("--tile", required=True)
    s.add_argument("--stats")
    s.add_argument("--fetch")
    s.add_argument("--write")
    s.add_argument("--pmc", action="append", default=[],
                   help="further counter_collection.csv files; the worker kernel's median per "
                        "dispatch of every counter in them is recorded")
    s.add_argument("--cmd", action="append", default=[])
    s.add_argument("--cus", type=int, default=256, help="compute units (MI355X: 256)")
    s.add_argument("--xcds", type=int, default=8, help="XCDs (MI355X: 8)")
    s.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    summarize(args)


if __name__ == "__main__":
    main()
