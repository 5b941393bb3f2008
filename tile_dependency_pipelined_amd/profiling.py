"""Helpers for rocprofv3 evidence: summarise kernel-trace statistics and PMC
counter dumps into the short text summaries kept under profiles/, and read
back the HBM traffic figure the benchmark reports.

Traffic summaries are named traffic_<workload>_<bm>x<bn>.txt and hold
`key: value` lines, among them the SHA-256 of the kernel source they were
taken on; a summary taken on another kernel source is ignored (traffic null).
"""
import csv
import glob
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = [os.path.join(PKG, "csrc", "cp_kernels.hip"), os.path.join(PKG, "csrc", "cp_device.h")]


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
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    return out


def load_traffic(profiles_dir, workload, tile):
    path = os.path.join(profiles_dir, f"traffic_{workload}_{tile[0]}x{tile[1]}.txt")
    if not os.path.exists(path):
        return None
    kv = parse_kv(path)
    if kv.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def read_counter_csv(path):
    """Rows of a rocprofv3 counter_collection.csv as dicts."""
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(rows, kernel_substr, counter):
    """{dispatch_id: summed counter value} for dispatches whose kernel name
    contains kernel_substr."""
    acc = {}
    for r in rows:
        name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
        if kernel_substr not in name:
            continue
        if (r.get("Counter_Name") or r.get("Counter-Name")) != counter:
            continue
        d = r.get("Dispatch_Id") or r.get("Dispatch-Id")
        acc[d] = acc.get(d, 0.0) + float(r.get("Counter_Value") or r.get("Counter-Value") or 0)
    return acc


def find_one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    return hits[-1] if hits else None
