"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m sparse_linear_attention_hsa_amd.profiling stats <stats_dir> <out.txt> --cmd "<command>" \
        [--bench-log <log of the profiled bench run>]
    python -m sparse_linear_attention_hsa_amd.profiling traffic --fetch <dir> --write <dir> \
        --copy-fetch <dir> --copy-write <dir> --copy-bytes N --kernel <regex> --workload <name> \
        --out <out.txt> --cmd "<command>"
    python -m sparse_linear_attention_hsa_amd.profiling mfma <pmc_dir> <out.txt> --kernels <regex> ... \
        --workload <name> --cmd "<command>"

`stats` condenses a `rocprofv3 --kernel-trace --stats --output-format csv`
run into a per-kernel table (calls, average / min / max duration, share).

`mfma` turns one counter run (`--pmc SQ_VALU_MFMA_BUSY_CYCLES
SQ_VALU_MFMA_COEXEC_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU
GRBM_GUI_ACTIVE`, `--output-format csv`) into matrix-core utilisation per
kernel.  Every counter is a whole-GPU sum per dispatch; GRBM_GUI_ACTIVE
counts the dispatch's busy cycles once per XCD, so a dispatch lasts
GRBM_GUI_ACTIVE / 8 cycles, and the matrix cores' capacity is 4 SIMDs x
256 CUs of those cycles.  The MFMA probe kernel (a chain of back-to-back
16x16x32 bf16 products on every SIMD) is listed beside them as the
calibration: it should read close to 1.

`traffic` turns two counter runs (`--pmc FETCH_SIZE`, then `--pmc
WRITE_SIZE`, both `--output-format csv`) into HBM bytes per launch of one
kernel.  Each counter is scaled by what it reads for a device-to-device copy
of known size (`bench.py --copy-probe` under the same two counters), so the
figure is in real bytes.  The summary records the SHA-256 of the attention
kernel's source; the benchmark reports the traffic only while that source is
unchanged.

Only CSV files are read; nothing here touches the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCE = os.path.join(PKG, "csrc", "sparse_attn.hip")
# the attention kernel's traffic depends on its source and on the host code
# that cuts rows into segments (the segment length sets the item order's L2 reuse)
TRAFFIC_SOURCES = (ATTN_SOURCE, os.path.join(PKG, "csrc", "host.cpp"))


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _short(name: str) -> str:
    if name.startswith("_Z"):  # a name the profiler left mangled: keep the kernel's own identifier
        i = 2
        while i < len(name):  # walk the length-prefixed source names
            m = re.match(r"\d+", name[i:])
            if not m:
                i += 1
                continue
            n, j = int(m.group(0)), i + len(m.group(0))
            ident = name[j:j + n]
            if ident.endswith("_kernel"):
                return f"hsa::{ident} (mangled)"
            i = j + n
        return name
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    name = re.sub(r"\(.*\)$", "", name)  # drop the parameter list
    return name.replace("void ", "", 1)


def kernel_stats(stats_dir: str):
    """[(name, calls, avg_us, min_us, max_us, percent)] from *_kernel_stats.csv."""
    path = _one(os.path.join(stats_dir, "**", "*kernel_stats.csv"))
    rows = []
    for r in csv.DictReader(open(path)):
        rows.append((_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                     float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda t: -t[5])
    return rows


def counter_per_dispatch(pmc_dir: str, counter: str, kernel_regex: str) -> float:
    """Average value of one counter over the dispatches of the matching kernel."""
    path = _one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    vals = defaultdict(float)  # per dispatch (a counter can be split over rows)
    rx = re.compile(kernel_regex)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and rx.search(r["Kernel_Name"]):
            vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not vals:
        raise ValueError(f"no {counter} rows for /{kernel_regex}/ in {path}")
    return sum(vals.values()) / len(vals)


def source_digest() -> str:
    """SHA-256 over the sources that fix the attention kernel's traffic, in order."""
    h = hashlib.sha256()
    for path in TRAFFIC_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def trace_durations(stats_dir: str, kernel_regex: str):
    """Durations (us) of the matching kernel's dispatches, in dispatch order."""
    path = _one(os.path.join(stats_dir, "**", "*kernel_trace.csv"))
    rx = re.compile(kernel_regex)
    rows = [r for r in csv.DictReader(open(path)) if rx.search(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]


def bench_line(log: str) -> dict:
    """The benchmark's JSON line from its log."""
    import json
    for line in reversed(open(log).read().splitlines()):
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    raise ValueError(f"no benchmark line in {log}")


def write_stats(stats_dir: str, out: str, cmd: str, bench_log: str = None) -> None:
    rows = kernel_stats(stats_dir)
    with open(out, "w") as f:
        f.write(f"# rocprofv3 kernel statistics\n# command: {cmd}\n")
        f.write(f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'share%':>7}\n")
        for name, calls, avg, mn, mx, pct in rows:
            f.write(f"{name[:72]:<72} {calls:>6} {avg:>10.1f} {mn:>10.1f} {mx:>10.1f} {pct:>7.2f}\n")
        if bench_log:
            # The benchmark times the attention kernel with HIP events in its
            # per-stage pass of `steps` steps, which is followed by the timed
            # pass of `steps` steps: compare with the same dispatches here.
            b = bench_line(bench_log)
            k = b["roofline"].get("kernel", "sparse_attn_kernel")
            n = int(b["steps"])
            d = trace_durations(stats_dir, k)[-2 * n:-n]
            prof_us = sum(d) / len(d)
            ev_us = 1e3 * float(b["roofline"]["kernel_ms"])
            f.write(f"# {k}: HIP-event average in the benchmark's own line {ev_us:.1f} us; "
                    f"rocprofv3 average of the same {len(d)} dispatches {prof_us:.1f} us "
                    f"(difference {100 * (ev_us - prof_us) / prof_us:+.1f}%)\n")
            f.write(f"# benchmark line under the profiler: value {b['value']} {b['unit']}, "
                    f"roofline achieved {b['roofline']['achieved']} {b['roofline']['unit']}\n")
            # The table above averages every dispatch, including the timed pass,
            # where the linear branch runs beside the sparse branch and waits for
            # CUs.  Each kernel runs once per step, so the per-stage pass (calls
            # in order on one stream) is the same window of dispatches for all.
            f.write(f"# per-kernel averages over the per-stage pass only ({n} steps, calls in order on one stream):\n")
            names = sorted({r["Kernel_Name"] for r in csv.DictReader(open(_one(os.path.join(stats_dir, "**", "*kernel_trace.csv"))))})
            rows = []
            for full in names:
                d = trace_durations(stats_dir, re.escape(full))
                if len(d) >= 2 * n:
                    w = d[-2 * n:-n]
                    rows.append((_short(full), sum(w) / len(w)))
            rows.sort(key=lambda t: -t[1])
            total = sum(us for _, us in rows)
            for name, us in rows:
                f.write(f"#   {name[:70]:<70} {us:>9.1f} us\n")
            f.write(f"#   {'sum of kernel times in one step':<70} {total:>9.1f} us\n")


def write_traffic(a) -> None:
    fetch_kib = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write_kib = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    copy_rx = r"copyBuffer"
    cf = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", copy_rx)
    cw = counter_per_dispatch(a.copy_write, "WRITE_SIZE", copy_rx)
    f_fetch = a.copy_bytes / (cf * 1024.0)
    f_write = a.copy_bytes / (cw * 1024.0)
    traffic = fetch_kib * 1024.0 * f_fetch + write_kib * 1024.0 * f_write
    with open(a.out, "w") as f:
        f.write(f"# HBM traffic per launch of /{a.kernel}/, workload {a.workload}\n")
        f.write(f"# command: {a.cmd}\n")
        f.write(f"workload: {a.workload}\n")
        f.write(f"fetch_kib_per_dispatch: {fetch_kib:.1f}\n")
        f.write(f"write_kib_per_dispatch: {write_kib:.1f}\n")
        f.write(f"copy_bytes: {a.copy_bytes}\n")
        f.write(f"copy_fetch_kib: {cf:.1f}\n")
        f.write(f"copy_write_kib: {cw:.1f}\n")
        f.write(f"fetch_scale: {f_fetch:.4f}\n")
        f.write(f"write_scale: {f_write:.4f}\n")
        f.write(f"traffic_bytes_per_launch: {traffic:.0f}\n")
        f.write(f"source_sha256: {source_digest()}\n")


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_MFMA",
                 "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE")
N_XCD, N_CU, SIMD_PER_CU = 8, 256, 4


def source_digests() -> dict:
    out = {}
    for path in sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))):
        with open(path, "rb") as f:
            out[os.path.basename(path)] = hashlib.sha256(f.read()).hexdigest()[:16]
    return out


def write_mfma(a) -> None:
    with open(a.out, "w") as f:
        f.write(f"# matrix-core utilisation per dispatch, workload {a.workload}\n")
        f.write(f"# command: {a.cmd}\n")
        f.write("# cycles = GRBM_GUI_ACTIVE / 8 (counted once per XCD); mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                "(4 SIMDs x 256 CUs x cycles);\n# coexec = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES "
                "(share of matrix-core busy cycles with a VALU op issued beside it);\n"
                "# busy_cu = SQ_BUSY_CU_CYCLES / (256 x cycles); valu_per_mfma = SQ_INSTS_VALU / SQ_INSTS_MFMA\n")
        hdr = (f"{'kernel':<40} {'cycles':>10} {'mfma_insts':>12} {'busy/inst':>9} {'mfma_busy':>9} "
               f"{'coexec':>7} {'busy_cu':>7} {'valu/mfma':>9}\n")
        f.write(hdr)
        for rx in a.kernels:
            v = {c: counter_per_dispatch(a.pmc_dir, c, rx) for c in MFMA_COUNTERS}
            cyc = v["GRBM_GUI_ACTIVE"] / N_XCD
            busy = v["SQ_VALU_MFMA_BUSY_CYCLES"]
            insts = v["SQ_INSTS_MFMA"]
            f.write(f"{rx[:40]:<40} {cyc:>10.0f} {insts:>12.0f} {busy / max(insts, 1):>9.1f} "
                    f"{busy / (SIMD_PER_CU * N_CU * cyc):>9.3f} {v['SQ_VALU_MFMA_COEXEC_CYCLES'] / max(busy, 1):>7.3f} "
                    f"{v['SQ_BUSY_CU_CYCLES'] / (N_CU * cyc):>7.3f} {v['SQ_INSTS_VALU'] / max(insts, 1):>9.2f}\n")
        f.write("# raw per-dispatch averages:\n")
        for rx in a.kernels:
            vals = " ".join(f"{c}={counter_per_dispatch(a.pmc_dir, c, rx):.4g}" for c in MFMA_COUNTERS)
            f.write(f"#   {rx}: {vals}\n")
        f.write("# source sha256 (first 16 hex digits): " +
                " ".join(f"{k}={h}" for k, h in source_digests().items()) + "\n")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_dir")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    s.add_argument("--bench-log", default=None, help="log of the profiled benchmark run (its JSON line)")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("pmc_dir")
    m.add_argument("out")
    m.add_argument("--kernels", nargs="+", required=True, help="one kernel-name regex per table row")
    m.add_argument("--workload", required=True)
    m.add_argument("--cmd", required=True)
    a = ap.parse_args(argv)
    if a.what == "stats":
        write_stats(a.stats_dir, a.out, a.cmd, a.bench_log)
    elif a.what == "mfma":
        write_mfma(a)
    else:
        write_traffic(a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
