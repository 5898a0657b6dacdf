"""Summaries of rocprofv3 CSV output for the kernels of libcsa2.so.

    python -m sparse_attention_decode_e2m1_amd.profiling stats TRACE_CSV
        per-kernel dispatch count and duration (mean / median / min / max)
        from a ``--kernel-trace --output-format csv`` run;

    python -m sparse_attention_decode_e2m1_amd.profiling traffic \
        --kernel index_score_kernel --fetch F.csv --write W.csv \
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N
        HBM bytes per dispatch of a kernel from two ``--pmc FETCH_SIZE`` /
        ``--pmc WRITE_SIZE`` runs, each scaled by the factor that makes the
        same counter read N bytes for a plain copy of N bytes;

    python -m sparse_attention_decode_e2m1_amd.profiling mfma \
        --kernel index_score_tokens_kernel --counters C.csv
        MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x
        SIMDs) and f16 MFMA flops per dispatch from one --pmc run.

The traffic summary also records a digest of the sources the kernel is built
from, so a reader can tell whether the counters still describe the kernel.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
# sources that define the indexer-scoring kernel's machine code
KERNEL_SOURCES = {
    "index_score_kernel": ["csrc/index_score.hip", "csrc/csa2_device.hpp",
                           "csrc/csa2_quant.hpp", "csrc/csa2_internal.hpp", "build.py"],
}


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = name.split("(")[0]
    for pre in ("void ", "csa2::"):
        name = name.replace(pre, "")
    return name.strip()


def kernel_stats(trace_csv: str) -> dict:
    """{kernel: [durations in us]} from a kernel-trace CSV."""
    d = defaultdict(list)
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            d[_short(r["Kernel_Name"])].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    return d


def counter_means(counter_csv: str, kernel: str) -> dict:
    """{counter: mean value per dispatch} over the dispatches of `kernel`
    (every kernel whose name contains it)."""
    vals = defaultdict(lambda: defaultdict(float))
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            if kernel not in r["Kernel_Name"]:
                continue
            vals[r["Counter_Name"]][r.get("Dispatch_Id") or r.get("Correlation_Id")] += \
                float(r["Counter_Value"])
    return {c: statistics.fmean(v.values()) for c, v in vals.items() if v}


COPY_KERNEL = "MulFunctor"  # bench.py --copy-kernel-bytes: one multiply-by-one pass


def cmd_stats(a):
    d = kernel_stats(a.trace)
    print(f"{'kernel':44s} {'calls':>6s} {'mean_us':>9s} {'median_us':>9s} {'min_us':>8s} {'max_us':>8s}")
    for k, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        print(f"{k[:44]:44s} {len(v):6d} {statistics.fmean(v):9.2f} {statistics.median(v):9.2f} "
              f"{min(v):8.2f} {max(v):8.2f}")


def cmd_traffic(a):
    cf = counter_means(a.copy_fetch, COPY_KERNEL)["FETCH_SIZE"]
    cw = counter_means(a.copy_write, COPY_KERNEL)["WRITE_SIZE"]
    f_fetch = a.copy_bytes / (cf * 1024.0)
    f_write = a.copy_bytes / (cw * 1024.0)
    kf = counter_means(a.fetch, a.kernel)["FETCH_SIZE"]
    kw = counter_means(a.write, a.kernel)["WRITE_SIZE"]
    fetch_b = kf * 1024.0 * f_fetch
    write_b = kw * 1024.0 * f_write
    print(f"kernel: {a.kernel}")
    print(f"source_digest: {source_digest(a.kernel)}")
    print(f"copy_bytes: {a.copy_bytes}")
    print(f"copy_fetch_kib: {cf:.1f}")
    print(f"copy_write_kib: {cw:.1f}")
    print(f"fetch_factor: {f_fetch:.4f}")
    print(f"write_factor: {f_write:.4f}")
    print(f"fetch_kib_per_dispatch: {kf:.1f}")
    print(f"write_kib_per_dispatch: {kw:.1f}")
    print(f"fetch_bytes_per_dispatch: {fetch_b:.0f}")
    print(f"write_bytes_per_dispatch: {write_b:.0f}")
    print(f"traffic_bytes_per_dispatch: {fetch_b + write_b:.0f}")


def cmd_mfma(a):
    """MFMA utilisation of a kernel from one --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F16 and GRBM_GUI_ACTIVE."""
    c = counter_means(a.counters, a.kernel)
    busy, mops, active = (c["SQ_VALU_MFMA_BUSY_CYCLES"], c["SQ_INSTS_VALU_MFMA_MOPS_F16"],
                          c["GRBM_GUI_ACTIVE"])
    util = busy / (active * a.simds)
    flops = mops * 512
    print(f"kernel: {a.kernel}")
    print(f"dispatches_averaged: yes")
    print(f"SQ_VALU_MFMA_BUSY_CYCLES_per_dispatch: {busy:.0f}")
    print(f"SQ_INSTS_VALU_MFMA_MOPS_F16_per_dispatch: {mops:.0f}")
    print(f"GRBM_GUI_ACTIVE_per_dispatch: {active:.0f}")
    print(f"simds: {a.simds}")
    print(f"mfma_busy_fraction: {util:.4f}")
    print(f"mfma_f16_flop_per_dispatch: {flops:.4g}")
    if "SQ_INSTS_VALU" in c:
        # 16x16x32 f16 MFMAs: 16384 flops each; SQ_INSTS_VALU counts them too
        n_mfma = flops / 16384
        print(f"SQ_INSTS_VALU_per_dispatch: {c['SQ_INSTS_VALU']:.0f}")
        print(f"other_valu_per_mfma: {(c['SQ_INSTS_VALU'] - n_mfma) / max(n_mfma, 1):.2f}")


def read_traffic(path: str, kernel: str):
    """HBM bytes per dispatch recorded in a traffic summary, or None when the
    file is absent or the kernel's sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", " ", "|")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel") != kernel or kv.get("source_digest") != source_digest(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", default="index_score_kernel")
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--kernel", required=True)
    m.add_argument("--counters", required=True)
    m.add_argument("--simds", type=int, default=1024)  # 256 CUs x 4 SIMDs
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
