"""Measurement support: turn rocprofv3 counter CSVs into the per-kernel-class
HBM traffic table that bench.py reads, and fingerprint the kernel sources so
a stale table is not used after the kernels change.

Usage (host side, after the counter runs):
  python -m matrix_aware_optimizer_muon_amd.profiling traffic \
      --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv \
      --copy-bytes N --workload NAME --command "..." > profiles/hbm_traffic_NAME.md
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
# The kernels and the planner (which decides the launches, tiles and forms
# whose traffic a profile records).
KERNEL_SOURCES = ("csrc/gemm.hip", "csrc/gemm_dma.hip", "csrc/rr_fused.hip", "csrc/direct_fused.hip",
                  "csrc/gemm_epilogue.hpp",
                  "csrc/elementwise.hip", "csrc/common.hpp", "csrc/kernels.h",
                  "csrc/muon_api.cpp")
EPI_CLASS = {0: "syrk", 1: "poly", 2: "pqpg", 3: "ph", 4: "final", 5: "xupd", 6: "xupd"}


def code_only(text: str) -> str:
    """The source without comments and with whitespace runs collapsed, so
    that editing a comment does not mark a profile as taken on other code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(read=None) -> str:
    """Fingerprint of the kernel and planner code (comments excluded).
    read(rel) -> text overrides reading the package's files."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(PKG, rel), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(code_only(text).encode())
    return h.hexdigest()[:16]


def kernel_class(name: str) -> str | None:
    """Map a demangled kernel name to the launch-profiler class."""
    m = re.search(r"gemm_dma_kernel<(\d+), (\d+)", name) or re.search(
        r"gemm_kernel<(\d+), \d+, (\d+)", name)
    if m:
        return EPI_CLASS[int(m.group(2))]
    for key, cls in (("rr_fused_kernel", "poly"), ("direct_fused_kernel", "xupd"),
                     ("xcast_kernel", "xcast"), ("wupd_kernel", "wupd"),
                     ("prep_tile_kernel", "prep"), ("prep_rows_kernel", "prep"),
                     ("norm_finalize", "norm"),
                     ("rownorm_rows", "rownorm"), ("rownorm_colsum", "colsum"),
                     ("rownorm_colfinal", "colfinal"), ("rownorm_colapply", "colapply")):
        if key in name:
            return cls
    return None


def _read(path: str, counter: str):
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def traffic_table(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes):
    """Per class: (launches, fetch bytes per launch, write bytes per launch),
    with FETCH_SIZE / WRITE_SIZE (KiB) scaled so that a plain copy of
    `copy_bytes` reads and writes exactly `copy_bytes`."""
    def copy_scale(path, counter):
        per = _read(path, counter)
        vals = [v for k, vs in per.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs]
        if not vals:
            raise SystemExit(f"no copy kernel in {path}")
        return copy_bytes / (max(vals) * 1024.0)
    sf = copy_scale(copy_fetch_csv, "FETCH_SIZE")
    sw = copy_scale(copy_write_csv, "WRITE_SIZE")
    out = {}
    for counter, path, scale, idx in (("FETCH_SIZE", fetch_csv, sf, 1), ("WRITE_SIZE", write_csv, sw, 2)):
        for k, vs in _read(path, counter).items():
            cls = kernel_class(k)
            if cls is None:
                continue
            e = out.setdefault(cls, [0, 0.0, 0.0])
            if idx == 1:
                e[0] += len(vs)
            e[idx] += sum(vs) * 1024.0 * scale
    return {c: (n, f / n, w / n) for c, (n, f, w) in out.items() if n}, sf, sw


def read_traffic(workload: str, root: str):
    """(fetch_bytes_per_launch, write_bytes_per_launch) per class from the
    committed table, or {} if absent or taken from other kernel sources."""
    path = os.path.join(root, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    m = re.search(r"kernel source hash: `([0-9a-f]+)`", text)
    if not m or m.group(1) != source_hash():
        return {}
    out = {}
    for line in text.splitlines():
        mm = re.match(r"\|\s*(\w+)\s*\|\s*(\d+)\s*\|\s*([\d.e+-]+)\s*\|\s*([\d.e+-]+)\s*\|", line)
        if mm:
            out[mm.group(1)] = (float(mm.group(3)) * 1e9, float(mm.group(4)) * 1e9)
    return out


def mfma_table(path, workload, command, xcds):
    """Per kernel class: MfmaUtil (rocprofv3's derived metric: MFMA-busy
    cycles over GPU-busy cycles x SIMDs, duration-weighted), executed MFMA
    flops per second (SQ_INSTS_VALU_MFMA_MOPS_{F16,BF16} x 512) and the clock
    implied by GRBM_GUI_ACTIVE over the dispatch duration (the counter is
    summed over the XCDs)."""
    per = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        d = per[int(r["Dispatch_Id"])]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["_name"] = r["Kernel_Name"]
        d["_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    agg = collections.OrderedDict()
    for d in per.values():
        cls = kernel_class(d["_name"])
        if cls is None or d["_s"] <= 0:
            continue
        a = agg.setdefault(cls, [0, 0.0, 0.0, 0.0, 0.0])
        a[0] += 1
        a[1] += d["_s"]
        a[2] += d.get("MfmaUtil", 0.0) * d["_s"]
        a[3] += (d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)) * 512
        a[4] += d.get("GRBM_GUI_ACTIVE", 0.0)
    print(f"# MFMA utilisation per launch class: {workload}\n")
    print("Counter run (MI355X, repository root), one refresh step:\n")
    print(f"```\n{command}\n```\n")
    print(f"kernel source hash: `{source_hash()}`\n")
    print("MfmaUtil is relative to the running clock; the clock column is only "
          "meaningful for launches much longer than the counter window's overhead "
          "(not for the ~20 us norm launches).\n")
    print("| class | launches | avg ms | MfmaUtil % | executed MFMA TFLOP/s | clock GHz |")
    print("|---|---:|---:|---:|---:|---:|")
    for cls, (n, sec, u, fl, g) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"| {cls} | {n} | {sec * 1e3 / n:.3f} | {u / sec:.1f} | {fl / sec / 1e12:.1f} | "
              f"{g / xcds / sec / 1e9:.2f} |")


def lds_table(path, workload, command):
    """Per kernel class: LdsUtil and LDSBankConflict (rocprofv3's derived
    metrics: cycles the LDS serves indexed accesses, and cycles it stalls on
    bank conflicts, over GPU-busy cycles x compute units; duration-weighted)
    and the LDS bytes read and written by ds instructions per second
    (SQ_INSTS_LDS_{LOAD,STORE}_BANDWIDTH x 64).  Direct-to-LDS global loads
    are not ds instructions and count in neither."""
    per = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        d = per[int(r["Dispatch_Id"])]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["_name"] = r["Kernel_Name"]
        d["_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    agg = collections.OrderedDict()
    for d in per.values():
        cls = kernel_class(d["_name"])
        if cls is None or d["_s"] <= 0:
            continue
        a = agg.setdefault(cls, [0, 0.0, 0.0, 0.0, 0.0, 0.0])
        a[0] += 1
        a[1] += d["_s"]
        a[2] += d.get("LdsUtil", 0.0) * d["_s"]
        a[3] += d.get("LDSBankConflict", 0.0) * d["_s"]
        a[4] += d.get("SQ_INSTS_LDS_LOAD_BANDWIDTH", 0.0) * 64
        a[5] += d.get("SQ_INSTS_LDS_STORE_BANDWIDTH", 0.0) * 64
    print(f"# LDS use per launch class: {workload}\n")
    print("Counter run (MI355X, repository root), one refresh step:\n")
    print(f"```\n{command}\n```\n")
    print(f"kernel source hash: `{source_hash()}`\n")
    print("LdsUtil and LDSBankConflict are percentages of GPU-busy cycles x compute units; "
          "the byte rates count ds_read / ds_write traffic only (the 256-tile kernels fill "
          "their operand ring with direct-to-LDS global loads, which add 32 KB per stage).\n")
    print("| class | launches | avg ms | LdsUtil % | LDSBankConflict % | ds read TB/s | ds write TB/s |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for cls, (n, sec, u, bc, rd, wr) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"| {cls} | {n} | {sec * 1e3 / n:.3f} | {u / sec:.1f} | {bc / sec:.2f} | "
              f"{rd / sec / 1e12:.2f} | {wr / sec / 1e12:.2f} |")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload", "--command"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    sub.add_parser("hash")
    mf = sub.add_parser("mfma")
    mf.add_argument("--csv", required=True)
    mf.add_argument("--workload", required=True)
    mf.add_argument("--command", required=True)
    mf.add_argument("--xcds", type=int, default=8)
    ld = sub.add_parser("lds")
    ld.add_argument("--csv", required=True)
    ld.add_argument("--workload", required=True)
    ld.add_argument("--command", required=True)
    k = sub.add_parser("trace")
    k.add_argument("--stats", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "hash":
        print(source_hash())
        return
    if a.cmd == "mfma":
        mfma_table(a.csv, a.workload, a.command, a.xcds)
        return
    if a.cmd == "lds":
        lds_table(a.csv, a.workload, a.command)
        return
    if a.cmd == "trace":
        rows = list(csv.DictReader(open(a.stats)))
        print(f"# Kernel trace: {a.title}\n")
        print("Command (MI355X, repository root):\n")
        print(f"```\n{a.command}\n```\n")
        print(f"kernel source hash: `{source_hash()}`\n")
        print("| kernel | class | calls | total ms | avg ms | % |")
        print("|---|---|---:|---:|---:|---:|")
        for r in rows:
            name = re.sub(r"\(.*", "", r["Name"]).replace("void ", "")
            if len(name) > 70:
                name = name[:67] + "..."
            cls = kernel_class(r["Name"]) or "-"
            print(f"| `{name}` | {cls} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                  f"{float(r['AverageNs']) / 1e6:.4f} | {float(r['Percentage']):.2f} |")
        per = collections.OrderedDict()
        for r in rows:
            cls = kernel_class(r["Name"])
            if cls is None:
                continue
            e = per.setdefault(cls, [0, 0.0])
            e[0] += int(r["Calls"])
            e[1] += float(r["TotalDurationNs"])
        print("\nPer launch-profiler class (every launch of the class, all shapes; the "
              "figure bench.py's roofline ms_per_launch is compared with):\n")
        print("| class | launches | total ms | avg ms per launch |")
        print("|---|---:|---:|---:|")
        for cls, (n, ns) in sorted(per.items(), key=lambda kv: -kv[1][1]):
            print(f"| {cls} | {n} | {ns / 1e6:.3f} | {ns / n / 1e6:.4f} |")
        return
    table, sf, sw = traffic_table(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes)
    print(f"# HBM traffic per launch: {a.workload}\n")
    print("Counter runs (MI355X, repository root), one refresh step each:\n")
    print(f"```\n{a.command}\n```\n")
    print(f"Scale factors from a plain device copy of {a.copy_bytes} bytes: "
          f"FETCH_SIZE x {sf:.3f}, WRITE_SIZE x {sw:.3f}.\n")
    print(f"kernel source hash: `{source_hash()}`\n")
    print("| class | launches | fetch GB/launch | write GB/launch |")
    print("|---|---:|---:|---:|")
    for c, (n, f, w) in sorted(table.items()):
        print(f"| {c} | {n} | {f / 1e9:.4f} | {w / 1e9:.4f} |")


if __name__ == "__main__":
    main()
