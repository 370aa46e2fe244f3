"""Summarise rocprofv3 output of one bench workload into profiles/.

    python -m kv_cache_decode_kvc_amd.profile_summary --workload C2 \\
        --trace DIR --fetch DIR --write DIR --out profiles/NAME.md

DIR are the -d directories of three rocprofv3 runs of the same bench command
(--kernel-trace --stats; --pmc FETCH_SIZE; --pmc WRITE_SIZE; all with
--output-format csv and -o bench).  The summary lists the library's kernels
(calls, average/min/max duration) and the HBM bytes per dispatch from the two
counters, each scaled by what the counter reads for the bench's known-size
copy (kvc_copy of 1 GiB).  It also records, in profiles/traffic.json, the
dominant kernel's scaled bytes per launch together with a hash of that
kernel's sources (its own file, the shared headers and the host side), which
bench.py uses only while those sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
COPY_BYTES = 1 << 30

# dominant kernel of each bench workload (substring of the demangled name)
DOMINANT = {
    "C1": "dense_generic_kernel<float, 64, false, true>",
    "C2": "dense_mfma_kernel<false, true, false, false, false>",
    "C3": "dense_persist_kernel<true, false, false, false>",
    "C4": "mla_kernel",
    "C5": "dense_mfma_kernel<true, false, false, false, false>",
    "C3F8": "dense_persist_kernel<false, true, false, false>",
    "C3F4": "dense_persist_kernel<false, false, false, true>",
    "C3W128": "dense_mfma_kernel<false, false, false, false, false>",
    "C3P16": "dense_persist_kernel<false, false, true, false>",
    "C5S": "seg_select_kernel",
}


# source file of each workload's dominant kernel
KERNEL_SOURCE = {w: "decode_dense.hip" for w in DOMINANT}
KERNEL_SOURCE.update({"C4": "decode_mla.hip", "C5S": "select.hip"})
# sources every kernel depends on (shared headers and the host side)
COMMON_SOURCES = ["kvc_device.h", "kvc_internal.h", "kvc_api.cpp"]


def source_hash(workload: str) -> str:
    """sha256 over the public header, the shared sources and the workload's
    dominant-kernel source, in that order: a change to another kernel's
    source leaves the recorded counters of this one valid."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    files = [os.path.join(ROOT, "include", "kvc.h")]
    files += [os.path.join(csrc, f) for f in COMMON_SOURCES + [KERNEL_SOURCE[workload]]]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _short(name: str) -> str:
    """Demangled name without "void " and the argument list (the
    parenthesised group that ends the name; "(anonymous namespace)" and
    parentheses inside the arguments are kept out of the way)."""
    name = name.replace("void ", "").strip()
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += name[i] == ")"
            depth -= name[i] == "("
            if depth == 0:
                return name[:i]
    return name


def _counters(path: str):
    out = {}
    for row in csv.DictReader(open(path)):
        name = _short(row["Kernel_Name"])
        if "kvc::" not in name:
            continue
        out.setdefault(name, []).append(float(row["Counter_Value"]) * 1024.0)
    return {k: sum(v) / len(v) for k, v in out.items()}, {k: len(v) for k, v in out.items()}


def _find(d: str, suffix: str) -> str:
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"{suffix} under {d}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True, choices=sorted(DOMINANT))
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--bench-line", default=None, help="file holding the bench JSON line")
    ap.add_argument("--command", action="append", default=[], help="command text to record")
    a = ap.parse_args()

    stats = []
    for row in csv.DictReader(open(_find(a.trace, "kernel_stats.csv"))):
        name = _short(row["Name"])
        if "kvc::" in name:
            stats.append((name, int(row["Calls"]), float(row["AverageNs"]) / 1e3,
                          float(row["MinNs"]) / 1e3, float(row["MaxNs"]) / 1e3))
    fetch, nf = _counters(_find(a.fetch, "counter_collection.csv"))
    write, nw = _counters(_find(a.write, "counter_collection.csv"))
    f_scale = COPY_BYTES / fetch["kvc::copy_kernel"]
    w_scale = COPY_BYTES / write["kvc::copy_kernel"]

    dom = DOMINANT[a.workload]
    dom_name = next(n for n in fetch if dom in n)
    dom_stats = next(s for s in stats if dom in s[0])
    fb = fetch[dom_name] * f_scale
    wb = write[dom_name] * w_scale

    lines = [f"# {dom_name} — workload {a.workload}", ""]
    if a.command:
        lines += ["Commands (run from /tmp on the GPU box, repository at $R):", ""]
        lines += [f"    {c}" for c in a.command]
        lines += [""]
    lines += ["Kernel durations (`--kernel-trace --stats`, kernel_stats.csv):", "",
              "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
    lines += [f"| `{n}` | {c} | {av:.2f} | {mn:.2f} | {mx:.2f} |" for n, c, av, mn, mx in stats]
    lines += ["", f"Counter scale from the 1 GiB `kvc_copy`: FETCH_SIZE x{f_scale:.3f}, "
                  f"WRITE_SIZE x{w_scale:.3f}.", "",
              "HBM bytes per dispatch (scaled counters, average over dispatches):", "",
              "| kernel | dispatches | fetch MB | write MB |", "|---|---|---|---|"]
    for n in sorted(fetch):
        lines.append(f"| `{n}` | {nf[n]} | {fetch[n] * f_scale / 1e6:.3f} | "
                     f"{write.get(n, 0.0) * w_scale / 1e6:.3f} |")
    lines += ["", f"Dominant kernel `{dom_name}`: average {dom_stats[2]:.2f} µs per dispatch; "
                  f"traffic {(fb + wb) / 1e6:.3f} MB per launch "
                  f"(fetch {fb / 1e6:.3f} MB + write {wb / 1e6:.3f} MB)."]
    if a.bench_line:
        txt = open(a.bench_line).read().strip().splitlines()
        js = [l for l in txt if l.startswith("{")]
        if js:
            d = json.loads(js[-1])
            lines += ["", "Bench line of the traced run: "
                      f"roofline.kernel_us = {d['roofline']['kernel_us']} (HIP events over back-to-back "
                      f"launches, includes the graph's inter-kernel gap), achieved "
                      f"{d['roofline']['achieved']} GB/s, value {d['value']} GB/s."]
    lines += ["", f"Kernel sources sha256 (include/kvc.h, {', '.join(COMMON_SOURCES)}, "
                  f"{KERNEL_SOURCE[a.workload]}): `{source_hash(a.workload)}`", ""]
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines))

    tj = os.path.join(os.path.dirname(os.path.abspath(a.out)), "traffic.json")
    data = json.load(open(tj)) if os.path.exists(tj) else {}
    data[a.workload] = {"kernel": dom_name, "fetch_bytes_per_launch": round(fb),
                        "write_bytes_per_launch": round(wb),
                        "avg_us_rocprof": round(dom_stats[2], 3),
                        "source_sha256": source_hash(a.workload)}
    with open(tj, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(f"wrote {a.out}")


if __name__ == "__main__":
    main()
