"""Build libkvc.so (HIP for gfx950) in place, next to this file.

    python -m kv_cache_decode_kvc_amd.build [--report]

Every .hip source and the host API are compiled with hipcc for gfx950 and
linked into one shared library.  --report prints the compiler's per-kernel
register, LDS and spill figures.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvc.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # single-lane atomics stay plain atomics: the wave-reduction rewrite
    # consumes the result right away and so waits for the round trip
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str, report: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if report and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    msgs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    return obj, msgs


def build(report: bool = False, quiet: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, report), srcs))
    objs = [o for o, _ in results]
    if report or not quiet:
        for (o, msgs) in results:
            if msgs.strip():
                print(f"== {os.path.basename(o)}\n{msgs}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(report="--report" in sys.argv, quiet=False)
    print(path)
