"""Builds libtwell.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: python -m activation_sparse_ffn_gate_amd._build [--jobs N]
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libtwell.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["gate_pack.hip", "gate_pack_skinny.hip", "fused_updown.hip", "sliced_updown.hip", "dense_ffn.hip", "dense_ring.hip",
           "compact_rows.hip", "backward.hip",
           "twell_api.hip"]

# Packed fp32 VALU ops are turned off for every device compile.
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libtwell)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(
        line for line in p.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in line
    )
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libtwell.so next to this file; returns its path."""
    cc = hipcc()
    jobs = jobs or min(8, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="twell_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]

        def compile_one(i):
            return _run([cc, *DEVICE_FLAGS, "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]])

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            logs = list(ex.map(compile_one, range(len(SOURCES))))
        if verbose:
            for s, log in zip(SOURCES, logs):
                if log.strip():
                    print(f"[{s}]\n{log}")
        tmp_lib = os.path.join(tmp, LIB_NAME)
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs])
        # copy then rename, so a loaded library is never overwritten in place
        shutil.copyfile(tmp_lib, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(args.jobs, args.verbose)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
