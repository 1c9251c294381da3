"""Build libsra.so in-tree with hipcc for gfx950.

Usage: ``python -m sparse_rank_adapter_amd.build`` (or ``__graft_entry__.build()``).
Every call recompiles every source; objects go to ``_build/`` next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsra.so")

SOURCES = [
    "abi.hip",
    "compress.hip",
    "ffi_format.hip",
    "f32_path.hip",
    "spmm24.hip",
    "spmm_xp.hip",
    "decode24.hip",
    "adapter.hip",
    "spmm_ffi.hip",
    "weight_grad.hip",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are disabled for all device code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return p.returncode, out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in srcs]
    cmds = [[HIPCC, *CFLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for s, (rc, out) in zip(srcs, results):
        if out.strip() and (verbose or rc):
            print(f"--- {s}\n{out}", file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("hipcc failed; see the messages above")
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
