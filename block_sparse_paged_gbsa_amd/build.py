"""Build libgbsa.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m block_sparse_paged_gbsa_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgbsa.so")
SOURCES = ["api.hip", "metadata.hip", "fwd_decode.hip", "fwd_prefill.hip", "validate.hip"]
# measurement probes (HBM ceilings for the benchmark), a library of their own
PROBE_LIB = os.path.join(HERE, "libgbsa_probe.so")
PROBE_SOURCES = ["probe.hip"]
# diagnostic build: libgbsa with the prefill slot trace (include/gbsa_slot_trace.h); only the
# prefill kernels' source is compiled differently
TRACE_LIB = os.path.join(HERE, "libgbsa_slot_trace.so")
TRACE_SOURCE = "fwd_prefill.hip"
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libgbsa)")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
        # packed fp32 VALU ops are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def _compile(src: str, verbose: bool, trace: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_slot_trace" if trace else "") + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + flags()
    if trace:
        cmd.append("-DGBSA_SLOT_TRACE")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(ln for ln in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in ln and ln.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if msg and verbose:
        print(msg, flush=True)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs_list = [(s, False) for s in SOURCES + PROBE_SOURCES] + [(TRACE_SOURCE, True)]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs_list))
    main = objs[:len(SOURCES)]
    _link(main, LIB, verbose)
    _link(objs[len(SOURCES):len(SOURCES) + len(PROBE_SOURCES)], PROBE_LIB, verbose)
    traced = [objs[-1] if src == TRACE_SOURCE else o for src, o in zip(SOURCES, main)]
    _link(traced, TRACE_LIB, verbose)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
