"""Build libdualkv.so in-tree with hipcc for gfx950.

    python -m sparse_kv_retrieval_amd.build [--jobs N] [--verbose]

Every .hip file under csrc/ is compiled to an object (in parallel) and linked
into sparse_kv_retrieval_amd/libdualkv.so.  Always rebuilds.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdualkv.so")
ARCH = "gfx950"

# Packed fp32 ALU ops stay off: the compiler may otherwise fuse fp32 pairs into
# v_pk_* instructions.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdualkv)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host pass does not know the packed-fp32 feature; that note is harmless
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    cc = hipcc()
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 8)
    with tempfile.TemporaryDirectory(prefix="dualkv_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s)[:-4] + ".o") for s in srcs]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            futs = [ex.submit(_run, [cc, *HIP_FLAGS, "-c", s, "-o", o], verbose)
                    for s, o in zip(srcs, objs)]
            for f in futs:
                f.result()
        tmp_lib = LIB + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        os.replace(tmp_lib, LIB)
    return LIB


PROBE_SRC = os.path.join(PKG, "probe", "read_ceiling.hip")
PROBE_LIB = os.path.join(PKG, "libdkprobe.so")


def build_probe(verbose: bool = False) -> str:
    """The read-ceiling probe library bench.py --ceiling loads (not part of libdualkv)."""
    tmp_lib = PROBE_LIB + ".tmp"
    _run([hipcc(), *HIP_FLAGS, "-shared", PROBE_SRC, "-o", tmp_lib], verbose)
    os.replace(tmp_lib, PROBE_LIB)
    return PROBE_LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    print(build_probe(a.verbose))


if __name__ == "__main__":
    sys.exit(main())
