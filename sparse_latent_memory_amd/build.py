"""Build libmsa.so (HIP, gfx950) in-tree with hipcc, and beside it
libmsa_readref.so, the reference streaming-read kernel that bench.py times
against the bank scan (measurement only, not part of libmsa).

    python -m sparse_latent_memory_amd.build [-v]

Every call recompiles; objects go to _build/ next to the package and the
libraries to sparse_latent_memory_amd/.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["msa_api.hip", "pool.hip", "route.hip", "route_scan.hip", "route_scan_wide.hip", "route_select.hip",
           "decode.hip", "attend.hip"]
LIB = os.path.join(HERE, "libmsa.so")
READREF_SOURCE = "read_ref.hip"
READREF_LIB = os.path.join(HERE, "libmsa_readref.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmsa)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return out


def build(verbose=False, jobs=4):
    """Compile every HIP source for gfx950 and link libmsa.so and
    libmsa_readref.so."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *CFLAGS, "-c", os.path.join(HERE, "csrc", src), "-o", obj])
    ref_obj = os.path.join(BUILD_DIR, READREF_SOURCE.replace(".hip", ".o"))
    cmds.append([hipcc, *CFLAGS, "-c", os.path.join(HERE, "csrc", READREF_SOURCE), "-o", ref_obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for lib, lib_objs in ((LIB, objs), (READREF_LIB, [ref_obj])):
        tmp = lib + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *lib_objs, "-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
