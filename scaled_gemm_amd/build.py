"""Build libptpc.so (hand-written HIP for gfx950) in-tree.

    python -m scaled_gemm_amd.build        # or __graft_entry__.build()

Every source is compiled by hipcc for gfx950 only, with FMA contraction off
(the quantizer's division sequence and the epilogue's two multiplies are
written out explicitly) and without packed-fp32 instruction selection.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libptpc.so")
# Debug variant: every pipelined GEMM kernel overwrites each LDS region it is
# about to refill with E4M3 NaN bytes first (tests compare it with LIB).
POISON_LIB = os.path.join(PKG, "libptpc_lds_poison.so")
# Debug variant: the main tiled GEMM kernel records per-workgroup timestamps
# (start, K loop entered, K loop done, stores done) into a buffer set with
# ptpc_debug_set_timeline (bench.py --timeline).
TIMELINE_LIB = os.path.join(PKG, "libptpc_timeline.so")
# Debug variant: the two-range K join never raises its flag and waits only a
# few sleeps, so every joined tile takes the path of a wait that runs out.
JOIN_LOST_LIB = os.path.join(PKG, "libptpc_join_lost.so")

SOURCES = ["ptpc_api.cpp", "plan.cpp", "quant.hip", "gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def _variant(name, defines):
    """(objects, compile commands, link command) of one build variant."""
    out_dir = os.path.join(BUILD, name)
    os.makedirs(out_dir, exist_ok=True)
    lib = {"release": LIB, "lds_poison": POISON_LIB, "timeline": TIMELINE_LIB,
           "join_lost": JOIN_LOST_LIB}[name]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *FLAGS, *defines, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-Bsymbolic",
            "-o", lib + ".tmp", *objs]
    return lib, cmds, link


def build(verbose: bool = False) -> str:
    """Build libptpc.so and its three debug variants."""
    variants = [_variant("release", []), _variant("lds_poison", ["-DPTPC_LDS_POISON"]),
                _variant("timeline", ["-DPTPC_TIMELINE"]),
                _variant("join_lost", ["-DPTPC_JOIN_LOST"])]
    cmds = [c for _, cs, _ in variants for c in cs]
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for out in ex.map(lambda c: _run(c, verbose), cmds):
            if verbose and out.strip():
                print(out)
    for lib, _, link in variants:
        _run(link, verbose)
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
