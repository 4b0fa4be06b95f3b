"""Build libavey.so (gfx950) in-tree with hipcc.

    python -m attention_free_long_amd.build [--jobs N] [--verbose]

Every HIP source under csrc/ is compiled to an object in _build/ and linked into
attention_free_long_amd/libavey.so. hipcc cross-compiles for gfx950 without a GPU.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libavey.so")

ARCH = "gfx950"
SOURCES = ["abi.hip", "prepare.hip", "maxsim_bf16.hip", "topk.hip", "compress_bf16.hip", "dyn_bf16.hip", "gemm_bf16.hip", "simt_f32.hip", "peak_probe.hip", "noalloc.hip"]

# Packed fp32 instructions are kept out of all device code (the host pass warns that it does not
# know the feature; that warning is harmless).
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Per-source additions. The MaxSim epilogue is a long chain of maxima over finite values: with
# the IEEE mode bit off (which needs relaxed NaN handling) v_max_f32 takes its operands as they
# are, so the compiler neither inserts a canonicalising v_max before each one nor splits the
# DPP-fed maxima into a move plus a max. NaN inputs give unspecified scores.
SOURCE_FLAGS = {
    "maxsim_bf16.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libavey)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # drop the host pass's notice about the device-only target feature
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(jobs: int | None = None, verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    flags = HIP_FLAGS + [f"-I{INCLUDE}", f"-I{CSRC}"] + list(extra_flags)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *flags, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    sys.exit(main())
