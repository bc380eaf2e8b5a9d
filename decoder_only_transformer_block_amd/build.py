"""Build libdtb.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m decoder_only_transformer_block_amd.build  [--jobs N]
The library is written next to this file; objects go to _build/.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdtb.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU ops stay off (v_pk_* fp32 forms are avoided)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the softmax / epilogue arithmetic on
    # them then needs no AGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(SRC, "*.hip")))
    jobs = jobs or min(8, len(srcs), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    # a kernel whose host-side stub was dropped (a template that did not
    # instantiate for the host pass) links but leaves an undefined symbol of
    # our own namespace, and the library then fails to load: refuse it here
    r = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    own = [l.split()[-1] for l in r.stdout.splitlines() if "_ZN3dtb" in l]
    if own:
        os.remove(tmp)
        raise RuntimeError("libdtb.so would reference undefined symbols of its own: " + ", ".join(own[:8]))
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    print(build(a.jobs))


if __name__ == "__main__":
    main()
