"""Build the gfx950 HIP library ``libmla_paged_kv.so`` in place.

Usage: ``python -m mla_paged_kv_get_amd.build`` (or ``build()`` from Python).
Compiles every ``csrc/*.hip`` with hipcc for gfx950 and links one shared
library next to this file.  hipcc cross-compiles, so no GPU is needed.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmla_paged_kv.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
    "-Wall", "-Wno-unused-function",
]
# Per-source flags.  mla_decode.hip (the 16- and 64-row decode variants):
# MFMA accumulators in VGPRs; the register allocator then keeps the 64-row
# variant's output accumulators in place across the tile loop (in AGPRs it
# copied all 128 of them to VGPRs and back on every tile) and parks the query
# fragments, which only MFMAs read, in AGPRs.  mla_decode_rows128.hip keeps the
# default AGPR accumulators: its 256 output accumulators per lane fill the AGPRs.
FILE_FLAGS = {
    "mla_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "not a recognized feature for this target" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int = 4) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for cmd, err in zip(cmds, ex.map(_run, cmds)):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    err = _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
