"""Build libbiverify.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m invariant_verify_verifier_amd.build

Compiles every ``csrc/*.hip`` with hipcc for gfx950 and links one shared
library next to this file.  hipcc cross-compiles, so no GPU is needed.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbiverify.so")
OBJ_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit contraction of a*b + c: every fused multiply-add in the
    # kernels is written out (fmaf / __fmaf_rn), so two kernels that state
    # the same arithmetic round it the same way whatever the compiler
    # schedules (several bit-for-bit equalities between kernels rest on it)
    "-ffp-contract=off",
]
# Per-source extras.  The attention kernel runs one wave per SIMD and also
# rescales and folds its MFMA accumulators with vector ALU code: keeping MFMA
# results in ordinary VGPRs avoids copying them to and from AGPRs every step.
EXTRA = {
    "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stdout}\n{p.stderr}")
    # the host pass does not know the gfx feature name; that warning is harmless
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in p.stderr.splitlines() if noise not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
