"""Build libmaxsim.so in place with hipcc for gfx950 (no GPU needed to compile)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmaxsim.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # NaN inputs are outside the contract (include/maxsim.h): maxima need no NaN
    # canonicalisation. Infinities are kept (-inf is the identity of a max).
    "-fno-honor-nans",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results stay in ordinary VGPRs: without it the accumulators live in
    # AGPRs and are copied to VGPRs for every max reduction
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-pass-failed",
    "-I", os.path.join(ROOT, "include"),
]


OBJ_DIR = os.path.join(PKG, "_build")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile libmaxsim.so (always recompiles): one object per .hip file, in parallel."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC, *compile_flags, "-c", "-o", so[1], so[0]], verbose),
                    zip(srcs, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
