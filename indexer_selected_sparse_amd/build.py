"""Build libqsa.so (all HIP kernels + the C ABI) for gfx950, in-tree.

Each .hip source is compiled to an object in parallel (`_build/` under the
package), then the objects are linked into `libqsa.so`.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqsa.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no implicit multiply-add fusion: kernels fuse explicitly where exact
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 instructions are kept out of generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


# Per-source extra flags.  The attention kernels keep their matrix-core
# accumulators in ordinary VGPRs (the compiler would otherwise pick AGPRs,
# and every online-softmax rescale would copy them out and back).
EXTRA_FLAGS = {"qsa_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
               "qsa_attn_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _filter(stderr: str) -> str:
    # the host pass does not know the packed-fp32 target feature: harmless
    return "\n".join(l for l in (stderr or "").splitlines() if "packed-fp32-ops" not in l)


def _compile(hipcc: str, src: str) -> tuple[str, int, str]:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []),
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return obj, r.returncode, _filter(r.stderr)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s), srcs))
    failed = False
    for (obj, rc, errs), src in zip(results, srcs):
        if errs.strip() and (verbose or rc != 0):
            sys.stderr.write(f"{os.path.basename(src)}:\n{errs}\n")
        failed |= rc != 0
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(_filter(r.stderr) + "\n")
        raise RuntimeError(f"hipcc link failed ({r.returncode})")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
