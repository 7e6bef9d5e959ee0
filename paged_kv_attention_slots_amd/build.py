"""Build libmsgl.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every HIP translation unit is compiled with hipcc for gfx950 only, with the
packed-fp32 instructions disabled, then linked into one shared library next to
this file.  The bench's read-ceiling probes (csrc/probes) go into a library of
their own, libmsgl_probes.so.  ``python -m paged_kv_attention_slots_amd.build``
rebuilds both.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
LIB_PATH = os.path.join(HERE, "libmsgl.so")
# read-bandwidth probes for the bench's ceilings (measurement only, not part of libmsgl)
PROBES_PATH = os.path.join(HERE, "libmsgl_probes.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Extra flags per translation unit.  The prefill kernel takes column maxima of
# MFMA results; with NaN-free inputs assumed, the compiler does not quieten
# every score before its max (one VALU instruction per score saved).
FILE_FLAGS = {
    "prefill_mfma.hip": ["-fno-honor-nans"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; only real warnings are shown
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip())
    if msg:
        print(msg, file=sys.stderr)
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(jobs, 16)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    probes = sorted(glob.glob(os.path.join(CSRC, "probes", "*.hip")))
    tmp = PROBES_PATH + f".tmp{os.getpid()}"
    cmd = [HIPCC, *COMMON_FLAGS, "-shared", "-o", tmp, *probes]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBES_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
