"""Build libw4a16.so in-tree with hipcc for gfx950.

    python -m int4_group_quantized_q4_amd.build

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel)
and the objects are linked into int4_group_quantized_q4_amd/libw4a16.so; the
bench's ceiling kernels (probe/ceilings.hip) go to libw4probe.so.  Both are
always rebuilt when this runs.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libw4a16.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++20",
    "-fPIC",
    # no packed fp32 math (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep fp32 subnormals (the repack compares quotients of subnormal weights)
    "-fno-gpu-flush-denormals-to-zero",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


PROBE = os.path.join(HERE, "probe")
PROBE_LIB = os.path.join(HERE, "libw4probe.so")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build_probe(verbose=True):
    """libw4probe.so: the bench's machine-ceiling kernels (not part of the ABI)."""
    src = os.path.join(PROBE, "ceilings.hip")
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    # accumulators in VGPRs: in the accumulator-register form the compiler
    # rotates the eight chains through copies on every iteration
    cmd = [HIPCC] + COMMON_FLAGS + ["-mllvm", "-amdgpu-mfma-vgpr-form", "-shared", src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("[build] wrote %s" % PROBE_LIB)
    return PROBE_LIB


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + COMMON_FLAGS + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    # hipcc's host pass does not know the gfx-only feature name: drop that noise
    warn = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose=True):
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found at %s" % HIPCC)
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    for (o, w) in results:
        if w and verbose:
            print("[build] %s:\n%s" % (os.path.basename(o), w), file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("[build] wrote %s" % LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    build()
