"""Compile the gfx950 library liblioncub.so in-tree with hipcc.

Every floating-point operation stays as written: no FMA contraction, no
packed-fp32 instructions, subnormals kept, correctly rounded fp32 division.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblioncub.so")
SOURCES = ["lioncub.cpp", "tables.hip", "static.hip", "step.hip", "l1.hip", "bits.hip",
           "wire.hip"]
# The measurement library (include/lioncub_probe.h): reference streams and the
# step-pattern probe, kept out of liblioncub.so.
PROBE_LIB = os.path.join(HERE, "liblioncub_probe.so")
PROBE_SOURCES = ["probe/probe.cpp", "probe/stream.hip", "probe/pattern.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
OBJ = os.path.join(ROOT, "_build")


def build(verbose=False, jobs=None):
    """Compile every source of both libraries to objects in parallel (the
    step kernels' template instantiations dominate), then link
    liblioncub.so and the measurement library liblioncub_probe.so."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(os.path.join(OBJ, "probe"), exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(OBJ, src + ".o")
        cmd = [HIPCC, *FLAGS, *inc, "-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    def link(lib, objs):
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)

    srcs = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(srcs), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    link(LIB, objs[: len(SOURCES)])
    link(PROBE_LIB, objs[len(SOURCES):])
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
