"""Compile example.c (a plain-C consumer of include/lioncub.h, checked
against the CPU oracle) into tests/c_abi/example with gcc.  Needs
liblioncub.so and oracle/liblco.so built first; host code only."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "communication_compressed_distributed_amd")
ORACLE = os.path.join(ROOT, "oracle")
EXE = os.path.join(HERE, "example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose=False):
    # a plain C compiler: the boundary needs nothing but its header and the
    # HIP runtime's C API
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           "-o", EXE + ".tmp", os.path.join(HERE, "example.c"),
           "-L", PKG, "-llioncub", "-L", ORACLE, "-llco", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ORACLE}",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
