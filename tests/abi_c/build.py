"""Build tests/abi_c/libfrom_c.so: a plain-C consumer of include/shortconv.h (gcc, C99), linked
against the built libshortconv.so and the HIP runtime, for tests/test_gpu_c_abi.py."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libfrom_c.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "causal_short_convolution_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-o", LIB + ".tmp",
           os.path.join(HERE, "from_c.c"), "-L", pkg, "-lshortconv",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../causal_short_convolution_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
