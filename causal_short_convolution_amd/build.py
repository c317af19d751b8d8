"""Build libshortconv.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

    python -m causal_short_convolution_amd.build [--save-temps DIR]

Flags: gfx950 only; -ffp-contract=off so the kernels' fused multiply-adds are exactly the
explicit ones; packed-fp32 instruction selection disabled; hidden visibility so the library
exports only the extern "C" entry points declared in include/shortconv.h.
"""
import argparse
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libshortconv.so")
SOURCES = [os.path.join(CSRC, f) for f in ("kernels.hip", "backward.hip", "abi.hip")]
# measurement companion used by bench.py (same-bytes copy ceiling); not part of the C ABI
PROBE_LIB = os.path.join(HERE, "libscprobe.so")
PROBE_SOURCES = [os.path.join(CSRC, "copy_probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: every fused multiply-add is written out, so prefill and decode round alike.
# -packed-fp32-ops: no packed fp32 instructions are generated.
# -fno-slp-vectorize: the kernels' arrays are per-lane registers; grouping them into vectors only
#   adds shuffles and, for some widths, doubles register use (bf16 prefill at width 4 spills).
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-slp-vectorize", "-Wall", "-Wno-unused-function",
]


def _hipcc(out, sources, verbose, save_temps=None):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *sources]
    cwd = None
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, "--save-temps")
        cwd = save_temps
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=cwd)
    os.replace(tmp, out)


def build(verbose: bool = False, save_temps: str = None) -> str:
    _hipcc(LIB, SOURCES, verbose, save_temps)
    _hipcc(PROBE_LIB, PROBE_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None, help="keep intermediate files (ISA) in DIR")
    args = ap.parse_args()
    print(build(verbose=True, save_temps=args.save_temps))
