"""Compile libdllm.so for gfx950 with hipcc (in-tree, next to this file), and the
seeded input generator dllm_inputs/libdllm_inputs.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdllm.so")
SOURCES = ["dllm_kernels.hip", "dllm_runtime.hip"]
# Packed fp32 VALU ops are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


# The seeded input generator (dllm_inputs, not part of the library above).
INPUTS_SRC = os.path.join(os.path.dirname(HERE), "dllm_inputs", "csrc", "gen_inputs.hip")
INPUTS_LIB = os.path.join(os.path.dirname(HERE), "dllm_inputs", "libdllm_inputs.so")


def _hipcc(sources, out, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    r = subprocess.run([hipcc] + FLAGS + sources + ["-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _hipcc([os.path.join(CSRC, s) for s in SOURCES], LIB, verbose)
    _hipcc([INPUTS_SRC], INPUTS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
