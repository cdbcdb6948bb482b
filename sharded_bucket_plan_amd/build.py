"""Build libsbp.so (the C-ABI library) in-tree with hipcc for gfx950."""

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsbp.so")
# measurement kernels for bench.py only (not part of the library's ABI)
PROBE_LIB = os.path.join(PKG, "libsbp_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: every binary32 operation rounds once (no fused
# multiply-add), which the shard step's results are defined by.
# -packed-fp32-ops: no packed fp32 instructions.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _hipcc(srcs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + srcs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(r.stderr)


def build(verbose=False):
    _hipcc(sources(), LIB, verbose)
    _hipcc(sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip"))), PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
