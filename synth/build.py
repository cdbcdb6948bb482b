"""Build the seeded-input generators: host (gcc + OpenMP) and device (hipcc, gfx950)."""

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, cwd=_HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def _atomic(out, cmd_with_tmp):
    tmp = out + ".tmp"
    _run(cmd_with_tmp(tmp))
    os.replace(tmp, out)


def build_host():
    out = os.path.join(_HERE, "libsbpsynth_host.so")
    _atomic(out, lambda tmp: ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp",
                              "-ffp-contract=off", "-o", tmp, "synth_host.c", "-lm"])
    return out


def build_dev():
    out = os.path.join(_HERE, "libsbpsynth_dev.so")
    _atomic(out, lambda tmp: [HIPCC] + HIP_FLAGS + ["-o", tmp, "synth_dev.hip"])
    return out


def build():
    return build_host(), build_dev()


if __name__ == "__main__":
    print(build())
