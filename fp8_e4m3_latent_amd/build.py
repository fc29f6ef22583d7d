"""Build libkv8.so (hand-written HIP for gfx950) in place.

    python -m fp8_e4m3_latent_amd.build [--asm]

--asm also writes the gfx950 assembly of every source to _build/ for reading
register counts and instruction schedules.
"""
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkv8.so")
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-I", INCLUDE, "-I", CSRC,
        # packed-FP32 instructions are disabled for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fno-gpu-flush-denormals-to-zero",
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Wall", "-Wno-unused-command-line-argument",
    ]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(asm=False, verbose=False):
    srcs = sources()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), "-shared", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if asm:
        out = os.path.join(ROOT, "_build")
        os.makedirs(out, exist_ok=True)
        for s in srcs:
            base = os.path.splitext(os.path.basename(s))[0]
            subprocess.run([hipcc(), *flags(), "--cuda-device-only", "-S", s, "-o",
                            os.path.join(out, base + ".s")], check=True)
    return LIB


if __name__ == "__main__":
    print(build(asm="--asm" in sys.argv, verbose=True))
