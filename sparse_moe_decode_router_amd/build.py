"""Compile the HIP decode-step library (``libmoe_decode.so``) for gfx950.

One translation unit (``csrc/moe_decode.hip``) holds the kernels and the C ABI
declared in ``include/moe_decode.h``.  Packed-f32 instruction selection is
switched off for the device code.
"""
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "moe_decode.hip")
LIB = os.path.join(HERE, "libmoe_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out: str, extra=()) -> list:
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            *extra, SRC, "-o", out]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def source_digest() -> str:
    """Digest of the device sources: ties a stored hardware-counter reading
    to the kernels it was taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
