"""Build libnvfp4_amd.so (the C-ABI library) for gfx950 with hipcc, in-tree.

The library is compiled from csrc/ only and links nothing else of this repository.
Flags:
  * --offload-arch=gfx950: CDNA4 only.
  * -Xclang -target-feature -Xclang -packed-fp32-ops: keep fp32 arithmetic
    on scalar-per-lane instructions (no v_pk_*_f32).
  * no fast-math: fp32 division stays correctly rounded and denormals are
    kept, which the bit-exact quantizer relies on.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4_amd.so")
SOURCES = ["quantize.hip", "gemm.hip", "linear_small.hip", "mx.hip", "abi.cpp"]


def hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    objs = []
    base = [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(build_dir, s + ".o")
        lang = ["-x", "hip"] if s.endswith(".hip") else []
        cmd = base + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {s}")
        objs.append(obj)
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
