"""Build step for the HIP library: compiles csrc/ into libfp4kv.so for gfx950.

Run ``python -m fp4_quantised_kv_amd.build`` (or ``__graft_entry__.build()``).
The library is placed next to this file and loaded from there.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIBRARY = os.path.join(HERE, "libfp4kv.so")
SOURCES = [os.path.join(HERE, "csrc", "fp4kv_api.cpp"),
           os.path.join(HERE, "csrc", "fp4kv_kernels.hip"),
           os.path.join(HERE, "csrc", "fp4kv_decode_mfma.hip"),
           os.path.join(HERE, "csrc", "fp4kv_decode_fp8.hip"),
           os.path.join(HERE, "csrc", "fp4kv_int_api.cpp"),
           os.path.join(HERE, "csrc", "fp4kv_int.hip"),
           os.path.join(HERE, "csrc", "fp4kv_scratch.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result", "-fvisibility=hidden",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the kernels rescale them on
    # the vector ALUs, and AGPR copies would cost more than they save
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-x", "hip"] + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
