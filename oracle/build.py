"""Build step for the CPU oracle (test infrastructure, not product code).

Compiles ``fp4kv_oracle.c`` with gcc into ``libfp4kv_oracle.so`` next to it.
Plain ``-O2`` with no fast-math flags, so every step keeps IEEE semantics.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "fp4kv_oracle.c")
LIBRARY = os.path.join(HERE, "libfp4kv_oracle.so")


def build() -> str:
    tmp = LIBRARY + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-o", tmp, SOURCE, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build())
