"""Build the oracle's C library (liboracle.so) next to its source with gcc.

TEST INFRASTRUCTURE: the oracle is only loaded by the tests, the smoke check
and the benchmark's CPU-baseline leg.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No fast-math and no FMA contraction: every operation is the plain IEEE one.
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
          "-shared", "-pthread", "-Wall", "-Wextra", "-Wno-unused-parameter"]


LIB_SANITIZED = os.path.join(HERE, "liboracle_asan.so")
# AddressSanitizer and UndefinedBehaviorSanitizer build of the same source,
# for the CPU test tier (loaded with libasan preloaded; see the sanitizer test).
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]


def build_sanitized(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, *SANITIZE, SRC, "-o", LIB_SANITIZED + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB_SANITIZED + ".tmp", LIB_SANITIZED)
    return LIB_SANITIZED


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
