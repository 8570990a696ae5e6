"""Build libkvfp8.so (the gfx950 HIP kernels and the C ABI) in place with hipcc."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvfp8.so")
SOURCES = ["api.cpp", "prefill_plan.cpp", "kv_cache_write.hip", "paged_decode.hip", "paged_decode_d64.hip",
           "paged_decode_d128.hip", "paged_decode_d256.hip", "paged_prefill.hip",
           "stream_read.hip", "decode_noalloc.hip"]
OBJDIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("KVFP8_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # IEEE fp32 division and no fast-math anywhere: the cache write must
    # divide by the scale exactly as the format definition says.
    "-fno-fast-math", "-ffp-contract=fast-honor-pragmas",
    # Packed-FP32 instructions are kept out of generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the decode loop adds them into the
    # FP32 running sum and rescales them with VALU code, which would
    # otherwise copy them out of (and back into) accumulation registers.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel: the decode kernels
    are split by head dimension so that no unit dominates), then link."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, s + ".o") for s in SOURCES]
    jobs = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    workers = max(1, min(len(jobs), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
