"""Build the hardware probes under tests/hw (standalone gfx950 programs the
GPU tests run as child processes) next to their sources, as <name>.bin."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> list:
    out = []
    for src in sorted(f for f in os.listdir(HERE) if f.endswith(".hip")):
        exe = os.path.join(HERE, src[:-4] + ".bin")
        cmd = [HIPCC, *FLAGS, os.path.join(HERE, src), "-o", exe + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
        os.replace(exe + ".tmp", exe)
        out.append(exe)
    return out
