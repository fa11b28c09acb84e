"""Build libmoda.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "moda_api.hip")
OUT = os.path.join(HERE, "libmoda.so")

# -packed-fp32-ops off: no packed float32 VALU instructions in device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc_command(out: str = OUT, extra=()):
    return (["hipcc"] + HIPCC_FLAGS + list(extra)
            + ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"), "-o", out, SRC])


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = hipcc_command(tmp)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
