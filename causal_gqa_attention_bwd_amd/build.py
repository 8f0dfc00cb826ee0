"""Build the HIP library in-tree: libattnbwd.so next to this file (gfx950 only)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f)
        for f in ("attnbwd.hip", "attnbwd_f16.hip", "attnbwd_decode.hip", "attnbwd_short.hip")]
LIB = os.path.join(HERE, "libattnbwd.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra: list | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, *(extra or []), "-I", INCLUDE, "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    # the host compilation pass does not know the GPU feature; that line is expected
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if err.strip():
        print(err, file=sys.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
