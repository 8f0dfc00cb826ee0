"""Build the HIP library in-tree: libattnbwd.so next to this file (gfx950 only).

Each source compiles to its own object in parallel (_build/ next to this
file, keeping the compiler's gfx950 assembly), then one link makes the
shared library.  Before the link the assembly goes through
codegen_check.scan: a library in which the register allocator placed a copy
inside a divergent branch's join block is refused."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f)
        for f in ("attnbwd.hip", "attnbwd_f16.hip", "attnbwd_decode.hip", "attnbwd_short.hip")]
LIB = os.path.join(HERE, "libattnbwd.so")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# the host compilation pass does not know the GPU feature; that line is expected
_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    return res.returncode, err


def build(verbose: bool = False, extra: list | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    pid = os.getpid()
    work = os.path.join(OBJDIR, str(pid))  # objects and the compiler's temporaries
    os.makedirs(work, exist_ok=True)
    objs = [os.path.join(work, os.path.basename(s)[:-4] + ".o") for s in SRCS]
    cmds = [[hipcc, *HIPCC_FLAGS, *(extra or []), "-save-temps=obj", "-I", INCLUDE, "-c", "-o",
             o, s] for s, o in zip(SRCS, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    failed = False
    for rc, err in results:
        if err.strip():
            print(err, file=sys.stderr)
        failed |= rc != 0
    tmp = LIB + ".tmp%d" % pid
    try:
        if failed:
            raise RuntimeError("hipcc failed")
        check_assembly([os.path.join(work, os.path.basename(s)[:-4] + "-hip-amdgcn-amd-amdhsa-gfx950.s")
                        for s in SRCS])
        rc, err = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       verbose)
        if err.strip():
            print(err, file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f"linking {LIB} failed ({rc})")
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(work, ignore_errors=True)
    return LIB


def check_assembly(paths):
    """Refuse the build when a join block of the gfx950 assembly holds a
    vector instruction before the execution mask is restored."""
    from causal_gqa_attention_bwd_amd.codegen_check import scan
    bad = []
    for p in paths:
        if not os.path.exists(p):
            raise RuntimeError(f"the compiler left no assembly at {p}")
        bad += [(os.path.basename(p), *hit) for hit in scan(open(p).read())]
    if bad:
        text = "\n".join(f"  {f}: {fn} line {line}: {ins[:3]}" for f, fn, line, ins in bad)
        raise RuntimeError("vector instructions between a join label and the restore of the "
                           "execution mask (a miscompile the library build refuses):\n" + text)


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
