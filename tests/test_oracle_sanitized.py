"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
errors abort) runs every entry point on small problems that reach its edge
cases -- a single row, rows that see no key, packed and arbitrary document
starts, GQA groups, the row-selected and RoPE entries, the single-query
backward, several threads -- in a child process with the sanitizer runtime
preloaded, and must give the same numbers as the normal build.  CPU only."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")

CHILD = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, {root!r})
    import oracle
    from causal_gqa_attention_bwd_amd.workloads import random_problem, seg_from_lengths

    def run_all():
        out = []
        rng = np.random.default_rng(77)
        cases = [(1, 2, 1, 16, None), (7, 3, 3, 4, [0, 0, 2, 2, 9, 9, 6]),
                 (40, 4, 2, 8, seg_from_lengths([5, 17, 30], 40)),
                 (33, 8, 2, 16, np.minimum(rng.integers(0, 33, 33), np.arange(33)))]
        for S, H, KV, d, seg in cases:
            p = random_problem(rng, S, H, KV, d, seg=seg)
            for nt in (1, 3):
                O, L = oracle.attn_fwd(p["Q"], p["K"], p["V"], p["seg"], p["scale"], nthreads=nt)
                out += [O, L]
                out += list(oracle.attn_bwd(p["Q"], p["K"], p["V"], p["dO"], L, p["seg"],
                                            p["scale"], nthreads=nt))
                out += list(oracle.attn_bwd(p["Q"], p["K"], p["V"], p["dO"], L, p["seg"],
                                            p["scale"], O=O, nthreads=nt))
                if d % 2 == 0:
                    out += list(oracle.attn_bwd(p["Q"], p["K"], p["V"], p["dO"], L, p["seg"],
                                                p["scale"], rope=(500.0, 3), nthreads=nt))
            rows = np.array(sorted(set([0, S // 2, S - 1])), np.int32)
            out += list(oracle.attn_fwd_rows(p["Q"], p["K"], p["V"], p["seg"], p["scale"], rows,
                                             want_o=True))
            out += list(oracle.attn_bwd_rows(p["Q"], p["K"], p["V"], p["dO"], L, p["seg"],
                                             p["scale"], rows, rows))
            q = p["Q"][0]
            P = np.exp(rng.standard_normal((H, S)))
            P = (P / P.sum(axis=1, keepdims=True)).astype(np.float32)
            out += list(oracle.attn_bwd_decode(q, p["K"], p["V"], P, p["dO"][0], p["scale"]))
        return out

    ref = run_all()
    with oracle._use_library(sys.argv[1]):
        got = run_all()
    assert len(ref) == len(got)
    for a, b in zip(ref, got):
        assert a is None and b is None or np.array_equal(a, b), "sanitized build differs"
    print("sanitized oracle: %d arrays equal" % len(got))
""")


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", str(so), SRC, "-lm"], check=True)
    script = tmp_path / "child.py"
    script.write_text(CHILD.format(root=ROOT))
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, str(script), str(so)], env=env, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "arrays equal" in res.stdout
