"""The oracle's whole-tensor results on the two large workloads (S=4096, H=32,
KV=8, d=128 plain causal; S=16384, H=16, KV=2, d=256 packed documents),
computed once per test session and shared by the full-size GPU tests.

For each: the seeded inputs, the oracle forward (O and LSE of every row, fp64
math rounded to fp32) and the oracle backward on that LSE with zero initial
outputs (D = sum_j P * dP, the pages' definition), all rows and heads.  The
host pays about 20 s (S=4096) and 60 s (S=16384) on 16 threads, once."""
import functools
import time

import numpy as np

import oracle
from causal_gqa_attention_bwd_amd.workloads import make_inputs


def say(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=2)
def reference(wid):
    """(inputs, O, LSE, (dQ, dK, dV)) of workload wid, from the oracle."""
    x = make_inputs(wid)
    w = x["workload"]
    t0 = time.perf_counter()
    say(f"[oracle] workload {wid}: forward, S={w.S} H={w.H} KV={w.KV} d={w.d}")
    O, lse = oracle.attn_fwd(x["Q"], x["K"], x["V"], x["seg"], x["scale"], want_o=True)
    t1 = time.perf_counter()
    say(f"[oracle] workload {wid}: forward {t1 - t0:.1f} s; backward of every row")
    grads = oracle.attn_bwd(x["Q"], x["K"], x["V"], x["dO"], lse, x["seg"], x["scale"])
    say(f"[oracle] workload {wid}: backward {time.perf_counter() - t1:.1f} s")
    return x, O, lse, grads


def rel_errs(got, ref):
    """max|got - ref| / max|ref| per tensor, over every element."""
    out = {}
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{name} has non-finite values"
        num = float(np.max(np.abs(g.astype(np.float64) - r.astype(np.float64))))
        out[name] = num / max(float(np.max(np.abs(r))), 1e-30)
    return out


@functools.lru_cache(maxsize=2)
def rope_reference(wid, base, pos_offset):
    """The oracle's dQ, dK, dV of workload wid with the page's RoPE backward
    (base, pos_offset) applied to dQ and dK, on the oracle's LSE."""
    x, _, lse, _ = reference(wid)
    t0 = time.perf_counter()
    say(f"[oracle] workload {wid}: backward with RoPE (base {base}, offset {pos_offset})")
    grads = oracle.attn_bwd(x["Q"], x["K"], x["V"], x["dO"], lse, x["seg"], x["scale"],
                            rope=(base, pos_offset))
    say(f"[oracle] workload {wid}: backward with RoPE {time.perf_counter() - t0:.1f} s")
    return grads
