"""attn_bwd_noalloc (the entry that allocates nothing: its workspace is the
library's fixed 32 MiB device array) against attn_bwd (the same backward on a
workspace from the library's pool), through the C ABI, at the parity bar:
max|noalloc - attn_bwd| <= 2e-3 * max|attn_bwd| per gradient, and both
against the oracle where it is cheap.  Three calls in a row, each smaller
than the one before, so a later call runs on what an earlier one left in the
shared array:
1. S=4096, H=32, KV=8, d=128 plain causal (the benchmark's shape): the
   tiles of one head (64 MiB) do not fit, so the key-major pass recomputes
   the scores;
2. S=1024, H=8, KV=8, d=64 with documents: the tiles of 7 heads fit, so the
   stored-tile passes run in head chunks;
3. S=512, H=4, KV=2, d=32, two documents: every head's tiles fit.
"""
import numpy as np
import pytest
import torch

import oracle
from causal_gqa_attention_bwd_amd import binding
from causal_gqa_attention_bwd_amd.workloads import make_inputs
from tests.gpu_helpers import TOL, rel_err, seg_dev, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def run(entry, t, lse, seg, scale):
    out = [torch.zeros_like(t["Q"]), torch.zeros_like(t["K"]), torch.zeros_like(t["V"])]
    entry(t["Q"], t["K"], t["V"], t["dO"], lse, seg, *out, scale)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def test_noalloc_matches_attn_bwd_on_shrinking_calls():
    for wid in (4, 3, 2):
        x = make_inputs(wid)
        w = x["workload"]
        t = {k: to_dev(x[k]) for k in ("Q", "K", "V", "dO")}
        seg = seg_dev(x["seg"]) if np.any(x["seg"]) else None
        scale = float(x["scale"])
        lse = torch.empty((w.S, w.H), dtype=torch.float32, device=t["Q"].device)
        binding.attn_fwd_lse(t["Q"], t["K"], t["V"], seg, None, lse, scale)
        say(f"[gpu] workload {wid}: attn_bwd_noalloc S={w.S} H={w.H} KV={w.KV} d={w.d}")
        got = run(binding.attn_bwd_noalloc, t, lse, seg, scale)
        want = run(binding.attn_bwd, t, lse, seg, scale)
        errs = {n: rel_err(g, r) for n, g, r in zip(("dQ", "dK", "dV"), got, want)}
        say(f"[gpu] workload {wid}: noalloc vs attn_bwd " +
            ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for n, e in errs.items():
            assert np.all(np.isfinite(got[("dQ", "dK", "dV").index(n)]))
            assert e <= TOL, f"workload {wid}: {n} {e:.3e} > {TOL}"
        if wid != 4:
            ref = oracle.attn_bwd(x["Q"], x["K"], x["V"], x["dO"], lse.cpu().numpy(), x["seg"],
                                  x["scale"])
            for n, g, r in zip(("dQ", "dK", "dV"), got, ref):
                e = rel_err(g, r)
                say(f"[gpu] workload {wid}: noalloc vs oracle {n}={e:.2e}")
                assert e <= TOL


def test_noalloc_refuses_a_row_term_beyond_its_scratch():
    # 262144 rows x 64 heads: the row term alone is 64 MiB; refused on the
    # host before any GPU work (the placeholders are never read)
    lib = binding.load()
    A = 0x10000
    st = lib.attn_bwd_noalloc(A, A, A, A, A, None, A, A, A, 262144, 64, 8, 64, 0.125, None)
    assert st == binding.ATTN_ERR_UNSUPPORTED
    assert "scratch" in binding.last_error()
