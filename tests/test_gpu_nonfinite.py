"""Non-finite inputs (the pages guard them with nan_guard / is_finite; here the
policy is IEEE propagation, with tile-sized isolation): a NaN or an infinity
in an input row of one document reaches no output row of another document
from which a boundary at a multiple of 128 rows separates it -- every kernel
tiles rows in aligned blocks of at most 128, a query tile sweeps keys only
from its rows' smallest document start, and a key tile visits only query
blocks that can see it -- so those rows come out bit for bit as without the
non-finite values.  Inside its own document the value propagates: a query row
that sees a NaN key gets a NaN gradient (rows that share a tile with it may
too, even where the mask hides it).

Two documents [0, 256) and [256, 512); NaN in K, V, Q, dO rows and +inf in a
K row of the second; every entry point, both ways of running the key-major
pass."""
import numpy as np
import pytest

import oracle
from causal_gqa_attention_bwd_amd.workloads import random_problem, seg_from_lengths
from tests.gpu_helpers import gpu_bwd

pytestmark = pytest.mark.gpu

ENTRIES = ["attn_bwd", "attn_bwd_recompute", "attn_bwd_o", "attn_bwd_rope", "attn_bwd_f16",
           "attn_bwd_f16_o", "attn_bwd_short", "attn_bwd_short_o", "attn_bwd_noalloc"]


def say(msg):
    print(msg, flush=True)


def run(entry, p, lse, O, scratch_limit):
    if entry == "attn_bwd_recompute":
        scratch_limit(0)
    kw = dict(O=O if entry.endswith("_o") else None, f16=entry.startswith("attn_bwd_f16"),
              short=entry.startswith("attn_bwd_short"),
              rope=(1e4, 0) if entry == "attn_bwd_rope" else None)
    if entry == "attn_bwd_noalloc":
        import torch
        from causal_gqa_attention_bwd_amd import binding
        from tests.gpu_helpers import seg_dev, to_dev
        t = {k: to_dev(p[k]) for k in ("Q", "K", "V", "dO")}
        out = [torch.zeros_like(t["Q"]), torch.zeros_like(t["K"]), torch.zeros_like(t["V"])]
        binding.attn_bwd_noalloc(t["Q"], t["K"], t["V"], t["dO"], to_dev(lse), seg_dev(p["seg"]),
                                 *out, float(p["scale"]))
        torch.cuda.synchronize()
        return [o.cpu().numpy() for o in out]
    return gpu_bwd(p, lse, **kw)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("entry", ENTRIES)
def test_nonfinite_input_stays_in_its_document(entry, d, scratch_limit):
    S, H, KV = 512, 4, 2
    rng = np.random.default_rng(9900 + d)
    p = random_problem(rng, S, H, KV, d, seg=seg_from_lengths([256, 256], S))
    O, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], p["seg"], p["scale"], want_o=True)
    clean = run(entry, p, lse, O, scratch_limit)
    bad = {k: p[k].copy() for k in ("Q", "K", "V", "dO")}
    bad["K"][300, 1, 5] = np.nan
    bad["K"][420, 0, 7] = np.inf
    bad["V"][333, 1, 2] = np.nan
    bad["Q"][400, 3, 9] = np.nan
    bad["dO"][470, 2, 11] = np.nan
    q = dict(p, **bad)
    got = run(entry, q, lse, O, scratch_limit)
    say(f"[gpu] {entry} d={d}: first document unchanged, second document non-finite")
    for name, c, g in zip(("dQ", "dK", "dV"), clean, got):
        assert np.all(np.isfinite(c[:256])), f"{entry}: clean {name} not finite"
        assert np.array_equal(c[:256], g[:256]), f"{entry}: {name} of the first document changed"
    # row 301 sees the NaN key 300 (same document, KV head 0 of head 1's group
    # is KV head 0; key 300 has the NaN in KV head 1, seen by heads 2 and 3)
    assert np.isnan(got[0][301, 2:]).any(), f"{entry}: a row that sees the NaN key stayed finite"
