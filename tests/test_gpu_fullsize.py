"""GPU parity at the full sizes of the two large workloads (S=4096, H=32, KV=8,
d=128 plain causal; S=16384, H=16, KV=2, d=256 packed documents), in the
launch configuration bench.py times.

Sampled parity: dQ rows of sampled queries and dK/dV rows of sampled keys
against the oracle's row-selected backward.  The oracle forward provides LSE
for every row those outputs depend on (the sampled queries and every query
that sees a sampled key); every other row gets the LSE of uniform attention
over its visible keys (ln of their count), a finite input that none of the
compared outputs depends on.

Invariants over all rows (any size): with an exact LSE the probabilities of a
row sum to one, so for every document and KV head sum_j dK_j = 0 and
sum_j dV_j = sum of dO over the document's queries and the group's heads.
These run on the GPU's own forward LSE.
"""
import numpy as np
import pytest
import torch

import oracle
from causal_gqa_attention_bwd_amd import binding
from causal_gqa_attention_bwd_amd.workloads import make_inputs
from tests.gpu_helpers import TOL, dev, gpu_bwd, seg_dev, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def doc_bounds(seg):
    starts = np.unique(np.asarray(seg, np.int64))
    ends = np.r_[starts[1:], len(seg)]
    return list(zip(starts.tolist(), ends.tolist()))


def sample_rows(x, rng):
    S = x["workload"].S
    base = [0, 1, 31, 32, 63, 64, 65, 127, S // 3, S // 2, S - 65, S - 33, S - 2, S - 1]
    q_rows = sorted(set(base + rng.integers(0, S, 10).tolist()))
    if not np.any(x["seg"]):
        k_rows = q_rows
    else:  # keys from the first, a middle and the last document, boundaries included
        docs = doc_bounds(x["seg"])
        pick = [docs[0], docs[len(docs) // 2], docs[-1]]
        k_rows = sorted(set(sum(([a, a + 1, (a + b) // 2, b - 2, b - 1] for a, b in pick), [])))
        k_rows = [k for k in k_rows if 0 <= k < S]
    return np.array(q_rows, np.int32), np.array(k_rows, np.int32)


@pytest.mark.parametrize("wid", [4, 5])
def test_fullsize_sampled_parity(wid):
    x = make_inputs(wid)
    w = x["workload"]
    rng = np.random.default_rng(7000 + wid)
    q_rows, k_rows = sample_rows(x, rng)
    need = oracle.rows_needed(x["seg"], w.S, q_rows, k_rows)
    say(f"[gpu] workload {wid}: oracle forward on {len(need)} rows")
    _, lse_need = oracle.attn_fwd_rows(x["Q"], x["K"], x["V"], x["seg"], x["scale"], need)
    n_vis = np.maximum(np.arange(w.S) - x["seg"].astype(np.int64) + 1, 1)
    lse = np.repeat(np.log(n_vis).astype(np.float32)[:, None], w.H, axis=1)
    lse[need] = lse_need
    say(f"[gpu] workload {wid}: oracle backward on {len(q_rows)} query / {len(k_rows)} key rows")
    rq, rk, rv = oracle.attn_bwd_rows(x["Q"], x["K"], x["V"], x["dO"], lse, x["seg"], x["scale"],
                                      q_rows, k_rows)
    say(f"[gpu] workload {wid}: attn_bwd S={w.S} H={w.H} KV={w.KV} d={w.d}")
    # a plain causal mask goes in as a NULL seg, as bench.py passes it
    dQ, dK, dV = gpu_bwd(x, lse, use_seg=bool(np.any(x["seg"])))
    errs = {}
    for name, got, ref in (("dQ", dQ[q_rows], rq), ("dK", dK[k_rows], rk), ("dV", dV[k_rows], rv)):
        assert np.all(np.isfinite(got))
        errs[name] = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    say(f"[gpu] workload {wid}: sampled rel err " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= TOL, f"workload {wid}: {name} rel err {e:.3e} > {TOL}"


@pytest.mark.parametrize("wid", [4, 5])
def test_fullsize_forward_lse_rows(wid):
    x = make_inputs(wid)
    w = x["workload"]
    rows = np.unique(np.r_[0, 1, 2, 33, w.S // 2, w.S - 1,
                           np.random.default_rng(8000 + wid).integers(0, w.S, 20)]).astype(np.int32)
    _, ref = oracle.attn_fwd_rows(x["Q"], x["K"], x["V"], x["seg"], x["scale"], rows)
    say(f"[gpu] workload {wid}: attn_fwd_lse")
    t = {k: to_dev(x[k]) for k in ("Q", "K", "V")}
    lse = torch.empty((w.S, w.H), dtype=torch.float32, device=dev())
    binding.attn_fwd_lse(t["Q"], t["K"], t["V"], seg_dev(x["seg"]), None, lse, float(x["scale"]))
    got = lse.cpu().numpy()[rows]
    assert np.max(np.abs(got - ref)) <= 2e-5 * max(1.0, float(np.max(np.abs(ref))))


@pytest.mark.parametrize("wid", [4, 5])
def test_fullsize_document_invariants(wid):
    x = make_inputs(wid)
    w = x["workload"]
    g = w.H // w.KV
    t = {k: to_dev(x[k]) for k in ("Q", "K", "V", "dO")}
    seg = seg_dev(x["seg"]) if np.any(x["seg"]) else None
    lse = torch.empty((w.S, w.H), dtype=torch.float32, device=dev())
    say(f"[gpu] workload {wid}: forward + backward for the invariants")
    binding.attn_fwd_lse(t["Q"], t["K"], t["V"], seg, None, lse, float(x["scale"]))
    dQ, dK, dV = (torch.zeros_like(t["Q"]), torch.zeros_like(t["K"]), torch.zeros_like(t["V"]))
    binding.attn_bwd(t["Q"], t["K"], t["V"], t["dO"], lse, seg, dQ, dK, dV, float(x["scale"]))
    torch.cuda.synchronize()
    dK, dV = dK.double().cpu().numpy(), dV.double().cpu().numpy()
    dO = x["dO"].astype(np.float64).reshape(w.S, w.KV, g, w.d).sum(axis=2)
    worst_k = worst_v = 0.0
    for a, b in doc_bounds(x["seg"]):
        sk = dK[a:b].sum(axis=0)                       # [KV, d]
        sv = dV[a:b].sum(axis=0) - dO[a:b].sum(axis=0)
        worst_k = max(worst_k, float(np.max(np.abs(sk)) / max(np.abs(dK[a:b]).sum(axis=0).max(), 1e-30)))
        worst_v = max(worst_v, float(np.max(np.abs(sv)) / max(np.abs(dO[a:b]).sum(axis=0).max(), 1e-30)))
    say(f"[gpu] workload {wid}: document sums: dK {worst_k:.2e}, dV - dO {worst_v:.2e} (relative to sum |.|)")
    assert worst_k <= 1e-4 and worst_v <= 1e-4
