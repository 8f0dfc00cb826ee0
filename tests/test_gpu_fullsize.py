"""GPU parity at the full sizes of the two large workloads (S=4096, H=32, KV=8,
d=128 plain causal; S=16384, H=16, KV=2, d=256 packed documents), element by
element over whole tensors, in the launch configuration bench.py times (a
plain causal mask goes in as a NULL seg, as bench.py passes it).

The oracle forward gives O and LSE of every row; the oracle backward on that
LSE gives dQ, dK, dV of every row (tests/fullsize_ref.py, computed once per
session).  Bar: max|gpu - oracle| <= 2e-3 * max|oracle| for each of dQ, dK,
dV.  Covered here: attn_bwd, attn_bwd_o (given the oracle's O: its row term
dO . O equals the pages' sum_j P dP up to the fp32 rounding of O and LSE,
about 1e-7 relative), the forward attn_fwd_lse, and the document-sum
invariants on the GPU's own forward LSE.  attn_bwd_f16 at these sizes is in
test_gpu_f16.py, on the same references."""
import numpy as np
import pytest
import torch

from causal_gqa_attention_bwd_amd import binding
from tests.fullsize_ref import reference, rel_errs
from tests.gpu_helpers import TOL, dev, gpu_bwd, seg_dev, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def doc_bounds(seg):
    starts = np.unique(np.asarray(seg, np.int64))
    ends = np.r_[starts[1:], len(seg)]
    return list(zip(starts.tolist(), ends.tolist()))


@pytest.mark.parametrize("entry", ["attn_bwd", "attn_bwd_o"])
@pytest.mark.parametrize("wid", [4, 5])
def test_fullsize_whole_tensor_parity(wid, entry):
    x, O, lse, ref = reference(wid)
    w = x["workload"]
    say(f"[gpu] workload {wid}: {entry} S={w.S} H={w.H} KV={w.KV} d={w.d}, every element")
    got = gpu_bwd(x, lse, use_seg=bool(np.any(x["seg"])), O=O if entry == "attn_bwd_o" else None)
    errs = rel_errs(got, ref)
    say(f"[gpu] workload {wid} {entry}: rel err " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= TOL, f"workload {wid} {entry}: {name} rel err {e:.3e} > {TOL}"


@pytest.mark.parametrize("wid", [4, 5])
def test_fullsize_forward(wid):
    x, O_ref, lse_ref, _ = reference(wid)
    w = x["workload"]
    say(f"[gpu] workload {wid}: attn_fwd_lse, every row")
    t = {k: to_dev(x[k]) for k in ("Q", "K", "V")}
    lse = torch.empty((w.S, w.H), dtype=torch.float32, device=dev())
    O = torch.empty_like(t["Q"])
    binding.attn_fwd_lse(t["Q"], t["K"], t["V"], seg_dev(x["seg"]), O, lse, float(x["scale"]))
    torch.cuda.synchronize()
    e_lse = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref)))
    e_o = float(np.max(np.abs(O.cpu().numpy().astype(np.float64) - O_ref))) / float(np.max(np.abs(O_ref)))
    say(f"[gpu] workload {wid}: forward max|LSE err| {e_lse:.2e}, O rel err {e_o:.2e}")
    assert e_lse <= 2e-5 * max(1.0, float(np.max(np.abs(lse_ref))))
    assert e_o <= TOL


@pytest.mark.parametrize("wid", [4, 5])
def test_fullsize_document_invariants(wid):
    # with an exact LSE the probabilities of a row sum to one, so for every
    # document and KV head sum_j dK_j = 0 and sum_j dV_j = the sum of dO over
    # the document's queries and the group's heads; here on the GPU's own LSE
    x, _, _, _ = reference(wid)
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
