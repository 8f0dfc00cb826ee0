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
test_gpu_f16.py, on the same references.  At S=32768 (H=32, KV=8, d=128)
attn_bwd and attn_bwd_f16 (its dS tiles stored, or formed again) are compared
on sampled rows."""
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


_LONG = {}


def long_sample():
    """S=32768, H=32, KV=8, d=128 plain causal (the long workload): its inputs,
    the sampled rows and the oracle's gradients of them, computed once per
    session.  The oracle computes LSE for the rows the compared outputs read
    and the gradients of sampled rows: 24 dQ rows spread over the sequence and
    the dK, dV rows of 6 keys in the last 256 positions (each output row covers
    every head); the other rows get ln(#visible keys), a finite LSE none of
    the compared outputs reads."""
    if not _LONG:
        import oracle
        from causal_gqa_attention_bwd_amd.workloads import make_inputs
        x = make_inputs(6)
        w = x["workload"]
        rng = np.random.default_rng(6060)
        q_rows = np.unique(np.r_[0, 1, 31, 32, 4095, 16384, w.S - 1,
                                 rng.integers(0, w.S, 17)]).astype(np.int32)
        k_rows = np.array([w.S - 256, w.S - 193, w.S - 128, w.S - 65, w.S - 2, w.S - 1], np.int32)
        need = oracle.rows_needed(None, w.S, q_rows, k_rows)
        say(f"[oracle] workload 6: LSE of {len(need)} rows, gradients of {len(q_rows)} dQ rows "
            f"and {len(k_rows)} dK/dV rows")
        lse = np.log(np.arange(1, w.S + 1, dtype=np.float64))[:, None].repeat(w.H, axis=1)
        _, lse_need = oracle.attn_fwd_rows(x["Q"], x["K"], x["V"], None, x["scale"], need,
                                           nthreads=16)
        lse = lse.astype(np.float32)
        lse[need] = lse_need
        ref = oracle.attn_bwd_rows(x["Q"], x["K"], x["V"], x["dO"], lse, None, x["scale"],
                                   q_rows, k_rows, nthreads=16)
        _LONG.update(x=x, lse=lse, q_rows=q_rows, k_rows=k_rows, ref=ref)
    return _LONG


def check_long_sample(tag, got):
    s = long_sample()
    rq, rk, rv = s["ref"]
    dQ, dK, dV = got
    for name, g, r in (("dQ", dQ[s["q_rows"]], rq), ("dK", dK[s["k_rows"]], rk),
                       ("dV", dV[s["k_rows"]], rv)):
        e = float(np.max(np.abs(g - r))) / float(np.max(np.abs(r)))
        say(f"[gpu] {tag} sampled {name}: rel err {e:.2e}")
        assert e <= TOL, f"{tag}: {name} rel err {e:.3e} > {TOL}"


def test_long_sequence_in_head_chunks_sampled():
    # the stored tiles of all heads (137 GB) exceed the default scratch limit,
    # so the stored-tile passes run in chunks of one KV group, the launch
    # configuration bench.py times for this workload; the sampled rows against
    # the oracle, then every row held to the document-sum invariants on the
    # GPU's own forward LSE
    s = long_sample()
    x, lse = s["x"], s["lse"]
    w = x["workload"]
    heads = binding.bwd_plan_heads(w.S, w.H, w.KV, w.d)[1]
    assert 0 < heads < w.H, "expected stored tiles in head chunks at this size"
    say(f"[gpu] workload 6: attn_bwd S={w.S} H={w.H} in chunks of {heads} heads")
    got = gpu_bwd(x, lse, use_seg=False)
    check_long_sample("workload 6", got)
    del got
    # invariants over every row: sum_j dK_j = 0 and sum_j dV_j = sum_s dO_s
    # (over the group's heads) with the GPU's own exact-row LSE
    t = {k: to_dev(x[k]) for k in ("Q", "K", "V", "dO")}
    L = torch.empty((w.S, w.H), dtype=torch.float32, device=dev())
    binding.attn_fwd_lse(t["Q"], t["K"], t["V"], None, None, L, float(x["scale"]))
    gq, gk, gv = (torch.zeros_like(t["Q"]), torch.zeros_like(t["K"]), torch.zeros_like(t["V"]))
    binding.attn_bwd(t["Q"], t["K"], t["V"], t["dO"], L, None, gq, gk, gv, float(x["scale"]))
    torch.cuda.synchronize()
    gk, gv = gk.double(), gv.double()
    sdo = t["dO"].double().reshape(w.S, w.KV, w.H // w.KV, w.d).sum(dim=(0, 2))
    ek = float(gk.sum(dim=0).abs().max() / gk.abs().sum(dim=0).max())
    ev = float((gv.sum(dim=0) - sdo).abs().max() / t["dO"].double().abs().reshape(
        w.S, w.KV, -1, w.d).sum(dim=(0, 2)).max())
    say(f"[gpu] workload 6: sums over every key: dK {ek:.2e}, dV - dO {ev:.2e}")
    assert ek <= 1e-4 and ev <= 1e-4


@pytest.mark.parametrize("stored", [False, True], ids=["ds_formed_again", "ds_stored"])
def test_f16_long_sequence_sampled(stored):
    # attn_bwd_f16 on the long workload: its dS tiles (2 KiB per block pair
    # and head, 34.4 GB) either just exceed the scratch limit (the query-major
    # pass forms dS again) or just fit it (k_dqs16 reads them), at the fp32
    # entry's bar
    s = long_sample()
    x, lse = s["x"], s["lse"]
    w = x["workload"]
    nblk = (w.S + 31) // 32
    ds_bytes = nblk * (nblk + 1) // 2 * w.H * 2048
    mode = "stored dS" if stored else "dS formed again"
    say(f"[gpu] workload 6: attn_bwd_f16 S={w.S} H={w.H}, {mode}")
    with binding.scratch_limit(ds_bytes if stored else ds_bytes - 1):
        got = gpu_bwd(x, lse, use_seg=False, f16=True)
    check_long_sample(f"workload 6 f16 {mode}", got)
