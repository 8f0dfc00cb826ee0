"""GPU parity of attn_bwd_o (the row term read off the forward output O)
against the oracle's O entry, on the same seeded inputs and the same fp32 O:
the workloads that finish quickly, edge shapes of every head-dim class, both
ways of running the key-major pass, accumulation into nonzero outputs, a
perturbed O (which the result must follow, so the kernels read D off O), and
sampled rows of the two large workloads."""
import numpy as np
import pytest

import oracle
from causal_gqa_attention_bwd_amd.workloads import make_inputs, random_problem
from tests.gpu_helpers import TOL, gpu_bwd
from tests.test_gpu_fullsize import sample_rows
from tests.test_gpu_parity import check_full, make_seg

pytestmark = pytest.mark.gpu

EDGE_O = [
    (2, 2, 1, 32, "causal"),
    (97, 3, 1, 64, "arbitrary"),
    (130, 8, 2, 80, "docs"),
    (65, 2, 2, 96, "empty_rows"),
    (129, 4, 1, 128, "causal"),
    (150, 4, 2, 160, "docs"),
    (257, 4, 2, 192, "docs"),
    (161, 4, 2, 256, "docs"),
]


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_o_entry_workloads(wid):
    check_full(make_inputs(wid), f"workload {wid}", with_o=True)


@pytest.mark.parametrize("case", EDGE_O, ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
@pytest.mark.parametrize("mb", ["default", "0"])
def test_o_entry_edge_shapes(case, mb, monkeypatch):
    if mb != "default":
        monkeypatch.setenv("ATTNBWD_SCRATCH_MB", mb)
    S, H, KV, d, kind = case
    rng = np.random.default_rng(6000 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    check_full(p, "edge " + "S%dH%dKV%dd%d_%s" % case + f" budget={mb}", with_o=True)


@pytest.mark.parametrize("mb", ["default", "0"])
def test_o_entry_follows_a_perturbed_O(mb, monkeypatch):
    if mb != "default":
        monkeypatch.setenv("ATTNBWD_SCRATCH_MB", mb)
    x = make_inputs(3)
    rng = np.random.default_rng(6003)
    shift = (0.5 * rng.standard_normal(x["Q"].shape)).astype(np.float32)
    check_full(x, f"workload 3 perturbed O budget={mb}", with_o=True, o_shift=shift)


def test_o_entry_accumulates():
    x = make_inputs(2)
    rng = np.random.default_rng(6002)
    init = [rng.standard_normal(x[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    check_full(x, "workload 2 += (O entry)", init=init, with_o=True)


@pytest.mark.parametrize("wid", [4, 5])
def test_o_entry_fullsize_sampled(wid):
    x = make_inputs(wid)
    w = x["workload"]
    q_rows, k_rows = sample_rows(x, np.random.default_rng(7100 + wid))
    need = oracle.rows_needed(x["seg"], w.S, q_rows, k_rows)
    say(f"[gpu] workload {wid}: oracle forward (O, LSE) on {len(need)} rows")
    o_need, lse_need = oracle.attn_fwd_rows(x["Q"], x["K"], x["V"], x["seg"], x["scale"], need,
                                            want_o=True)
    n_vis = np.maximum(np.arange(w.S) - x["seg"].astype(np.int64) + 1, 1)
    lse = np.repeat(np.log(n_vis).astype(np.float32)[:, None], w.H, axis=1)
    lse[need] = lse_need
    O = np.zeros(x["Q"].shape, np.float32)   # rows no compared output depends on: D = 0
    O[need] = o_need
    say(f"[gpu] workload {wid}: oracle backward (O entry) on {len(q_rows)} / {len(k_rows)} rows")
    rq, rk, rv = oracle.attn_bwd_rows(x["Q"], x["K"], x["V"], x["dO"], lse, x["seg"], x["scale"],
                                      q_rows, k_rows, O=O)
    say(f"[gpu] workload {wid}: attn_bwd_o S={w.S} H={w.H} KV={w.KV} d={w.d}")
    dQ, dK, dV = gpu_bwd(x, lse, O=O, use_seg=bool(np.any(x["seg"])))
    for name, got, ref in (("dQ", dQ[q_rows], rq), ("dK", dK[k_rows], rk), ("dV", dV[k_rows], rv)):
        assert np.all(np.isfinite(got))
        e = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        say(f"[gpu] workload {wid}: {name} sampled rel err {e:.2e}")
        assert e <= TOL, f"workload {wid}: {name} rel err {e:.3e} > {TOL}"
