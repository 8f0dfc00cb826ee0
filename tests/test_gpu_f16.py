"""GPU parity of attn_bwd_f16 (fp16 matrix-core operands, fp32 accumulation)
against the fp64 oracle.  The oracle computes the exact sums; the variant's
error comes from rounding the product operands to fp16 (unit roundoff
u = 2^-11, about 4.9e-4).

Bars: the five workloads (whole, or on sampled rows at full size) are held to
the same bar as the fp32 path, max|gpu - oracle| <= 2e-3 * max|oracle| per
gradient (they measure 4e-4 .. 1.2e-3).  The small edge shapes are held to
2e-2 (about 40 u): on rows that see one or two keys, under arbitrary
document starts or with rows that see no key, dS = P (dP - D) is a small
difference of nearly equal fp16 products and the error relative to the
largest gradient grows to tens of u (measured at most 5.7e-3 here, at S = 2,
and 1.56e-2 over 1000 seeded random shapes, with every token its own
document).

Covered: the small workloads whole, every padded head-dim class with ragged
tails and every mask kind (plain causal, documents, arbitrary starts, empty
rows), with and without the forward output, nonzero initial outputs (+=),
the paired schedule of plain causal calls against the unpaired one (bit for
bit), repeatability, and the two large workloads on sampled rows in the
launch configuration bench.py times.
"""
import numpy as np
import pytest

import oracle
from causal_gqa_attention_bwd_amd.workloads import make_inputs, random_problem
from tests.gpu_helpers import TOL, gpu_bwd
from tests.test_gpu_fullsize import sample_rows
from tests.test_gpu_parity import EDGE, check_full, make_seg

pytestmark = pytest.mark.gpu

TOL_F16_EDGE = 2e-2  # edge shapes: about 40 fp16 unit roundoffs (see above)
# With every token its own document, dQ and dK are zero in exact arithmetic,
# but with fp16 operands P = 1 holds only up to the fp16 rounding of the
# recomputed score against the given LSE, so they carry residues of order
# u * |score| * |dP| * |K|, which no fraction of the largest gradient bounds;
# that case is held to the bar through the fp32 entries only.
EDGE_F16 = [c for c in EDGE if c[4] != "singletons"]


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("wid", [1, 2, 3])
def test_f16_workload_parity(wid, with_o):
    check_full(make_inputs(wid), f"workload {wid} f16", with_o=with_o, f16=True)


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("case", EDGE_F16, ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
def test_f16_edge_parity(case, with_o):
    S, H, KV, d, kind = case
    rng = np.random.default_rng(3000 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    check_full(p, "edge f16 " + "S%dH%dKV%dd%d_%s" % case, with_o=with_o, f16=True,
               tol=TOL_F16_EDGE)


def test_f16_accumulates():
    x = make_inputs(3)
    rng = np.random.default_rng(2103)
    init = [rng.standard_normal(x[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    check_full(x, "workload 3 += f16", init=init, f16=True)


@pytest.mark.parametrize("shape", [(65, 2, 2, 32), (333, 4, 1, 256), (700, 8, 2, 128)],
                         ids=lambda c: "S%dH%dKV%dd%d" % c)
def test_f16_paired_equals_unpaired_and_repeats(shape):
    S, H, KV, d = shape
    p = random_problem(np.random.default_rng(9400 + S), S, H, KV, d)
    O, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], None, p["scale"])
    for o in (None, O):
        say(f"[gpu] f16 paired vs unpaired S{S} H{H} KV{KV} d{d} O={'yes' if o is not None else 'no'}")
        a = gpu_bwd(p, lse, use_seg=False, O=o, f16=True)
        b = gpu_bwd(p, lse, O=o, f16=True)
        c = gpu_bwd(p, lse, use_seg=False, O=o, f16=True)
        for x, y, z in zip(a, b, c):
            assert np.array_equal(x, y) and np.array_equal(x, z)


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("wid", [4, 5])
def test_f16_fullsize_sampled(wid, with_o):
    x = make_inputs(wid)
    w = x["workload"]
    q_rows, k_rows = sample_rows(x, np.random.default_rng(7200 + wid))
    need = oracle.rows_needed(x["seg"], w.S, q_rows, k_rows)
    say(f"[gpu] workload {wid} f16: oracle forward on {len(need)} rows")
    o_need, lse_need = oracle.attn_fwd_rows(x["Q"], x["K"], x["V"], x["seg"], x["scale"], need,
                                            want_o=True)
    n_vis = np.maximum(np.arange(w.S) - x["seg"].astype(np.int64) + 1, 1)
    lse = np.repeat(np.log(n_vis).astype(np.float32)[:, None], w.H, axis=1)
    lse[need] = lse_need
    O = None
    if with_o:
        O = np.zeros(x["Q"].shape, np.float32)  # rows no compared output depends on: D = 0
        O[need] = o_need
    say(f"[gpu] workload {wid} f16: oracle backward on {len(q_rows)} / {len(k_rows)} rows")
    rq, rk, rv = oracle.attn_bwd_rows(x["Q"], x["K"], x["V"], x["dO"], lse, x["seg"], x["scale"],
                                      q_rows, k_rows, O=O)
    say(f"[gpu] workload {wid}: attn_bwd_f16 S={w.S} H={w.H} KV={w.KV} d={w.d}")
    dQ, dK, dV = gpu_bwd(x, lse, O=O, use_seg=bool(np.any(x["seg"])), f16=True)
    for name, got, ref in (("dQ", dQ[q_rows], rq), ("dK", dK[k_rows], rk), ("dV", dV[k_rows], rv)):
        assert np.all(np.isfinite(got))
        e = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        say(f"[gpu] workload {wid} f16: {name} sampled rel err {e:.2e}")
        assert e <= TOL, f"workload {wid}: {name} rel err {e:.3e} > {TOL}"
