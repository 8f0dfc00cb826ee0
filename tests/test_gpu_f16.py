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
bit), repeatability, and the two large workloads element by element over
whole tensors in the launch configuration bench.py times.
"""
import numpy as np
import pytest

import oracle
from causal_gqa_attention_bwd_amd.workloads import make_inputs, random_problem
from tests.gpu_helpers import TOL, gpu_bwd
from tests.fullsize_ref import reference, rel_errs
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
def test_f16_fullsize_whole_tensor(wid, with_o):
    # every element of dQ, dK, dV against the oracle's backward (the oracle's
    # forward O and LSE of every row as inputs), at the spec bar
    x, O, lse, ref = reference(wid)
    w = x["workload"]
    say(f"[gpu] workload {wid}: attn_bwd_f16 S={w.S} H={w.H} KV={w.KV} d={w.d} "
        f"O={'given' if with_o else 'none'}, every element")
    got = gpu_bwd(x, lse, O=O if with_o else None, use_seg=bool(np.any(x["seg"])), f16=True)
    errs = rel_errs(got, ref)
    say(f"[gpu] workload {wid} f16: rel err " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= TOL, f"workload {wid} f16: {name} rel err {e:.3e} > {TOL}"
