"""GPU parity of attn_bwd_f16 (fp16 matrix-core operands, fp32 accumulation)
against the fp64 oracle.  The oracle computes the exact sums; the variant's
error comes from rounding the product operands to fp16 (unit roundoff
u = 2^-11, about 4.9e-4).

Bars: the five workloads (whole tensors, also at full size) are held to the
same bar as the fp32 path, max|gpu - oracle| <= 2e-3 * max|oracle| per
gradient (they measure 4e-4 .. 1.2e-3).  The small edge shapes, where rows
see one or two keys and dS = P (dP - D) is a small difference of nearly equal
fp16 products, are held element by element to twice the first-order fp16
rounding bound derived from the inputs before the run (tests/f16_bounds.py),
including the shapes with every token its own document, whose dQ and dK are
zero in exact arithmetic.

Covered: the small workloads whole, every padded head-dim class with ragged
tails and every mask kind (plain causal, documents, arbitrary starts, empty
rows), with and without the forward output, nonzero initial outputs (+=),
dQ from the dS tiles the key-major pass stores and, below the scratch limit
they need, with dS formed again by the query-major pass,
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

U16 = 2.0 ** -11     # fp16 unit roundoff
# With every token its own document, dQ and dK are zero in exact arithmetic,
# but with fp16 operands P = 1 holds only up to the fp16 rounding of the
# recomputed score against the given LSE, so they carry residues of order
# u * |score| * |dP| * |K|, which no fraction of the largest gradient bounds:
# those shapes get the element-wise bound derived in singleton_bounds below.
SINGLETONS = [c for c in EDGE if c[4] == "singletons"]


def singleton_bounds(p):
    """Element-wise bounds on |dQ|, |dK| (zero in exact arithmetic) and on
    |dV - exact dV| when every token is its own document, from fp16 operand
    rounding (u = 2^-11; fp32 sums and exponentials add terms of 1e-7).

    Row s sees only key s (head h, KV head kv = h / g), P = 1 exactly.  With
    the operands rounded, the score moves by at most a = 2u scale sum_i
    |q_i k_i| and dP by at most 2u b, b = sum_i |dO_i v_i|, so P = 1 + e with
    |e| <= a (to first order), and dS/scale = P (dP - D) is at most
    |dP| a + 2u b whether D comes from the same P and dP (D = P dP) or from
    the forward output (D = dO . v exactly).  Then |dQ_s| <= scale |dS/scale|
    |K_s|, |dK_s| <= scale sum_h |dS/scale|_h |Q_s,h|, and |dV_s - sum_h dO_s,h|
    <= sum_h (a + 2u) |dO_s,h|, each times (1 + 3u) for the rounding of the
    last product's operands; a factor 2 covers second-order terms."""
    Q, K, V, dO = (np.asarray(p[k], np.float64) for k in ("Q", "K", "V", "dO"))
    S, H, d = Q.shape
    KV = K.shape[1]
    g = H // KV
    sc = float(p["scale"])
    Kh = np.repeat(K, g, axis=1)            # [S, H, d]: the key of each head's group
    Vh = np.repeat(V, g, axis=1)
    a = 2 * U16 * sc * np.sum(np.abs(Q * Kh), axis=2)          # [S, H]
    b = np.sum(np.abs(dO * Vh), axis=2)
    dP = np.sum(dO * Vh, axis=2)
    ds = np.abs(dP) * a + 2 * U16 * b                           # bound on |dS/scale|
    f = 2 * (1 + 3 * U16)
    bq = f * sc * ds[:, :, None] * np.abs(Kh)                   # [S, H, d]
    bk = f * sc * (ds[:, :, None] * np.abs(Q)).reshape(S, KV, g, d).sum(axis=2)
    bv = f * ((a + 2 * U16)[:, :, None] * np.abs(dO)).reshape(S, KV, g, d).sum(axis=2)
    exact_dv = dO.reshape(S, KV, g, d).sum(axis=2)
    return bq, bk, bv, exact_dv


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("wid", [1, 2, 3])
def test_f16_workload_parity(wid, with_o):
    check_full(make_inputs(wid), f"workload {wid} f16", with_o=with_o, f16=True)


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("case", EDGE, ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
def test_f16_edge_parity(case, with_o):
    # every element within twice its fp16 rounding bound (tests/f16_bounds.py)
    S, H, KV, d, kind = case
    rng = np.random.default_rng(3000 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    check_full(p, "edge f16 " + "S%dH%dKV%dd%d_%s" % case, with_o=with_o, f16=True,
               f16_bound=True)


DS_CASES = [(513, 16, 2, 64, "docs"), (320, 8, 1, 128, "arbitrary"), (257, 4, 2, 192, "docs"),
            (161, 4, 2, 256, "docs"), (300, 2, 1, 240, "empty_rows"), (700, 8, 2, 128, "causal")]


def ds_tile_bytes(S, H):
    # the stored dS/scale tiles of every slot of the causal bound, 2 KiB each
    nblk = (S + 31) // 32
    return nblk * (nblk + 1) // 2 * H * 2048


@pytest.mark.parametrize("rope", [None, (500.0, 13)], ids=["plain", "rope"])
@pytest.mark.parametrize("limit", ["exact", "below"])
@pytest.mark.parametrize("case", DS_CASES, ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
def test_f16_stored_and_recomputed_ds(case, limit, rope, scratch_limit):
    # dQ from the dS tiles the key-major pass stored (a scratch limit they
    # fill exactly), or, one byte below it, with dS formed again by the
    # query-major pass; both with and without the forward output
    S, H, KV, d, kind = case
    rng = np.random.default_rng(9700 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    scratch_limit(ds_tile_bytes(S, H) - (limit == "below"))
    for with_o in (False, True):
        check_full(p, f"f16 dS {limit} rope={rope} " + "S%dH%dKV%dd%d_%s" % case, init=init,
                   with_o=with_o, f16=True, rope=rope, f16_bound=True)


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
    # forward O and LSE of every row as inputs), within 2e-3 of the largest element of each gradient
    x, O, lse, ref = reference(wid)
    w = x["workload"]
    say(f"[gpu] workload {wid}: attn_bwd_f16 S={w.S} H={w.H} KV={w.KV} d={w.d} "
        f"O={'given' if with_o else 'none'}, every element")
    got = gpu_bwd(x, lse, O=O if with_o else None, use_seg=bool(np.any(x["seg"])), f16=True)
    errs = rel_errs(got, ref)
    say(f"[gpu] workload {wid} f16: rel err " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= TOL, f"workload {wid} f16: {name} rel err {e:.3e} > {TOL}"


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("case", SINGLETONS, ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
def test_f16_singletons_within_the_rounding_bound(case, with_o):
    # every token its own document: dQ = dK = 0 and dV = sum of dO over the
    # group in exact arithmetic; the fp16 operands leave residues that must
    # stay inside the element-wise rounding bounds derived up front
    S, H, KV, d, kind = case
    rng = np.random.default_rng(3000 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    O, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], p["seg"], p["scale"], want_o=True)
    dQ, dK, dV = gpu_bwd(p, lse, O=O if with_o else None, f16=True)
    bq, bk, bv, exact_dv = singleton_bounds(p)
    say(f"[gpu] singletons f16 S{S} H{H} KV{KV} d{d}: |dQ|/bound {np.max(np.abs(dQ) / bq):.2f}, "
        f"|dK|/bound {np.max(np.abs(dK) / bk):.2f}, |dV err|/bound {np.max(np.abs(dV - exact_dv) / bv):.2f}")
    assert np.all(np.abs(dQ) <= bq)
    assert np.all(np.abs(dK) <= bk)
    assert np.all(np.abs(dV - exact_dv) <= bv)
