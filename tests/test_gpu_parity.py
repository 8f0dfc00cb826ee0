"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bar: max|gpu - oracle| <= 2e-3 * max|oracle| for each of
dQ, dK, dV; the LSE fed to both sides comes from the oracle forward."""
import numpy as np
import pytest

import oracle
from causal_gqa_attention_bwd_amd import binding
from causal_gqa_attention_bwd_amd.workloads import make_inputs, random_problem, seg_from_lengths
from tests.gpu_helpers import TOL, gpu_bwd, gpu_fwd, rel_err

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def check_full(p, tag, init=None, with_o=False, o_shift=None, rope=None, f16=False, tol=TOL,
               short=False, f16_bound=False):
    """GPU vs oracle on the whole problem.  with_o: through attn_bwd_o with the
    oracle's forward output (plus o_shift, if given) on both sides.  rope =
    (base, pos_offset): through attn_bwd_rope.  f16: through attn_bwd_f16 (with
    the forward output when with_o).  short: through attn_bwd_short (likewise).
    f16_bound: hold every element to twice the fp16 rounding bound derived in
    tests/f16_bounds.py (instead of tol times the largest gradient)."""
    O, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], p["seg"], p["scale"], want_o=with_o)
    if with_o and o_shift is not None:
        O = (O + o_shift).astype(np.float32)
    ref = oracle.attn_bwd(p["Q"], p["K"], p["V"], p["dO"], lse, p["seg"], p["scale"],
                          *(init if init is not None else ()), O=O if with_o else None, rope=rope)
    entry = ("attn_bwd_short" if short else
             ("attn_bwd_f16_rope" if rope is not None else "attn_bwd_f16") if f16 else
             "attn_bwd_rope" if rope is not None else "attn_bwd_o" if with_o else "attn_bwd")
    say(f"[gpu] {tag}: {entry} S={p['Q'].shape[0]} H={p['Q'].shape[1]} "
        f"KV={p['K'].shape[1]} d={p['Q'].shape[2]}")
    got = gpu_bwd(p, lse, init=init, O=O if with_o else None, rope=rope, f16=f16, short=short)
    errs = {}
    pairs = []
    outs = []   # |the output tensors|, for the fp32 rounding of the += result
    for name, g, w, i0 in zip(("dQ", "dK", "dV"), got, ref,
                              init if init is not None else (None,) * 3):
        g, w = g.astype(np.float64), w.astype(np.float64)
        outs.append(np.abs(w))
        if i0 is not None and rope is None:   # compare the accumulated gradients
            g, w = g - i0, w - i0
        assert np.all(np.isfinite(g)), f"{tag}: {name} has non-finite values"
        pairs.append((name, g, w))
    # A tensor that is zero in exact arithmetic (dQ and dK when every row sees
    # only its own key: S = 1, or every token its own document) holds only
    # rounding noise on both sides; its bound is then taken relative to the
    # largest of the three gradients instead: a floor of 1e-3 of it for fp32
    # operands, and of 5e-2 of it for fp16 operands.  There P = 1 only up to
    # the rounding of the given LSE against the recomputed score, and dS =
    # P (dP - D) keeps a few units of rounding of dP (fp32: up to 2.8e-7 of
    # the largest gradient measured over 1000 random shapes; fp16: 2^-11
    # relative) -- the absolute bound on a zero tensor is then 2e-6 of the
    # largest gradient for fp32 operands (16 units of rounding) and 1e-3 for
    # fp16 operands (2 units).
    if f16_bound:
        from tests.f16_bounds import U32, f16_bounds, rotated
        bounds = f16_bounds(p, lse, O if with_o else None)
        if rope is not None:
            d = p["Q"].shape[2]
            bounds = (rotated(bounds[0], d), rotated(bounds[1], d), bounds[2])
        worst = 0.0
        # both sides round the accumulated output (initial value + gradient)
        # to fp32, so the allowance counts that rounding of the output, not
        # only of the gradient: with a nonzero initial value it can exceed
        # the gradient's own fp16 bound where the gradient is small
        for (name, g, w), b, o in zip(pairs, bounds, outs):
            allowed = 2.0 * b + 4.0 * U32 * (np.abs(w) + o + 1e-30)
            ratio = float(np.max(np.abs(g - w) / allowed)) if w.size else 0.0
            worst = max(worst, ratio)
            errs[name] = ratio
        say(f"[gpu] {tag}: |err| / (2 x fp16 rounding bound) " +
            ", ".join(f"{k}={v:.3f}" for k, v in errs.items()))
        for name, r in errs.items():
            assert r <= 1.0, f"{tag}: {name} exceeds twice its fp16 rounding bound ({r:.3f})"
        return got, ref
    overall = max(float(np.max(np.abs(w))) if w.size else 0.0 for _, _, w in pairs)
    floor = 5e-2 if f16 else 1e-3
    for name, g, w in pairs:
        ref_scale = max(float(np.max(np.abs(w))) if w.size else 0.0, floor * overall, 1e-30)
        errs[name] = float(np.max(np.abs(g - w))) / ref_scale if w.size else 0.0
    say(f"[gpu] {tag}: rel err " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= tol, f"{tag}: {name} rel err {e:.3e} > {tol}"
    return got, ref


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_workload_full_parity(wid):
    x = make_inputs(wid)
    check_full(x, f"workload {wid}")


# (S, H, KV, d, seg kind): every padded head-dim class, ragged tails, GQA ratios
EDGE = [
    (1, 1, 1, 16, "causal"),
    (2, 2, 1, 32, "causal"),
    (33, 4, 2, 48, "docs"),
    (97, 3, 1, 64, "arbitrary"),
    (130, 8, 2, 80, "docs"),
    (65, 2, 2, 96, "empty_rows"),
    (200, 4, 4, 112, "docs"),
    (129, 4, 1, 128, "causal"),
    (100, 2, 1, 144, "arbitrary"),
    (150, 4, 2, 160, "docs"),
    (70, 2, 2, 176, "causal"),
    (257, 4, 2, 192, "docs"),
    (90, 2, 1, 208, "arbitrary"),
    (64, 3, 3, 224, "causal"),
    (300, 2, 1, 240, "docs"),
    (161, 4, 2, 256, "docs"),
    (513, 16, 2, 64, "docs"),
    (320, 8, 1, 128, "arbitrary"),
    (5, 32, 4, 96, "singletons"),
    (3, 3, 3, 192, "singletons"),
    (70, 4, 2, 256, "singletons"),
]


def make_seg(rng, S, kind):
    if kind == "causal":
        return None
    if kind == "docs":
        lengths = []
        while sum(lengths) < S:
            lengths.append(int(rng.integers(1, max(2, S // 2))))
        return seg_from_lengths(lengths, S)
    if kind == "arbitrary":  # any 0 <= seg[s] <= s, not monotone
        return np.minimum(rng.integers(0, S, S), np.arange(S)).astype(np.uint32)
    if kind == "singletons":  # every token its own document: dQ = dK = 0 exactly
        return np.arange(S, dtype=np.uint32)
    if kind == "empty_rows":  # some rows see no key at all (seg[s] > s)
        seg = np.minimum(rng.integers(0, S, S), np.arange(S)).astype(np.uint32)
        seg[5::7] = np.minimum(np.arange(S)[5::7] + 3, 2**31 - 1)
        return seg
    raise ValueError(kind)


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
def test_edge_shapes_full_parity(case):
    S, H, KV, d, kind = case
    rng = np.random.default_rng(3000 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    check_full(p, "edge " + "S%dH%dKV%dd%d_%s" % case)


def test_accumulates_into_nonzero_outputs():
    x = make_inputs(2)
    rng = np.random.default_rng(2002)
    init = [rng.standard_normal(x[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    check_full(x, "workload 2 +=", init=init)


def test_null_seg_equals_zero_seg_and_is_deterministic():
    # a NULL seg takes the paired schedule, whose dK/dV sums over a mirror
    # tile run in the opposite order: equal to rounding there, else bit for bit
    rng = np.random.default_rng(4)
    p = random_problem(rng, 300, 4, 2, 64)
    _, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], None, p["scale"], want_o=False)
    say("[gpu] null seg vs zero seg")
    a = gpu_bwd(p, lse, use_seg=False)
    a2 = gpu_bwd(p, lse, use_seg=False)
    b = gpu_bwd(p, lse)
    c = gpu_bwd(p, lse)
    for name, x, x2, y, z in zip(("dQ", "dK", "dV"), a, a2, b, c):
        assert np.array_equal(x, x2) and np.array_equal(y, z)
        if name == "dQ":
            assert np.array_equal(x, y)
        else:
            assert float(np.max(np.abs(x - y))) <= 1e-4 * float(np.max(np.abs(y)))


def test_masked_keys_exactly_zero_and_unseen_changes_do_not_matter():
    rng = np.random.default_rng(5)
    S, H, KV, d = 160, 4, 2, 64
    seg = seg_from_lengths([50, 70, 40], S)
    p = random_problem(rng, S, H, KV, d, seg=seg)
    s_star = 100                       # in the document [50, 120)
    p["dO"][np.arange(S) != s_star] = 0.0
    _, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], seg, p["scale"], want_o=False)
    say("[gpu] masked-key zeros")
    dQ, dK, dV = gpu_bwd(p, lse)
    outside = np.r_[0:50, s_star + 1:S]
    assert np.all(dK[outside] == 0) and np.all(dV[outside] == 0)
    assert np.any(dK[50:s_star + 1] != 0)
    q2 = dict(p)
    q2["K"] = p["K"].copy()
    q2["V"] = p["V"].copy()
    q2["K"][outside] *= 50.0           # huge logits where the row cannot look
    q2["V"][outside] = -3.0
    dQ2, _, _ = gpu_bwd(q2, lse)
    assert np.array_equal(dQ2[s_star], dQ[s_star])


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_forward_lse_and_output(wid):
    x = make_inputs(wid)
    O_ref, L_ref = oracle.attn_fwd(x["Q"], x["K"], x["V"], x["seg"], x["scale"])
    say(f"[gpu] attn_fwd_lse workload {wid}")
    O, L = gpu_fwd(x)
    assert np.max(np.abs(L - L_ref)) <= 2e-5 * max(1.0, np.max(np.abs(L_ref)))
    assert rel_err(O, O_ref) <= 1e-4
    _, L2 = gpu_fwd(x, want_o=False)
    assert np.array_equal(L2, L)


def test_forward_empty_rows():
    rng = np.random.default_rng(6)
    S = 70
    seg = make_seg(rng, S, "empty_rows")
    p = random_problem(rng, S, 2, 1, 32, seg=seg)
    O_ref, L_ref = oracle.attn_fwd(p["Q"], p["K"], p["V"], seg, p["scale"])
    say("[gpu] attn_fwd_lse empty rows")
    O, L = gpu_fwd(p)
    empty = seg.astype(np.int64) > np.arange(S)
    assert np.all(np.isneginf(L[empty])) and np.all(O[empty] == 0)
    assert np.max(np.abs(L[~empty] - L_ref[~empty])) <= 2e-5 * max(1.0, np.abs(L_ref[~empty]).max())
    assert rel_err(O, O_ref) <= 1e-4


# (S, H, KV, d, splits): calls with a seg whose key-major pass has few
# workgroups (64-key tiles x KV heads) split each group's heads over `splits`
# workgroups; the first adds into dK, dV, the others' partial sums go
# through the workspace.  The plan's workspace size shows the split count;
# parity with nonzero initial outputs (the += contract through the partial
# sums) through attn_bwd and attn_bwd_rope (each partial rotated back on its
# own), and through attn_bwd_o.
HEAD_SPLITS = [
    (100, 4, 2, 64, 2),
    (130, 8, 2, 96, 4),
    (200, 16, 2, 128, 8),
    (450, 8, 1, 256, 8),
]


@pytest.mark.parametrize("case", HEAD_SPLITS, ids=lambda c: "S%dH%dKV%dd%d_x%d" % c)
@pytest.mark.parametrize("mode", ["plain", "o", "rope"])
def test_head_splits_parity(case, mode):
    S, H, KV, d, splits = case
    nbytes, stored = binding.bwd_plan(S, H, KV, d)
    nblk = (S + 31) // 32
    up = lambda n: (n + 255) // 256 * 256
    meta = up(up(up(S * H * 4) + 2 * nblk * 4) + (nblk + 1) * 8)
    tiles = nblk * (nblk + 1) // 2 * H * 8192
    assert stored and nbytes == meta + tiles + 2 * (splits - 1) * S * KV * d * 4
    rng = np.random.default_rng(4400 + S + H)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, "docs"))
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    check_full(p, "head splits x%d %s" % (splits, mode), init=init, with_o=mode == "o",
               rope=(10000.0, 7) if mode == "rope" else None)
