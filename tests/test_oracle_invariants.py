"""Pins 2, 3, 7, 8 of the oracle: properties the mathematics fixes.

- sum_j dS[s,h,j] = 0 for every row (debug hook of the oracle), and its
  output-level consequences per document and KV head: sum_j dK_j = 0 and
  sum_j dV_j = sum of dO over the document's queries and the group's heads.
- zero gradient on masked keys (page "llm.istanbul -- 10_backward_attention.wgsl",
  kernel attention_backward: keys before the document start or after the query
  give P = dP = 0).
- closed forms: S = 1, Q = 0, forward at S = 1 and at position 0 (cf. page
  "tang 0.2.0 -- src/gpu/llm.rs", tests causal_attention_identity_kv and
  causal_attention_mask_works).
- linearity in dO and the "+=" output contract (header comment of the wgsl page).
"""
import numpy as np
import pytest

from causal_gqa_attention_bwd_amd.workloads import random_problem, seg_from_lengths


def f64_grads(oracle, p, debug=False):
    _, LSE = oracle.attn_fwd_f64(p["Q"], p["K"], p["V"], p["seg"], float(p["scale"]))
    return oracle.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"], float(p["scale"]),
                               debug=debug)


@pytest.mark.parametrize("seg_kind", ["causal", "docs", "arbitrary"])
def test_row_sum_of_dS_is_zero(oracle_mod, seg_kind):
    rng = np.random.default_rng(11)
    S = 96
    seg = {"causal": None,
           "docs": seg_from_lengths([17, 40, 3, 36], S),
           "arbitrary": np.minimum(rng.integers(0, S, S), np.arange(S))}[seg_kind]
    p = random_problem(rng, S, 4, 2, 16, seg=seg, dtype=np.float64)
    dQ, dK, dV, D, rs = f64_grads(oracle_mod, p, debug=True)
    assert np.max(np.abs(D)) > 1e-3          # D is not trivially zero
    assert np.max(np.abs(rs)) <= 1e-12, np.max(np.abs(rs))


def test_document_sums_of_dK_dV(oracle_mod):
    rng = np.random.default_rng(12)
    S, H, KV, d = 120, 6, 2, 8
    lengths = [31, 1, 50, 38]
    seg = seg_from_lengths(lengths, S)
    p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float64)
    dQ, dK, dV = f64_grads(oracle_mod, p)
    g = H // KV
    start = 0
    for L in lengths:
        doc = slice(start, start + L)
        for kv in range(KV):
            sk = dK[doc, kv].sum(axis=0)
            sv = dV[doc, kv].sum(axis=0)
            want_v = p["dO"][doc, kv * g:(kv + 1) * g].sum(axis=(0, 1))
            assert np.max(np.abs(sk)) <= 1e-10 * max(1.0, np.abs(dK[doc, kv]).sum())
            assert np.max(np.abs(sv - want_v)) <= 1e-10 * max(1.0, np.abs(p["dO"][doc]).sum())
        start += L


def test_masked_keys_get_zero_gradient(oracle_mod):
    rng = np.random.default_rng(13)
    S, H, KV, d = 40, 4, 2, 8
    seg = seg_from_lengths([9, 14, 17], S)
    p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float32)
    s_star = 18                              # inside the second document [9, 23)
    dO = np.zeros_like(p["dO"])
    dO[s_star] = p["dO"][s_star]
    _, LSE = oracle_mod.attn_fwd(p["Q"], p["K"], p["V"], seg, p["scale"])
    dQ, dK, dV = oracle_mod.attn_bwd(p["Q"], p["K"], p["V"], dO, LSE, seg, p["scale"])
    lo, hi = int(seg[s_star]), s_star
    outside = np.r_[0:lo, hi + 1:S]
    assert np.all(dK[outside] == 0) and np.all(dV[outside] == 0)
    assert np.any(dK[lo:hi + 1] != 0) and np.any(dV[lo:hi + 1] != 0)
    assert np.all(dQ[np.r_[0:s_star, s_star + 1:S]] == 0)
    # changing keys/values the query cannot see leaves its dQ bitwise unchanged
    K2, V2 = p["K"].copy(), p["V"].copy()
    K2[outside] = 1e3 * rng.standard_normal(K2[outside].shape)
    V2[outside] = -7.0
    dQ2, _, _ = oracle_mod.attn_bwd(p["Q"], K2, V2, dO, LSE, seg, p["scale"])
    assert np.array_equal(dQ2[s_star], dQ[s_star])


def test_closed_form_single_token(oracle_mod):
    rng = np.random.default_rng(14)
    H, KV, d = 6, 3, 5
    p = random_problem(rng, 1, H, KV, d, dtype=np.float64)
    O, LSE = oracle_mod.attn_fwd_f64(p["Q"], p["K"], p["V"], None, float(p["scale"]))
    g = H // KV
    for h in range(H):
        kv = h // g
        assert np.allclose(O[0, h], p["V"][0, kv], rtol=0, atol=1e-15)
        assert abs(LSE[0, h] - float(p["scale"]) * p["Q"][0, h] @ p["K"][0, kv]) <= 1e-14
    dQ, dK, dV = oracle_mod.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], LSE, None,
                                         float(p["scale"]))
    assert np.all(dQ == 0) and np.all(dK == 0)
    want = p["dO"][0].reshape(KV, g, d).sum(axis=1)
    assert np.allclose(dV[0], want, rtol=0, atol=1e-14)


def test_closed_form_first_position_sees_itself(oracle_mod):
    rng = np.random.default_rng(15)
    p = random_problem(rng, 9, 4, 1, 6, dtype=np.float64)
    O, _ = oracle_mod.attn_fwd_f64(p["Q"], p["K"], p["V"], None, float(p["scale"]))
    for h in range(4):
        assert np.allclose(O[0, h], p["V"][0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("seg_kind", ["causal", "docs"])
def test_closed_form_zero_queries(oracle_mod, seg_kind):
    rng = np.random.default_rng(16)
    S, H, KV, d = 33, 4, 2, 6
    seg = None if seg_kind == "causal" else seg_from_lengths([5, 20, 8], S)
    p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float64)
    p["Q"][:] = 0.0
    dQ, dK, dV = f64_grads(oracle_mod, p)
    assert np.all(dK == 0)
    segv = np.zeros(S, int) if seg is None else np.asarray(seg, int)
    n = np.arange(S) - segv + 1                  # keys each query sees
    g = H // KV
    want = np.zeros((S, KV, d))
    for j in range(S):
        for s in range(j, S):
            if segv[s] <= j:
                want[j] += p["dO"][s].reshape(KV, g, d).sum(axis=1) / n[s]
    assert np.allclose(dV, want, rtol=0, atol=1e-13)


def test_linearity_and_accumulation(oracle_mod):
    rng = np.random.default_rng(17)
    S, H, KV, d = 50, 4, 2, 8
    seg = seg_from_lengths([20, 30], S)
    p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float64)
    _, LSE = oracle_mod.attn_fwd_f64(p["Q"], p["K"], p["V"], seg, float(p["scale"]))
    args = (p["Q"], p["K"], p["V"])
    g1 = oracle_mod.attn_bwd_f64(*args, p["dO"], LSE, seg, float(p["scale"]))
    g3 = oracle_mod.attn_bwd_f64(*args, -2.5 * p["dO"], LSE, seg, float(p["scale"]))
    for a, b in zip(g1, g3):
        assert np.allclose(b, -2.5 * a, rtol=1e-13, atol=1e-15)
    # "+=" contract of the fp32 entry point: out(init) - init == out(0) up to fp32 rounding
    p32 = {k: (v.astype(np.float32) if isinstance(v, np.ndarray) and v.dtype == np.float64 else v)
           for k, v in p.items()}
    _, L32 = oracle_mod.attn_fwd(p32["Q"], p32["K"], p32["V"], seg, p32["scale"])
    zero = oracle_mod.attn_bwd(p32["Q"], p32["K"], p32["V"], p32["dO"], L32, seg, p32["scale"])
    init = [rng.standard_normal(z.shape).astype(np.float32) for z in zero]
    acc = oracle_mod.attn_bwd(p32["Q"], p32["K"], p32["V"], p32["dO"], L32, seg, p32["scale"],
                              dQ=init[0], dK=init[1], dV=init[2])
    for z, i0, a in zip(zero, init, acc):
        assert np.allclose(a.astype(np.float64) - i0, z, rtol=0,
                           atol=2 * np.finfo(np.float32).eps * (np.abs(i0).max() + np.abs(z).max()))


def test_deterministic_across_thread_counts(oracle_mod):
    rng = np.random.default_rng(18)
    p = random_problem(rng, 70, 4, 2, 8, seg=seg_from_lengths([30, 40], 70))
    _, L = oracle_mod.attn_fwd(p["Q"], p["K"], p["V"], p["seg"], p["scale"])
    a = oracle_mod.attn_bwd(p["Q"], p["K"], p["V"], p["dO"], L, p["seg"], p["scale"], nthreads=1)
    b = oracle_mod.attn_bwd(p["Q"], p["K"], p["V"], p["dO"], L, p["seg"], p["scale"], nthreads=7)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_selected_rows_equal_full_backward(oracle_mod):
    rng = np.random.default_rng(19)
    S, H, KV, d = 64, 4, 2, 8
    seg = seg_from_lengths([10, 30, 24], S)
    p = random_problem(rng, S, H, KV, d, seg=seg)
    _, L = oracle_mod.attn_fwd(p["Q"], p["K"], p["V"], seg, p["scale"])
    full = oracle_mod.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], L, seg, float(p["scale"]))
    qr, kr = [0, 9, 10, 40, 63], [0, 5, 10, 39, 63]
    dq, dk, dv = oracle_mod.attn_bwd_rows(p["Q"], p["K"], p["V"], p["dO"], L, seg, p["scale"], qr, kr)
    assert np.array_equal(dq, full[0][qr])
    assert np.array_equal(dk, full[1][kr])
    assert np.array_equal(dv, full[2][kr])


def test_selected_forward_rows_equal_full_forward(oracle_mod):
    rng = np.random.default_rng(20)
    S, H, KV, d = 50, 4, 2, 8
    seg = seg_from_lengths([10, 3, 37], S)
    p = random_problem(rng, S, H, KV, d, seg=seg)
    O, L = oracle_mod.attn_fwd(p["Q"], p["K"], p["V"], seg, p["scale"])
    rows = [0, 9, 12, 13, 49]
    Os, Ls = oracle_mod.attn_fwd_rows(p["Q"], p["K"], p["V"], seg, p["scale"], rows, want_o=True)
    assert np.array_equal(Ls, L[rows]) and np.array_equal(Os, O[rows])
    need = oracle_mod.rows_needed(seg, S, [5], [11])
    assert list(need) == [5] + list(range(11, 13))   # key 11 lives in the doc [10, 13)
