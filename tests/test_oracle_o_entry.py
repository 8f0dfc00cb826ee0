"""Pins of the oracle's forward-output entry points (the _o variants), which
read the row term off the forward output: D = dO . O instead of
sum_j P * dP.  Everything here runs on the CPU.

1. At the exact forward output the two definitions agree: sum_j P_j (dO . v_j)
   = dO . (sum_j P_j v_j) = dO . O.
2. A perturbed O' = O + E changes only the row term, by dD = dO . E, and each
   gradient by a closed form built from independent parts of the oracle:
     dV' = dV,
     dQ' - dQ = -scale * dD_s * sum_j P_sj k_j     (a forward with V := K),
     dK' - dK = -scale * sum_{s,h} P_sj dD_sh q_s  (the dV sum with dO := dD * Q).
3. A row that sees no key has O = 0, so D = 0 and it contributes nothing.
Each planted mistake in the O path makes one of them fail.
"""
import os
import subprocess

import numpy as np
import pytest

from causal_gqa_attention_bwd_amd.workloads import random_problem, seg_from_lengths

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "attn_oracle.c")

CASES = [
    (7, 4, 2, 5, [0, 0, 0, 3, 3, 3, 6]),        # packed documents, GQA 2:1
    (9, 3, 1, 4, [0, 1, 1, 0, 2, 5, 3, 7, 8]),  # arbitrary (non-monotone) starts, MQA
    (6, 2, 2, 3, None),                          # plain causal, MHA
]


def o_pins_fail(oracle):
    failed = set()
    rng = np.random.default_rng(77)
    for S, H, KV, d, seg in CASES:
        p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float64)
        sc = float(p["scale"])
        O, LSE = oracle.attn_fwd_f64(p["Q"], p["K"], p["V"], p["seg"], sc)
        ref = oracle.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"], sc, debug=True)
        got = oracle.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"], sc, debug=True,
                                  O=O)
        # pin 1: same D, same gradients at the exact forward output
        for a, b in zip(got[:4], ref[:4]):
            if np.max(np.abs(a - b)) > 1e-12 * max(np.max(np.abs(b)), 1.0):
                failed.add("identity_at_exact_O")
        # pin 2: closed-form effect of a perturbed O
        E = rng.standard_normal(O.shape)
        dQ2, dK2, dV2, D2, _ = oracle.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"],
                                                   sc, debug=True, O=O + E)
        dD = np.sum(p["dO"] * E, axis=2)                              # [S, H]
        g = H // KV
        pk = oracle.attn_fwd_f64(p["Q"], p["K"], p["K"], p["seg"], sc)[0]  # sum_j P k_j
        want_dQ = got[0] - sc * dD[:, :, None] * pk
        want_dK = got[1] - sc * oracle.attn_bwd_f64(p["Q"], p["K"], p["V"], dD[:, :, None] * p["Q"],
                                                    LSE, p["seg"], sc)[2]
        tol = 1e-11
        if not np.allclose(D2, got[3] + dD, rtol=tol, atol=tol):
            failed.add("perturbed_O_row_term")
        if not (np.allclose(dQ2, want_dQ, rtol=tol, atol=tol)
                and np.allclose(dK2, want_dK, rtol=tol, atol=tol)
                and np.array_equal(dV2, got[2])):
            failed.add("perturbed_O_gradients")
        assert g >= 1
    # pin 3: empty rows (seg[s] > s) have O = 0 and contribute nothing
    S, H, KV, d = 6, 2, 1, 3
    seg = np.array([0, 3, 0, 5, 1, 9], np.uint32)   # rows 1, 3, 5 see no key
    p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float64)
    sc = float(p["scale"])
    O, LSE = oracle.attn_fwd_f64(p["Q"], p["K"], p["V"], seg, sc)
    empty = seg.astype(np.int64) > np.arange(S)
    dQ, dK, dV, D, _ = oracle.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], LSE, seg, sc,
                                           debug=True, O=O)
    if not (np.all(O[empty] == 0) and np.all(D[empty] == 0) and np.all(dQ[empty] == 0)):
        failed.add("empty_rows")
    return sorted(failed)


def test_o_entry_pins_hold(oracle_mod):
    assert o_pins_fail(oracle_mod) == []


def test_float_o_entry_matches_f64(oracle_mod):
    # the fp32 entry widens, runs the same fp64 backward, and adds into its outputs
    rng = np.random.default_rng(78)
    p = random_problem(rng, 40, 4, 2, 8, seg=seg_from_lengths([13, 20, 7], 40))
    sc = p["scale"]
    O, LSE = oracle_mod.attn_fwd(p["Q"], p["K"], p["V"], p["seg"], sc)
    init = [rng.standard_normal(x.shape).astype(np.float32) for x in (p["Q"], p["K"], p["V"])]
    got = oracle_mod.attn_bwd(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"], sc, *init, O=O)
    ref = oracle_mod.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"], sc, O=O)
    for a, i0, b in zip(got, init, ref):
        assert np.array_equal(a, (i0.astype(np.float64) + b).astype(np.float32))
    # selected rows agree with the full backward
    q_rows, k_rows = np.array([0, 12, 13, 39], np.int32), np.array([0, 13, 32, 39], np.int32)
    rq, rk, rv = oracle_mod.attn_bwd_rows(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"], sc,
                                          q_rows, k_rows, O=O)
    assert np.allclose(rq, ref[0][q_rows], rtol=1e-12, atol=1e-14)
    assert np.allclose(rk, ref[1][k_rows], rtol=1e-12, atol=1e-14)
    assert np.allclose(rv, ref[2][k_rows], rtol=1e-12, atol=1e-14)


O_MUTANTS = {
    "none": [],
    "D_reads_O_twice": [("if (p->O) D = dot(q_row(p, p->dO, s, h), q_row(p, p->O, s, h), p->d);",
                         "if (p->O) D = dot(q_row(p, p->O, s, h), q_row(p, p->O, s, h), p->d);")],
    "O_ignored": [("if (p->O) D = dot(", "if (0) D = dot(")],
    "O_wrong_head": [("q_row(p, p->O, s, h), p->d);", "q_row(p, p->O, s, 0), p->d);")],
    "D_sign": [("if (p->O) D = dot(q_row(p, p->dO, s, h), q_row(p, p->O, s, h), p->d);",
                "if (p->O) D = -dot(q_row(p, p->dO, s, h), q_row(p, p->O, s, h), p->d);")],
}


@pytest.mark.parametrize("name", list(O_MUTANTS))
def test_o_pins_catch_planted_mistake(oracle_mod, tmp_path, name):
    src = open(SRC).read()
    for old, new in O_MUTANTS[name]:
        assert old in src, f"mutation site vanished: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / f"o_{name}.c"
    so = tmp_path / f"o_{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(so), str(c),
                    "-lm"], check=True)
    with oracle_mod._use_library(str(so)):
        failed = o_pins_fail(oracle_mod)
    if name == "none":
        assert failed == [], failed
    else:
        assert failed, f"no pin caught mutant {name}"
