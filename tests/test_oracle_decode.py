"""Pins of the oracle's single-query backward over a KV history (page "rullama
0.5.0 -- src/backend/dispatch/training.rs", attention_backward_dq_chained and
attention_backward_dkv_chained: stored probabilities, pass 1 writes dq and the
score gradients, pass 2 the key-major dK and dV).  CPU only.

1. Finite differences: with P = softmax(scale q.k) over the history (computed
   here in numpy), the gradients of L = sum_h dO_h . (sum_j P_hj v_j) with
   respect to q, K and V are the oracle's dq, dK, dV.
2. Agreement with the main backward (itself pinned in test_oracle_fd.py,
   test_oracle_invariants.py, test_oracle_dense.py and test_oracle_golden.py): a
   plain causal problem whose dO is zero except on its last row s* gives, in
   the main oracle, dK and dV equal to the decode backward's for the query
   q = Q[s*] with P from the same LSE, dQ[s*] equal to its dq, and dQ = 0
   on every other row.
3. T = 1: the only key has P = 1, so dS = 0: dq = dK = 0 and dV = the sum of
   dO over the group's heads.
4. History sums: each row of P sums to one, so sum_j dS_j = 0 and the keys'
   dK sum to zero, while the keys' dV sum to the group's sum of dO.
Each planted mistake makes one of them fail.
"""
import os
import subprocess

import numpy as np
import pytest

from causal_gqa_attention_bwd_amd.workloads import random_problem

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "attn_oracle.c")


def softmax_probs(q, K, scale):
    """P[h, j] = softmax_j(scale * q_h . k_j) with kv head h // (H // KV)."""
    H = q.shape[0]
    g = H // K.shape[1]
    x = np.stack([scale * K[:, h // g, :] @ q[h] for h in range(H)])  # [H, T]
    x -= x.max(axis=1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=1, keepdims=True)


def decode_loss(q, K, V, dO, scale):
    P = softmax_probs(q, K, scale)
    g = q.shape[0] // K.shape[1]
    return sum(float(dO[h] @ (P[h] @ V[:, h // g, :])) for h in range(q.shape[0]))


def decode_pins_fail(oracle):
    failed = set()
    rng = np.random.default_rng(61)
    # 1. finite differences
    T, H, KV, d, sc = 5, 4, 2, 3, 0.7
    q, dO = rng.standard_normal((H, d)), rng.standard_normal((H, d))
    K, V = rng.standard_normal((T, KV, d)), rng.standard_normal((T, KV, d))
    got = oracle.attn_bwd_decode_f64(q, K, V, softmax_probs(q, K, sc), dO, sc)
    eps = 1e-6
    for X, G in ((q, got[0]), (K, got[1]), (V, got[2])):
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            keep = X[idx]
            X[idx] = keep + eps
            lp = decode_loss(q, K, V, dO, sc)
            X[idx] = keep - eps
            lm = decode_loss(q, K, V, dO, sc)
            X[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        if np.max(np.abs(fd - G)) > 1e-6 * max(np.max(np.abs(G)), 1e-3):
            failed.add("finite_differences")
    # 2. the last row of a causal problem through the main backward
    S, H, KV, d = 9, 4, 2, 5
    p = random_problem(rng, S, H, KV, d, dtype=np.float64)
    sc = float(p["scale"])
    dO = np.zeros_like(p["dO"])
    dO[S - 1] = p["dO"][S - 1]
    _, LSE = oracle.attn_fwd_f64(p["Q"], p["K"], p["V"], None, sc)
    mq, mk, mv = oracle.attn_bwd_f64(p["Q"], p["K"], p["V"], dO, LSE, None, sc)
    q = p["Q"][S - 1]
    g = H // KV
    P = np.exp(np.stack([sc * p["K"][:, h // g, :] @ q[h] for h in range(H)])
               - LSE[S - 1][:, None])
    dq, dk, dv = oracle.attn_bwd_decode_f64(q, p["K"], p["V"], P, dO[S - 1], sc)
    tol = 1e-12 * max(np.max(np.abs(mk)), np.max(np.abs(mv)), 1.0)
    if not (np.max(np.abs(mk - dk)) <= tol and np.max(np.abs(mv - dv)) <= tol
            and np.max(np.abs(mq[S - 1] - dq)) <= tol and not np.any(mq[:S - 1])):
        failed.add("last_row_of_causal")
    # 3. a history of one key
    H, KV, d = 6, 3, 4
    q, dO = rng.standard_normal((H, d)), rng.standard_normal((H, d))
    K, V = rng.standard_normal((1, KV, d)), rng.standard_normal((1, KV, d))
    dq, dk, dv = oracle.attn_bwd_decode_f64(q, K, V, np.ones((H, 1)), dO, 0.3)
    want_v = dO.reshape(KV, H // KV, d).sum(axis=1)
    if np.any(dq) or np.any(dk) or not np.allclose(dv[0], want_v, rtol=1e-14, atol=1e-14):
        failed.add("single_key")
    # 4. history sums
    T, H, KV, d, sc = 40, 8, 2, 6, 0.4
    q, dO = rng.standard_normal((H, d)), rng.standard_normal((H, d))
    K, V = rng.standard_normal((T, KV, d)), rng.standard_normal((T, KV, d))
    dq, dk, dv = oracle.attn_bwd_decode_f64(q, K, V, softmax_probs(q, K, sc), dO, sc)
    if np.max(np.abs(dk.sum(axis=0))) > 1e-12 * np.abs(dk).sum(axis=0).max():
        failed.add("dK_sums_to_zero")
    if not np.allclose(dv.sum(axis=0), dO.reshape(KV, H // KV, d).sum(axis=1), rtol=1e-12,
                       atol=1e-12):
        failed.add("dV_sums_to_dO")
    return sorted(failed)


def test_decode_pins_hold(oracle_mod):
    assert decode_pins_fail(oracle_mod) == []


def test_float_decode_entry_adds_and_rounds_once(oracle_mod):
    rng = np.random.default_rng(62)
    T, H, KV, d, sc = 33, 4, 2, 8, np.float32(0.35)
    q, dO = (rng.standard_normal((H, d)).astype(np.float32) for _ in range(2))
    K, V = (rng.standard_normal((T, KV, d)).astype(np.float32) for _ in range(2))
    P = softmax_probs(q.astype(np.float64), K.astype(np.float64), float(sc)).astype(np.float32)
    init = [rng.standard_normal(s).astype(np.float32) for s in ((H, d), (T, KV, d), (T, KV, d))]
    got = oracle_mod.attn_bwd_decode(q, K, V, P, dO, sc, *init)
    ref = oracle_mod.attn_bwd_decode_f64(q, K, V, P, dO, float(sc))
    for a, i0, b in zip(got, init, ref):
        assert np.array_equal(a, (i0.astype(np.float64) + b).astype(np.float32))


DECODE_MUTANTS = {
    "none": [],
    "D_sign": [("ds[k] = P[k] * (ds[k] - D);", "ds[k] = P[k] * (ds[k] + D);")],
    "dK_without_scale": [("const double wk = scale * ds[(size_t)h * T + j], wv",
                          "const double wk = ds[(size_t)h * T + j], wv")],
    "dV_from_dS": [("wv = P[(size_t)h * T + j];", "wv = ds[(size_t)h * T + j];")],
    "kv_head_modulo": [("    const int kvh = h / g;\n    const double *doh",
                        "    const int kvh = h % KV;\n    const double *doh")],
    "dq_from_v": [("const double *kj = K + ((size_t)j * KV + kvh) * d;",
                   "const double *kj = V + ((size_t)j * KV + kvh) * d;")],
}


@pytest.mark.parametrize("name", list(DECODE_MUTANTS))
def test_decode_pins_catch_planted_mistake(oracle_mod, tmp_path, name):
    src = open(SRC).read()
    for old, new in DECODE_MUTANTS[name]:
        assert old in src, f"mutation site vanished: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / f"dec_{name}.c"
    so = tmp_path / f"dec_{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(so), str(c),
                    "-lm"], check=True)
    with oracle_mod._use_library(str(so)):
        failed = decode_pins_fail(oracle_mod)
    if name == "none":
        assert failed == [], failed
    else:
        assert failed, f"no pin caught mutant {name}"
