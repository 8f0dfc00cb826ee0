"""Pins of the oracle's RoPE backward (page "llm.istanbul --
10_backward_attention.wgsl", kernels rope_q_backward / rope_k_backward) and of
the backward composed with it.  Everything here runs on the CPU.

1. Finite differences: with q = R q0 and k = R k0 rotated by the forward
   rotation, the gradients of L = sum O * dO with respect to q0 and k0 are
   the attention backward's dQ, dK rotated back.
2. Relative positions: the scores depend only on key minus query position,
   so those gradients do not change when pos_offset shifts every position.
3. The angle ladder: pair 0 turns by exactly the position (base^0 = 1) for any
   base, each further pair's angle is base^(-2/d) times the previous one, and
   the angle depends on the position and pos_offset only through their sum.
4. The rotation is orthogonal: backward(forward(x)) = x and pair norms hold.
Each planted mistake makes one of them fail.
"""
import os
import subprocess

import numpy as np
import pytest

from causal_gqa_attention_bwd_amd.workloads import random_problem

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "attn_oracle.c")


def loss(oracle, q0, k0, V, dO, seg, scale, base, off):
    q = oracle.rope_f64(q0, base, off, backward=False)
    k = oracle.rope_f64(k0, base, off, backward=False)
    return float(np.sum(oracle.attn_fwd_f64(q, k, V, seg, scale)[0] * dO))


def grads(oracle, q0, k0, V, dO, seg, scale, base, off):
    q = oracle.rope_f64(q0, base, off, backward=False)
    k = oracle.rope_f64(k0, base, off, backward=False)
    _, LSE = oracle.attn_fwd_f64(q, k, V, seg, scale)
    dQ, dK, dV = oracle.attn_bwd_f64(q, k, V, dO, LSE, seg, scale)
    return (oracle.rope_f64(dQ, base, off, backward=True),
            oracle.rope_f64(dK, base, off, backward=True), dV)


def rope_pins_fail(oracle):
    failed = set()
    rng = np.random.default_rng(91)
    # 1. finite differences through the rotated forward
    p = random_problem(rng, 5, 2, 1, 4, seg=[0, 0, 0, 3, 3], dtype=np.float64)
    sc, base, off = float(p["scale"]), 100.0, 3
    gq, gk, _ = grads(oracle, p["Q"], p["K"], p["V"], p["dO"], p["seg"], sc, base, off)
    h = 1e-6
    for X, G in ((p["Q"], gq), (p["K"], gk)):
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            keep = X[idx]
            X[idx] = keep + h
            lp = loss(oracle, p["Q"], p["K"], p["V"], p["dO"], p["seg"], sc, base, off)
            X[idx] = keep - h
            lm = loss(oracle, p["Q"], p["K"], p["V"], p["dO"], p["seg"], sc, base, off)
            X[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        if np.max(np.abs(fd - G)) > 1e-6 * max(np.max(np.abs(G)), 1e-3):
            failed.add("finite_differences")
    # 2. invariance under a shift of every position
    p = random_problem(rng, 12, 4, 2, 8, seg=[0] * 5 + [5] * 7, dtype=np.float64)
    sc = float(p["scale"])
    a = grads(oracle, p["Q"], p["K"], p["V"], p["dO"], p["seg"], sc, 1000.0, 0)
    b = grads(oracle, p["Q"], p["K"], p["V"], p["dO"], p["seg"], sc, 1000.0, 37)
    if not all(np.allclose(x, y, rtol=1e-9, atol=1e-12) for x, y in zip(a, b)):
        failed.add("offset_invariance")
    # 3. the angle ladder, read off rotations of the unit vector (1, 0)
    d, base = 8, 500.0
    for t, off in ((0, 5), (3, 4), (1, 0)):
        e = np.zeros((t + 1, 1, d))
        e[t, 0, 0::2] = 1.0
        r = oracle.rope_f64(e, base, off, backward=False)[t, 0]
        ang = np.arctan2(r[1::2], r[0::2])
        want = (t + off) * base ** (-2.0 * np.arange(d // 2) / d)
        if not np.allclose(np.cos(ang), np.cos(want), atol=1e-12) or \
           not np.allclose(np.sin(ang), np.sin(want), atol=1e-12):
            failed.add("angle_ladder")
    # 4. orthogonality
    x = rng.standard_normal((6, 3, 8))
    y = oracle.rope_f64(x, 10000.0, 11, backward=False)
    if not np.allclose(oracle.rope_f64(y, 10000.0, 11, backward=True), x, atol=1e-12) or \
       not np.allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.hypot(x[..., 0::2], x[..., 1::2]),
                       atol=1e-12):
        failed.add("orthogonal")
    return sorted(failed)


def test_rope_pins_hold(oracle_mod):
    assert rope_pins_fail(oracle_mod) == []


def test_float_rope_entry_composes(oracle_mod):
    # the fp32 entry = round(R^T(init + gradient)) for dQ and dK, dV untouched by RoPE
    rng = np.random.default_rng(92)
    p = random_problem(rng, 30, 4, 2, 16, seg=[0] * 12 + [12] * 18)
    sc, base, off = p["scale"], 10000.0, 7
    O, LSE = oracle_mod.attn_fwd(p["Q"], p["K"], p["V"], p["seg"], sc)
    init = [rng.standard_normal(x.shape).astype(np.float32) for x in (p["Q"], p["K"], p["V"])]
    for o in (None, O):
        got = oracle_mod.attn_bwd(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"], sc, *init, O=o,
                                  rope=(base, off))
        g = oracle_mod.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"], sc, O=o)
        wq = oracle_mod.rope_f64(init[0].astype(np.float64) + g[0], base, off, backward=True)
        wk = oracle_mod.rope_f64(init[1].astype(np.float64) + g[1], base, off, backward=True)
        assert np.array_equal(got[0], wq.astype(np.float32))
        assert np.array_equal(got[1], wk.astype(np.float32))
        assert np.array_equal(got[2], (init[2].astype(np.float64) + g[2]).astype(np.float32))


ROPE_MUTANTS = {
    "none": [],
    "backward_not_transposed": [("x[0] = x0 * c + x1 * sn;\n          x[1] = -x0 * sn + x1 * c;",
                                 "x[0] = x0 * c - x1 * sn;\n          x[1] = x0 * sn + x1 * c;")],
    "freq_p_over_d": [("double freq = pow(base, -2.0 * pr / (double)d);",
                       "double freq = pow(base, -1.0 * pr / (double)d);")],
    "ignores_pos_offset": [("double ang = (double)(t + pos_offset) * freq;",
                            "double ang = (double)t * freq;")],
    "pairs_shifted": [("double freq = pow(base, -2.0 * pr / (double)d);",
                       "double freq = pow(base, -2.0 * (pr + 1) / (double)d);")],
}


@pytest.mark.parametrize("name", list(ROPE_MUTANTS))
def test_rope_pins_catch_planted_mistake(oracle_mod, tmp_path, name):
    src = open(SRC).read()
    for old, new in ROPE_MUTANTS[name]:
        assert old in src, f"mutation site vanished: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / f"r_{name}.c"
    so = tmp_path / f"r_{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(so), str(c),
                    "-lm"], check=True)
    with oracle_mod._use_library(str(so)):
        failed = rope_pins_fail(oracle_mod)
    if name == "none":
        assert failed == [], failed
    else:
        assert failed, f"no pin caught mutant {name}"
