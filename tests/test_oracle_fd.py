"""Pin 1: the oracle's backward equals fp64 central finite differences of
L(Q, K, V) = sum(O * dO), with the forward (and its LSE) recomputed at every
perturbed point.  Method after page "tang 0.2.0 -- src/gpu/llm.rs", test
helper finite_diff_cpu and attention_backward_gradient_check (central
differences of a scalar loss through attention), done here in fp64."""
import numpy as np
import pytest

from causal_gqa_attention_bwd_amd.workloads import random_problem

CASES = [
    # (S, H, KV, d, seg)
    (6, 4, 2, 4, [0, 0, 0, 3, 3, 3]),          # two packed documents, GQA 2:1
    (5, 2, 1, 3, None),                         # plain causal, one KV head
    (2, 2, 1, 2, None),                         # the gradient-check shape of the tang page
    (7, 3, 3, 5, [0, 0, 1, 0, 2, 3, 6]),        # arbitrary (non-monotone) document starts
    (5, 2, 2, 4, [0, 0, 5, 1, 1]),              # row 2 sees no key (seg > s)
]


def loss(oracle, p, Q, K, V):
    O, _ = oracle.attn_fwd_f64(Q, K, V, p["seg"], float(p["scale"]), nthreads=1)
    return float(np.sum(O * p["dO"]))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{c[0]}H{c[1]}KV{c[2]}d{c[3]}")
def test_oracle_matches_finite_differences(oracle_mod, case):
    S, H, KV, d, seg = case
    rng = np.random.default_rng(7 + S * 31 + d)
    p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float64)
    Q, K, V, dO = p["Q"], p["K"], p["V"], p["dO"]
    _, LSE = oracle_mod.attn_fwd_f64(Q, K, V, p["seg"], float(p["scale"]))
    dQ, dK, dV = oracle_mod.attn_bwd_f64(Q, K, V, dO, LSE, p["seg"], float(p["scale"]))
    h = 1e-6
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            keep = X[idx]
            X[idx] = keep + h
            lp = loss(oracle_mod, p, Q, K, V)
            X[idx] = keep - h
            lm = loss(oracle_mod, p, Q, K, V)
            X[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        scale_ref = max(np.max(np.abs(G)), 1e-3)
        err = np.max(np.abs(fd - G))
        assert err <= 1e-6 * scale_ref, f"d{name}: max|fd-analytic|={err:.3e} vs max|grad|={scale_ref:.3e}"
