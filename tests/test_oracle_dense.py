"""Pins 4-6 of the oracle against an independent dense implementation.

The reference here is torch CPU float64 autograd of masked softmax attention,
per head, the textbook algorithm that page "tang 0.2.0 -- src/gpu/llm.rs"
(GpuCausalAttention::backward) writes out for plain causal attention: softmax
of scaled scores, grad_attn = dO.V^T, dV += P^T.dO, grad_scores =
P*(grad_attn - rowsum(grad_attn*P))*scale, dQ = grad_scores.K,
dK = grad_scores^T.Q.  The library routines (softmax, matmul, autograd) share
nothing with the oracle's C code.
"""
import numpy as np
import pytest
import torch

from causal_gqa_attention_bwd_amd.workloads import random_problem, seg_from_lengths


def torch_dense(p):
    Q = torch.tensor(p["Q"], dtype=torch.float64, requires_grad=True)
    K = torch.tensor(p["K"], dtype=torch.float64, requires_grad=True)
    V = torch.tensor(p["V"], dtype=torch.float64, requires_grad=True)
    dO = torch.tensor(p["dO"], dtype=torch.float64)
    S, H, d = Q.shape
    KV = K.shape[1]
    g = H // KV
    seg = torch.tensor(np.asarray(p["seg"], np.int64))
    s_idx = torch.arange(S)[:, None]
    j_idx = torch.arange(S)[None, :]
    visible = (j_idx <= s_idx) & (j_idx >= seg[:, None])
    outs, lses = [], []
    for h in range(H):
        logits = float(p["scale"]) * (Q[:, h, :] @ K[:, h // g, :].T)
        logits = logits.masked_fill(~visible, float("-inf"))
        lses.append(torch.logsumexp(logits, dim=1))
        outs.append(torch.softmax(logits, dim=1) @ V[:, h // g, :])
    O = torch.stack(outs, dim=1)
    (O * dO).sum().backward()
    return (O.detach().numpy(), torch.stack(lses, 1).detach().numpy(),
            Q.grad.numpy(), K.grad.numpy(), V.grad.numpy())


def oracle_all(oracle, p):
    O, LSE = oracle.attn_fwd_f64(p["Q"], p["K"], p["V"], p["seg"], float(p["scale"]))
    return (O, LSE) + oracle.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], LSE, p["seg"],
                                          float(p["scale"]))


SHAPES = [(48, 4, 2, 16), (33, 3, 1, 7), (64, 8, 8, 32), (40, 8, 2, 24)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "S%dH%dKV%dd%d" % s)
@pytest.mark.parametrize("seg_kind", ["causal", "docs"])
def test_oracle_equals_torch_dense(oracle_mod, shape, seg_kind):
    S, H, KV, d = shape
    rng = np.random.default_rng(100 + S + d)
    seg = None if seg_kind == "causal" else seg_from_lengths([S // 3, 1, S // 2], S)
    p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float64)
    got = oracle_all(oracle_mod, p)
    want = torch_dense(p)
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), got, want):
        assert np.allclose(a, b, rtol=1e-11, atol=1e-12), (name, np.max(np.abs(a - b)))


def test_packed_equals_per_document(oracle_mod):
    rng = np.random.default_rng(21)
    lengths = [13, 1, 27, 9, 14]
    S, H, KV, d = sum(lengths), 4, 2, 12
    seg = seg_from_lengths(lengths, S)
    p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float64)
    _, _, dQ, dK, dV = oracle_all(oracle_mod, p)
    start = 0
    for L in lengths:
        sl = slice(start, start + L)
        sub = {k: (v[sl] if isinstance(v, np.ndarray) and v.ndim == 3 else v) for k, v in p.items()}
        sub["seg"] = None
        _, _, q1, k1, v1 = oracle_all(oracle_mod, sub)
        assert np.allclose(dQ[sl], q1, rtol=1e-12, atol=1e-14)
        assert np.allclose(dK[sl], k1, rtol=1e-12, atol=1e-14)
        assert np.allclose(dV[sl], v1, rtol=1e-12, atol=1e-14)
        start += L


def test_gqa_equals_replicated_mha(oracle_mod):
    rng = np.random.default_rng(22)
    S, H, KV, d = 37, 6, 2, 10
    g = H // KV
    seg = seg_from_lengths([12, 25], S)
    p = random_problem(rng, S, H, KV, d, seg=seg, dtype=np.float64)
    _, _, dQ, dK, dV = oracle_all(oracle_mod, p)
    rep = dict(p)
    rep["K"] = np.repeat(p["K"], g, axis=1)     # head h reads KV head h // g
    rep["V"] = np.repeat(p["V"], g, axis=1)
    _, _, q2, k2, v2 = oracle_all(oracle_mod, rep)
    assert np.allclose(dQ, q2, rtol=1e-12, atol=1e-14)
    assert np.allclose(dK, k2.reshape(S, KV, g, d).sum(axis=2), rtol=1e-12, atol=1e-13)
    assert np.allclose(dV, v2.reshape(S, KV, g, d).sum(axis=2), rtol=1e-12, atol=1e-13)
