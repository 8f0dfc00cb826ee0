"""The HIP path against the hand-worked examples of tests/golden/, through the
C ABI: expected values derived on paper from the definitions of page
"llm.istanbul -- 10_backward_attention.wgsl" (header comment and kernel
attention_backward), not from the oracle.

The fixtures have head_dim 1; the inputs are zero-padded to 16 columns, which
changes no dot product, so the padded gradients are the fixture's in column 0
and zero elsewhere.  Bounds, per tensor, relative to max|expected|: 2e-5 for
the fp32 entries (a few fp32 roundings of ln 3, exp and the sums), 2e-2 for
attn_bwd_f16 (fp16 operands: 2 ln 3 and the probabilities each carry up to
5e-4 of rounding).

The single-query entry (page "rullama 0.5.0", KV-history backward) takes row 1
of the fixture as its query, keys 0 and 1 as its history and that row's
probabilities exp(scale*q.k - LSE) as P; its gradients are row 1's part of the
hand derivation.
"""
import numpy as np
import pytest
import torch

from causal_gqa_attention_bwd_amd import binding
from tests.gpu_helpers import dev, gpu_bwd, gpu_fwd, to_dev
from tests.golden_io import golden_files, load_golden, pad_head_dim

pytestmark = pytest.mark.gpu

FILES = golden_files()
TOL32 = 2e-5
TOL16 = 2e-2


def check(got, want, tol, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    inf = np.isinf(want)                           # LSE of a row that sees no key
    assert np.array_equal(got[inf], want[inf]), f"{what}: infinite entries differ"
    got, want = got[~inf], want[~inf]
    err = float(np.max(np.abs(got - want)))
    assert err <= tol * max(float(np.max(np.abs(want))), 1e-30), f"{what}: max err {err:.3e}"


def problem(path):
    g = pad_head_dim(load_golden(path), 16)
    p = {k: g[k].astype(np.float32) for k in ("Q", "K", "V", "dO")}
    p["seg"], p["scale"] = g["seg"], g["scale"]
    return g, p


@pytest.mark.parametrize("entry", ["attn_bwd", "attn_bwd_o", "attn_bwd_short",
                                   "attn_bwd_short_o", "attn_bwd_f16", "attn_bwd_f16_o"])
@pytest.mark.parametrize("path", FILES, ids=lambda p: p.rsplit("/", 1)[-1])
def test_backward_matches_hand_worked(path, entry):
    print(f"golden {path.rsplit('/', 1)[-1]} through {entry}", flush=True)
    g, p = problem(path)
    O = g["O"] if entry.endswith("_o") else None
    out = gpu_bwd(p, g["LSE"], O=O, short="short" in entry, f16="f16" in entry)
    tol = TOL16 if "f16" in entry else TOL32
    for name, got in zip(("dQ", "dK", "dV"), out):
        check(got, g[name], tol, f"{entry} {name}")


@pytest.mark.parametrize("path", FILES, ids=lambda p: p.rsplit("/", 1)[-1])
def test_forward_matches_hand_worked(path):
    print(f"golden {path.rsplit('/', 1)[-1]} through attn_fwd_lse", flush=True)
    g, p = problem(path)
    O, LSE = gpu_fwd(p)
    check(LSE, g["LSE"], TOL32, "LSE")
    check(O, g["O"], TOL32, "O")


# Row 1's part of each hand derivation (keys 0 and 1): dK and dV per key, column 0, [T, KV].
ROW1 = {
    "hand_worked_s3_h2_kv1_d1.txt": ([[-0.75 * np.log(3)], [0.75 * np.log(3)]],
                                     [[0.75], [1.25]]),
    "hand_worked_s4_h4_kv2_d1.txt": ([[-2 / 3 * np.log(2)] * 2, [2 / 3 * np.log(2)] * 2],
                                     [[4 / 3, 5 / 6], [5 / 3, 7 / 6]]),
}


@pytest.mark.parametrize("name", sorted(ROW1))
def test_decode_matches_row_1_of_hand_worked(name):
    path = next(f for f in FILES if f.endswith(name))
    print(f"golden {path.rsplit('/', 1)[-1]} row 1 through attn_bwd_decode", flush=True)
    g = pad_head_dim(load_golden(path), 16)
    assert g["seg"][1] == 0                        # row 1 sees keys 0 and 1
    T = 2
    q = g["Q"][1]                                  # [H, d]
    K, V = g["K"][:T], g["V"][:T]                  # [T, KV, d]
    grp = np.arange(g["H"]) // (g["H"] // g["KV"])  # KV head of each query head
    Kh, Vh = K[:, grp, :], V[:, grp, :]            # [T, H, d]
    P = np.exp(g["scale"] * np.einsum("hd,thd->ht", q, Kh) - g["LSE"][1][:, None])   # [H, T]
    # row 1's part of the hand derivation: dS = scale*P*(dP - D) with D = sum_j P*dP
    dP = np.einsum("hd,thd->ht", g["dO"][1], Vh)
    dS = g["scale"] * P * (dP - np.sum(P * dP, axis=1, keepdims=True))
    want_dq = np.einsum("ht,thd->hd", dS, Kh)
    want_dK = np.zeros_like(K)
    want_dV = np.zeros_like(V)
    for h in range(g["H"]):
        want_dK[:, grp[h], :] += dS[h][:, None] * q[h]
        want_dV[:, grp[h], :] += P[h][:, None] * g["dO"][1][h]
    # the same numbers the fixture's derivation writes out for row 1
    assert np.allclose(want_dq[:, 0], g["dQ"][1][:, 0])
    assert np.allclose(want_dK[:, :, 0], ROW1[name][0])
    assert np.allclose(want_dV[:, :, 0], ROW1[name][1])
    t = [to_dev(x.astype(np.float32)) for x in (q, K, V, P, g["dO"][1])]
    dq, dK, dV = torch.zeros_like(t[0]), torch.zeros_like(t[1]), torch.zeros_like(t[2])
    binding.attn_bwd_decode(*t, dq, dK, dV, float(g["scale"]))
    torch.cuda.synchronize()
    check(dq.cpu().numpy(), want_dq, TOL32, "decode dq")
    check(dK.cpu().numpy(), want_dK, TOL32, "decode dK")
    check(dV.cpu().numpy(), want_dV, TOL32, "decode dV")
