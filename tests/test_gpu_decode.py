"""GPU parity of attn_bwd_decode (single-query backward over a KV history with
stored probabilities, page "rullama 0.5.0", pass 1 and 2 of 2) against the
fp64 oracle, element by element: max|gpu - oracle| <= 2e-3 * max|oracle| per
gradient, with nonzero initial outputs (the += contract; the accumulated
parts are compared).  P is the softmax of scale * q.k over the history, as a
forward would store it.  Shapes cover one key, ragged last chunks (128-key
chunks, 16-key wave steps), every head-dim class of the score pass (d <= 64,
<= 128, <= 256, with d / 4 not a power of two), every head-batch class of the
dK/dV pass (groups of <= 4, <= 8 and more heads, and groups of 20 and 80 that
take several 16-head batches), and the full-size benchmark history."""
import numpy as np
import pytest
import torch

import oracle
from causal_gqa_attention_bwd_amd import binding
from tests.gpu_helpers import TOL, dev, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [  # T, H, KV, d
    (1, 2, 1, 16),
    (7, 4, 2, 48),
    (64, 8, 2, 64),
    (65, 4, 4, 80),
    (300, 32, 8, 128),
    (129, 40, 2, 96),     # group of 20: two 16-head batches in the dK/dV pass
    (200, 80, 1, 32),     # group of 80: two 64-head batches in the score pass
    (1000, 16, 1, 256),
    (500, 24, 4, 112),    # group of 6: the 8-head batch
    (333, 12, 1, 160),    # group of 12: one partly filled 16-head batch
    (4096, 32, 8, 128),
]


def say(msg):
    print(msg, flush=True)


def problem(T, H, KV, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d)).astype(np.float32)
    K = rng.standard_normal((T, KV, d)).astype(np.float32)
    V = rng.standard_normal((T, KV, d)).astype(np.float32)
    dO = rng.standard_normal((H, d)).astype(np.float32)
    scale = np.float32(1.0 / np.sqrt(d))
    g = H // KV
    x = np.stack([float(scale) * K[:, h // g, :].astype(np.float64) @ q[h].astype(np.float64)
                  for h in range(H)])
    x -= x.max(axis=1, keepdims=True)
    P = np.exp(x)
    P = (P / P.sum(axis=1, keepdims=True)).astype(np.float32)
    init = [rng.standard_normal(s).astype(np.float32) for s in ((H, d), (T, KV, d), (T, KV, d))]
    return q, K, V, P, dO, scale, init


def gpu_decode(q, K, V, P, dO, scale, init):
    t = [to_dev(x) for x in (q, K, V, P, dO)]
    out = [to_dev(x.copy()) for x in init]
    binding.attn_bwd_decode(*t, *out, float(scale))
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "T%dH%dKV%dd%d" % c)
def test_decode_parity(shape):
    T, H, KV, d = shape
    q, K, V, P, dO, scale, init = problem(T, H, KV, d, 9500 + T + H)
    ref = oracle.attn_bwd_decode_f64(q, K, V, P, dO, float(scale))
    say(f"[gpu] attn_bwd_decode T={T} H={H} KV={KV} d={d}")
    got = gpu_decode(q, K, V, P, dO, scale, init)
    overall = max(float(np.max(np.abs(r))) for r in ref)
    for name, g, i0, r in zip(("dq", "dK", "dV"), got, init, ref):
        g = g.astype(np.float64) - i0
        assert np.all(np.isfinite(g))
        # a gradient that is zero in exact arithmetic (one key) holds rounding
        # noise only: its bound is then relative to the largest gradient
        e = float(np.max(np.abs(g - r))) / max(float(np.max(np.abs(r))), 1e-4 * overall, 1e-30)
        say(f"[gpu]   {name} rel err {e:.2e}")
        assert e <= TOL, f"{name} rel err {e:.3e} > {TOL}"


def test_decode_is_repeatable_and_empty_history_is_a_no_op():
    q, K, V, P, dO, scale, init = problem(777, 16, 4, 64, 9601)
    a = gpu_decode(q, K, V, P, dO, scale, init)
    b = gpu_decode(q, K, V, P, dO, scale, init)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    H, d = q.shape
    dq = to_dev(init[0].copy())
    empty = torch.zeros((0, 4, d), dtype=torch.float32, device=dev())
    binding.attn_bwd_decode(to_dev(q), empty, empty, torch.zeros((H, 0), dtype=torch.float32,
                                                                 device=dev()),
                            to_dev(dO), dq, empty.clone(), empty.clone(), float(scale))
    torch.cuda.synchronize()
    assert np.array_equal(dq.cpu().numpy(), init[0])


def test_decode_fullsize_bench_workload():
    from causal_gqa_attention_bwd_amd.workloads import DECODE_WORKLOAD, make_decode_inputs
    wl = DECODE_WORKLOAD
    x = make_decode_inputs(wl["T"], wl["H"], wl["KV"], wl["d"])
    say(f"[gpu] attn_bwd_decode, the benchmark workload {wl['name']}: oracle ...")
    ref = oracle.attn_bwd_decode_f64(x["q"], x["K"], x["V"], x["P"], x["dO"], float(x["scale"]))
    init = [np.zeros_like(x["q"]), np.zeros_like(x["K"]), np.zeros_like(x["V"])]
    got = gpu_decode(x["q"], x["K"], x["V"], x["P"], x["dO"], x["scale"], init)
    for name, g, r in zip(("dq", "dK", "dV"), got, ref):
        e = float(np.max(np.abs(g - r)) / np.max(np.abs(r)))
        say(f"[gpu]   {name} rel err {e:.2e}")
        assert e <= TOL, f"{name} rel err {e:.3e} > {TOL}"
