"""GPU parity on seeded random shapes, through every general entry: attn_bwd
and attn_bwd_f16 with nonzero initial outputs (the += contract), attn_bwd_o
and attn_bwd_f16 with the forward output.  Shapes draw the group size (1, 2,
4, 8), the KV head count, every padded head-dim class, lengths up to 900 and
every mask kind (plain causal, packed documents, arbitrary starts, rows that
see no key), so they reach the paired and unpaired schedules, the head
splits and the fp16 full-block steps in combinations the fixed lists do not.
Also random shapes through attn_bwd_short (its range: S <= 1024, head_dim <=
128), attn_bwd_rope (random position offsets) and attn_bwd_decode.  Bars as
in the fixed tests: 2e-3 of the largest gradient for fp32 operands; for fp16
operands every element within twice its rounding bound derived from the
inputs (tests/f16_bounds.py)."""
import numpy as np
import pytest

import oracle
from causal_gqa_attention_bwd_amd.workloads import random_problem
from tests.gpu_helpers import TOL
from tests.test_gpu_decode import gpu_decode, problem
from tests.test_gpu_parity import check_full, make_seg

pytestmark = pytest.mark.gpu


def draw(i):
    rng = np.random.default_rng(7700 + i)
    g = int(rng.choice([1, 2, 4, 8]))
    KV = int(rng.choice([1, 2, 3, 4]))
    H = g * KV
    d = int(rng.choice([16, 32, 48, 64, 96, 128, 160, 192, 256]))
    S = int(rng.integers(1, 900))
    while S * H * d > 900 * 16 * 64:  # the oracle finishes each in well under a second
        S = max(1, S // 2)
    kind = str(rng.choice(["causal", "docs", "arbitrary", "empty_rows"]))
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    return p, init, f"random {i}: S={S} H={H} KV={KV} d={d} {kind}"


# draw 2299 (S=686, H=4, KV=4, d=32, documents) has dV entries far smaller
# than their nonzero initial values: there the fp32 rounding of the output
# exceeds the gradient's own fp16 bound, which the allowance now counts
@pytest.mark.parametrize("mode", ["plain", "o", "f16", "f16o"])
@pytest.mark.parametrize("i", list(range(24)) + [2299])
def test_random_shape_parity(i, mode):
    p, init, tag = draw(i)
    f16 = mode.startswith("f16")
    with_o = mode in ("o", "f16o")
    check_full(p, f"{tag} {mode}", init=None if with_o else init, with_o=with_o, f16=f16,
               tol=TOL, f16_bound=f16)


def draw_short(i):
    """attn_bwd_short's range: S <= 1024, head_dim <= 128."""
    rng = np.random.default_rng(7800 + i)
    g = int(rng.choice([1, 2, 4, 8]))
    KV = int(rng.choice([1, 2, 3, 4]))
    H, d = g * KV, int(rng.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    S = int(rng.integers(1, 1025))
    kind = str(rng.choice(["causal", "docs", "arbitrary", "empty_rows"]))
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    return p, init, f"random short {i}: S={S} H={H} KV={KV} d={d} {kind}"


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("i", range(16))
def test_random_short_parity(i, with_o):
    p, init, tag = draw_short(i)
    check_full(p, tag, init=None if with_o else init, with_o=with_o, short=True)


@pytest.mark.parametrize("i", range(12))
def test_random_rope_parity(i):
    p, _, tag = draw(100 + i)
    pos = int(np.random.default_rng(7900 + i).integers(0, 5000))
    check_full(p, f"{tag} rope pos {pos}", rope=(10000.0, pos), with_o=bool(i % 2))


@pytest.mark.parametrize("i", range(12))
def test_random_decode_parity(i):
    rng = np.random.default_rng(8000 + i)
    g = int(rng.choice([1, 2, 4, 8, 12]))
    KV = int(rng.choice([1, 2, 4]))
    H, d = g * KV, int(rng.choice([16, 32, 64, 80, 128, 160, 256]))
    T = int(rng.integers(1, 3000))
    q, K, V, P, dO, scale, init = problem(T, H, KV, d, 8100 + i)
    ref = oracle.attn_bwd_decode_f64(q, K, V, P, dO, float(scale))
    print(f"[gpu] random decode {i}: T={T} H={H} KV={KV} d={d}", flush=True)
    got = gpu_decode(q, K, V, P, dO, scale, init)
    overall = max(float(np.max(np.abs(r))) for r in ref)
    for name, gg, i0, r in zip(("dq", "dK", "dV"), got, init, ref):
        e = float(np.max(np.abs(gg.astype(np.float64) - i0 - r))) / max(
            float(np.max(np.abs(r))), 1e-4 * overall, 1e-30)
        assert e <= TOL, f"decode {i} {name} rel err {e:.3e} > {TOL}"
