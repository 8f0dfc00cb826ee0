"""GPU tests of the paired schedule of plain causal calls (seg = NULL).

With a plain causal mask every workgroup serves a tile and its mirror
(n - 1 - t), so the grids halve; each tile's arithmetic is unchanged, except
that the dK/dV pass sweeps a mirror tile's query tiles upwards (so that the
workgroups read the same Q and dO rows at the same time), which reorders the
fp32 sums of those dK and dV rows.  The results must therefore equal, bit
for bit, those of the same problem given an all-zero seg (served one tile
per workgroup, and held to the oracle by the other parity tests), in every
mode: stored tiles and recomputed scores, the row term computed or read off
the forward output, with and without the RoPE backward -- dK and dV to
rounding only (1e-4 of their largest entry, a twentieth of the parity
bound).  Unpaired calls of few key
tiles also split each group's heads over workgroups whose partial dK, dV are
summed afterwards, which reorders those sums once more.  The shapes give odd and even tile counts of both tile heights,
ragged last tiles, and sequences shorter than one tile.  A few are also held
to the oracle directly, with nonzero initial outputs.
"""
import numpy as np
import pytest

import oracle
from causal_gqa_attention_bwd_amd.workloads import random_problem
from tests.gpu_helpers import TOL, gpu_bwd, rel_err

pytestmark = pytest.mark.gpu
ROUNDING = 1e-4  # two fp32 sums of the same terms in opposite orders

SHAPES = [  # S, H, KV, d
    (1, 2, 1, 64),
    (33, 2, 2, 16),
    (65, 2, 2, 32),
    (129, 4, 2, 128),
    (191, 3, 1, 96),
    (300, 4, 2, 64),
    (333, 4, 1, 256),
    (448, 2, 1, 192),
    (700, 8, 2, 128),
]


def say(msg):
    print(msg, flush=True)


def problem(shape):
    S, H, KV, d = shape
    return random_problem(np.random.default_rng(9100 + S + d), S, H, KV, d)


@pytest.mark.parametrize("entry", ["plain", "o", "rope"])
@pytest.mark.parametrize("mode", ["stored", "recompute"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "S%dH%dKV%dd%d" % c)
def test_paired_equals_unpaired(shape, mode, entry, scratch_limit):
    if mode == "recompute":
        scratch_limit(0)
    p = problem(shape)
    O, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], None, p["scale"])
    rng = np.random.default_rng(9200 + shape[0])
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    kw = dict(init=init, O=O if entry == "o" else None,
              rope=(10000.0, 5) if entry == "rope" else None)
    say(f"[gpu] pairing S{shape[0]} H{shape[1]} KV{shape[2]} d{shape[3]} {mode} {entry}")
    paired = gpu_bwd(p, lse, use_seg=False, **kw)
    unpaired = gpu_bwd(p, lse, **kw)
    # a gradient that is zero in exact arithmetic (dK with one key: dS = 0)
    # holds rounding noise only: its bound is then relative to the largest one
    overall = max(float(np.max(np.abs(b - i0))) for b, i0 in zip(unpaired, init))
    for name, a, b, i0 in zip(("dQ", "dK", "dV"), paired, unpaired, init):
        if name != "dQ":
            ref = max(float(np.max(np.abs(b - i0))), 1e-2 * overall, 1e-30)
            e = float(np.max(np.abs(a - b))) / ref
            assert e <= ROUNDING, f"{name}: paired and unpaired schedules differ by {e:.2e}"
        else:
            assert np.array_equal(a, b), f"{name}: paired and unpaired schedules differ"


@pytest.mark.parametrize("shape", [SHAPES[1], SHAPES[4], SHAPES[6], SHAPES[8]],
                         ids=lambda c: "S%dH%dKV%dd%d" % c)
def test_paired_matches_oracle(shape):
    p = problem(shape)
    _, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], None, p["scale"], want_o=False)
    rng = np.random.default_rng(9300 + shape[0])
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    ref = oracle.attn_bwd_f64(p["Q"], p["K"], p["V"], p["dO"], lse, None, p["scale"])
    say(f"[gpu] pairing vs oracle S{shape[0]} H{shape[1]} KV{shape[2]} d{shape[3]}")
    got = gpu_bwd(p, lse, init=init, use_seg=False)
    for name, g, i0, r in zip(("dQ", "dK", "dV"), got, init, ref):
        e = rel_err(g.astype(np.float64) - i0, r)
        say(f"[gpu]   {name} rel err {e:.2e}")
        assert e <= TOL, f"{name} rel err {e:.3e} > {TOL}"
