"""GPU parity of attn_bwd_rope (the backward with the page's RoPE backward
fused into the write-back of dQ and dK) against the oracle's composition
R^T(init + gradient): every head-dim class (the epilogues pair columns inside
a lane or across neighbouring lanes depending on the class), both key-major
paths, with and without the forward output O, nonzero initial outputs, and a
large pos_offset."""
import numpy as np
import pytest

from causal_gqa_attention_bwd_amd.workloads import make_inputs, random_problem
from tests.test_gpu_parity import check_full, make_seg

pytestmark = pytest.mark.gpu

ROPE_EDGE = [
    (70, 2, 1, 32, "causal"),      # one column per lane (pairs across lanes)
    (97, 3, 1, 64, "arbitrary"),
    (130, 8, 2, 80, "docs"),       # three columns per lane
    (65, 2, 2, 96, "empty_rows"),
    (200, 4, 4, 112, "docs"),
    (129, 4, 1, 128, "causal"),
    (150, 4, 2, 160, "docs"),
    (257, 4, 2, 192, "docs"),      # column halves of three per lane
    (161, 4, 2, 256, "docs"),
]


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_rope_workloads(wid):
    check_full(make_inputs(wid), f"workload {wid} rope", rope=(10000.0, 0))


@pytest.mark.parametrize("case", ROPE_EDGE, ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
@pytest.mark.parametrize("mode", ["stored", "recompute", "stored_o", "recompute_o"])
def test_rope_edge_shapes(case, mode, scratch_limit):
    if mode.startswith("recompute"):
        scratch_limit(0)
    S, H, KV, d, kind = case
    rng = np.random.default_rng(8000 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    check_full(p, "edge " + "S%dH%dKV%dd%d_%s" % case + f" rope {mode}", init=init,
               with_o=mode.endswith("_o"), rope=(500.0, 13))


@pytest.mark.parametrize("mode", ["stored", "recompute"])
def test_rope_large_offset(mode, scratch_limit):
    if mode == "recompute":
        scratch_limit(0)
    check_full(make_inputs(3), f"workload 3 rope offset 1e6 {mode}", rope=(10000.0, 1_000_000))
