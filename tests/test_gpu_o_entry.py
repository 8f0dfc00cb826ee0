"""GPU parity of attn_bwd_o (the row term read off the forward output O)
against the oracle's O entry, on the same seeded inputs and the same fp32 O:
the workloads that finish quickly, edge shapes of every head-dim class, both
ways of running the key-major pass, accumulation into nonzero outputs, a
perturbed O (which the result must follow, so the kernels read D off O).
The two large workloads are compared element by element in
test_gpu_fullsize.py."""
import numpy as np
import pytest

from causal_gqa_attention_bwd_amd.workloads import make_inputs, random_problem
from tests.test_gpu_parity import check_full, make_seg

pytestmark = pytest.mark.gpu

EDGE_O = [
    (2, 2, 1, 32, "causal"),
    (97, 3, 1, 64, "arbitrary"),
    (130, 8, 2, 80, "docs"),
    (65, 2, 2, 96, "empty_rows"),
    (129, 4, 1, 128, "causal"),
    (150, 4, 2, 160, "docs"),
    (257, 4, 2, 192, "docs"),
    (161, 4, 2, 256, "docs"),
]


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_o_entry_workloads(wid):
    check_full(make_inputs(wid), f"workload {wid}", with_o=True)


@pytest.mark.parametrize("case", EDGE_O, ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
@pytest.mark.parametrize("mb", ["default", "0"])
def test_o_entry_edge_shapes(case, mb, scratch_limit):
    if mb != "default":
        scratch_limit(0)
    S, H, KV, d, kind = case
    rng = np.random.default_rng(6000 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    check_full(p, "edge " + "S%dH%dKV%dd%d_%s" % case + f" budget={mb}", with_o=True)


@pytest.mark.parametrize("mb", ["default", "0"])
def test_o_entry_follows_a_perturbed_O(mb, scratch_limit):
    if mb != "default":
        scratch_limit(0)
    x = make_inputs(3)
    rng = np.random.default_rng(6003)
    shift = (0.5 * rng.standard_normal(x["Q"].shape)).astype(np.float32)
    check_full(x, f"workload 3 perturbed O budget={mb}", with_o=True, o_shift=shift)


def test_o_entry_accumulates():
    x = make_inputs(2)
    rng = np.random.default_rng(6002)
    init = [rng.standard_normal(x[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    check_full(x, "workload 2 += (O entry)", init=init, with_o=True)
