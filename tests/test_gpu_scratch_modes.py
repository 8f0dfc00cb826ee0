"""GPU parity of attn_bwd's two ways of running the key-major pass, against the
oracle: reading the stored P / P*dP tiles, here with a budget that the
tiles fill exactly (every slot of the causal bound), and recomputing the
scores (a budget one byte short of the bound, and the stored tiles disabled).
The default budget stores the tiles at these sizes, which the other parity
tests cover too."""
import numpy as np
import pytest

from causal_gqa_attention_bwd_amd import binding
from causal_gqa_attention_bwd_amd.workloads import make_inputs, random_problem
from tests.test_gpu_parity import check_full, make_seg

pytestmark = pytest.mark.gpu

CASES = [
    ("workload", 3),
    ("edge", (513, 16, 2, 64, "docs")),
    ("edge", (320, 8, 1, 128, "arbitrary")),
    ("edge", (257, 4, 2, 192, "docs")),
    ("edge", (161, 4, 2, 256, "docs")),
    ("edge", (300, 2, 1, 240, "empty_rows")),
]


def problem(case):
    kind, arg = case
    if kind == "workload":
        return make_inputs(arg), f"workload {arg}"
    S, H, KV, d, segkind = arg
    rng = np.random.default_rng(5000 + S + d)
    return (random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, segkind)),
            "S%dH%dKV%dd%d_%s" % arg)


def tile_bytes(S, H):
    nblk = (S + 31) // 32
    return nblk * (nblk + 1) // 2 * H * 8192


@pytest.mark.parametrize("case", CASES, ids=lambda c: str(c[1]))
def test_stored_tiles_at_the_exact_budget(case, monkeypatch):
    p, tag = problem(case)
    S, H, d = p["Q"].shape
    monkeypatch.setenv("ATTNBWD_SCRATCH_MB", repr(tile_bytes(S, H) / 2**20))
    assert binding.bwd_plan(S, H, p["K"].shape[1], d)[1]
    check_full(p, f"{tag} stored")


@pytest.mark.parametrize("mb", ["short", "0"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: str(c[1]))
def test_recomputed_scores(case, mb, monkeypatch):
    p, tag = problem(case)
    S, H, d = p["Q"].shape
    budget = repr((tile_bytes(S, H) - 1) / 2**20) if mb == "short" else mb
    monkeypatch.setenv("ATTNBWD_SCRATCH_MB", budget)
    assert not binding.bwd_plan(S, H, p["K"].shape[1], d)[1]
    check_full(p, f"{tag} recomputed")
