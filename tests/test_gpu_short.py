"""GPU parity of attn_bwd_short (the short-sequence backward: one launch with
the forward output O, two without) against the fp64 oracle, element by
element: max|gpu - oracle| <= 2e-3 * max|oracle| per gradient (the fp32 path's
bar; fp32 products and sums).

Covered: the three short workloads whole, with and without O; every padded
head-dim class (32, 64, 96, 128) with d = 16 .. 128, and above 128 columns (144,
192, 256), where the entry runs the general path; every mask kind (plain causal,
documents, arbitrary starts, rows that see no key); lengths 1, 2, ragged
tails (33, 97, 1000) and the maximum 1024 with several waves' worth of blocks;
KV groups of 1 .. 8 heads, with the key blocks' heads split over 1, 2, 4 and 8
workgroups (the split count follows from the shape: 2 at S=200 with 8 heads
per group, 4 at S=1024 with 4 (or 8 heads per group over 2 KV heads), 8 at
S=1024 with 8 heads over one KV head); nonzero initial outputs
(+=); repeatability (the
sums have a fixed order, so two calls agree bit for bit); agreement of the O
and row-term forms; and the size limit (ATTN_ERR_UNSUPPORTED above 1024
positions).
"""
import numpy as np
import pytest
import torch

import oracle
from causal_gqa_attention_bwd_amd import binding
from causal_gqa_attention_bwd_amd.workloads import make_inputs, random_problem
from tests.gpu_helpers import dev, gpu_bwd, to_dev
from tests.test_gpu_parity import check_full, make_seg

pytestmark = pytest.mark.gpu

SHORT_EDGE = [  # S, H, KV, d, mask
    (1, 1, 1, 16, "causal"),
    (2, 2, 1, 32, "causal"),
    (33, 4, 2, 48, "docs"),
    (97, 3, 1, 64, "arbitrary"),
    (64, 2, 2, 16, "empty_rows"),
    (200, 8, 1, 32, "docs"),
    (333, 6, 3, 64, "arbitrary"),
    (1000, 4, 4, 64, "docs"),
    (1024, 8, 2, 32, "causal"),
    (1024, 2, 1, 64, "empty_rows"),
    (700, 12, 2, 48, "causal"),     # group of 6: two head splits of 3
    (1024, 16, 2, 64, "docs"),      # group of 8: four head splits
    (1024, 8, 1, 32, "docs"),       # group of 8: eight head splits
    (130, 8, 2, 80, "docs"),        # 96-column tiles
    (65, 2, 2, 96, "empty_rows"),
    (321, 4, 1, 112, "arbitrary"),  # 128-column tiles
    (1024, 8, 8, 128, "docs"),
    (1024, 16, 2, 128, "causal"),   # group of 8 split over the key role
    (3, 3, 3, 128, "singletons"),
    # above 128 columns: the general path's kernels
    (200, 4, 2, 144, "docs"),
    (1024, 8, 2, 192, "causal"),
    (513, 4, 1, 256, "arbitrary"),
    (300, 2, 2, 256, "empty_rows"),
    (64, 4, 2, 256, "singletons"),
]


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("with_o", [True, False], ids=["fwd_out", "rowterm"])
@pytest.mark.parametrize("wid", [1, 2, 3])
def test_short_workload_parity(wid, with_o):
    check_full(make_inputs(wid), f"workload {wid} short", with_o=with_o, short=True)


@pytest.mark.parametrize("with_o", [True, False], ids=["fwd_out", "rowterm"])
@pytest.mark.parametrize("case", SHORT_EDGE, ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
def test_short_edge_parity(case, with_o):
    S, H, KV, d, kind = case
    rng = np.random.default_rng(5100 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    check_full(p, "edge short " + "S%dH%dKV%dd%d_%s" % case, with_o=with_o, short=True)


@pytest.mark.parametrize("with_o", [True, False], ids=["fwd_out", "rowterm"])
def test_short_accumulates(with_o):
    x = make_inputs(2)
    rng = np.random.default_rng(5200)
    init = [rng.standard_normal(x[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    check_full(x, "workload 2 += short", init=init, with_o=with_o, short=True)


def test_short_repeats_bit_for_bit():
    p = random_problem(np.random.default_rng(5300), 700, 8, 2, 64,
                       seg=make_seg(np.random.default_rng(5301), 700, "docs"))
    O, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], p["seg"], p["scale"], want_o=True)
    for o in (O, None):
        say(f"[gpu] short repeatability S700 H8 KV2 d64 O={'yes' if o is not None else 'no'}")
        a = gpu_bwd(p, lse, O=o, short=True)
        b = gpu_bwd(p, lse, O=o, short=True)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("S,d", [(1025, 32), (1025, 256)])
def test_short_rejects_sizes_beyond_its_limits(S, d):
    H = KV = 1
    z = lambda *shape: torch.zeros(shape, dtype=torch.float32, device=dev())
    Q, K, V, dO, dQ, dK, dV = z(S, H, d), z(S, KV, d), z(S, KV, d), z(S, H, d), z(S, H, d), \
        z(S, KV, d), z(S, KV, d)
    lse = z(S, H)
    with pytest.raises(binding.AttnError) as e:
        binding.attn_bwd_short(Q, K, V, None, dO, lse, None, dQ, dK, dV, 0.125)
    assert e.value.status == 2  # ATTN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert not dQ.any() and not dK.any() and not dV.any()
