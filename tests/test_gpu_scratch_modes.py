"""GPU parity of attn_bwd's ways of running the key-major pass, against the
oracle:
- reading the stored P / P*dP tiles, with a scratch limit that the tiles of
  all heads fill exactly (every slot of the causal bound);
- reading stored tiles in head chunks, when the limit holds the tiles of only
  some heads: whole KV groups per chunk (also a smaller last chunk), or a
  share of one group's heads (the chunks then add into the same dK, dV
  rows one after another), with head splits, the forward output, RoPE,
  nonzero initial outputs and the paired plain-causal schedule;
- recomputing the scores (a limit below one head's tiles, and the tiles
  disabled).
The default limit stores the tiles of all heads at these sizes, which the
other parity tests cover too."""
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
def test_stored_tiles_at_the_exact_limit(case, scratch_limit):
    p, tag = problem(case)
    S, H, d = p["Q"].shape
    scratch_limit(tile_bytes(S, H))
    assert binding.bwd_plan_heads(S, H, p["K"].shape[1], d)[1] == H
    check_full(p, f"{tag} stored")


@pytest.mark.parametrize("mb", ["short", "0"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: str(c[1]))
def test_recomputed_scores(case, mb, scratch_limit):
    p, tag = problem(case)
    S, H, d = p["Q"].shape
    scratch_limit(tile_bytes(S, 1) - 1 if mb == "short" else 0)
    assert not binding.bwd_plan(S, H, p["K"].shape[1], d)[1]
    check_full(p, f"{tag} recomputed")


# (S, H, KV, d, seg kind, heads whose tiles fit the limit, heads per chunk)
CHUNKS = [
    (513, 16, 2, 64, "docs", 12, 8),        # one whole group per chunk, head splits
    (513, 16, 2, 64, "docs", 3, 2),         # a quarter of a group per chunk
    (513, 16, 2, 64, "docs", 1, 1),         # one head per chunk
    (300, 12, 4, 64, "docs", 9, 9),         # three groups, then a last chunk of one
    (700, 8, 2, 128, "causal", 5, 4),       # plain causal (paired), one group per chunk
    (333, 8, 1, 256, "causal", 6, 4),       # plain causal, half a group per chunk
    (257, 6, 3, 192, "arbitrary", 4, 4),    # two groups of two heads, then one group
    (161, 4, 2, 96, "empty_rows", 1, 1),
]


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("case", CHUNKS, ids=lambda c: "S%dH%dKV%dd%d_%s_fit%d" % c[:6])
def test_stored_tiles_in_head_chunks(case, with_o, scratch_limit):
    S, H, KV, d, kind, fit, chunk = case
    rng = np.random.default_rng(5200 + S + d + fit)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    scratch_limit(tile_bytes(S, fit))
    assert binding.bwd_plan_heads(S, H, KV, d)[1] == chunk
    check_full(p, "S%dH%dKV%dd%d_%s chunks of %d" % (S, H, KV, d, kind, chunk), init=init,
               with_o=with_o)


@pytest.mark.parametrize("case", [CHUNKS[1], CHUNKS[3], CHUNKS[4]],
                         ids=lambda c: "S%dH%dKV%dd%d_%s_fit%d" % c[:6])
def test_rope_in_head_chunks(case, scratch_limit):
    S, H, KV, d, kind, fit, chunk = case
    rng = np.random.default_rng(5300 + S + d + fit)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    scratch_limit(tile_bytes(S, fit))
    assert binding.bwd_plan_heads(S, H, KV, d)[1] == chunk
    check_full(p, "S%dH%dKV%dd%d_%s rope, chunks of %d" % (S, H, KV, d, kind, chunk), init=init,
               rope=(500.0, 7))


def test_head_chunks_match_one_piece(scratch_limit):
    # the same problem in one piece and in chunks of one group: dQ is formed
    # per head either way (bit for bit); dK and dV too, since each group's
    # sums run over the same heads in the same order
    from tests.gpu_helpers import gpu_bwd
    import oracle
    S, H, KV, d = 1000, 8, 2, 64
    rng = np.random.default_rng(5400)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, "docs"))
    _, lse = oracle.attn_fwd(p["Q"], p["K"], p["V"], p["seg"], p["scale"], want_o=False)
    whole = gpu_bwd(p, lse)
    scratch_limit(tile_bytes(S, 4))
    assert binding.bwd_plan_heads(S, H, KV, d)[1] == 4
    chunked = gpu_bwd(p, lse)
    for a, b in zip(whole, chunked):
        assert np.array_equal(a, b)
