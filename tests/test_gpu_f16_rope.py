"""GPU parity of attn_bwd_f16_rope (fp16 matrix-core operands, with the page's
RoPE backward fused into the write-back of dQ and dK) against the oracle's
composition R^T(init + gradient), at the fp16 bars of test_gpu_f16.py: the
five workloads (the two large ones element by element over whole tensors)
within 2e-3 of the largest gradient, the small edge shapes of every head-dim
class element by element within twice their fp16 rounding bound (turned by
the rotation: each column of a pair gets the pair's summed bound).  Covered: with and without the forward output,
nonzero initial outputs (which the rotation turns too), a large
pos_offset, plain causal calls whose key-major pass splits each group's
heads (the partial sums are then added and dK rotated after the pass) and
document masks."""
import numpy as np
import pytest

from causal_gqa_attention_bwd_amd.workloads import make_inputs, random_problem
from tests.fullsize_ref import reference, rel_errs, rope_reference
from tests.gpu_helpers import TOL, gpu_bwd
from tests.test_gpu_parity import check_full, make_seg
from tests.test_gpu_rope import ROPE_EDGE

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("wid", [1, 2, 3])
def test_f16_rope_workloads(wid, with_o):
    check_full(make_inputs(wid), f"workload {wid} f16 rope", with_o=with_o, f16=True,
               rope=(10000.0, 0))


@pytest.mark.parametrize("with_o", [False, True], ids=["rowterm", "fwd_out"])
@pytest.mark.parametrize("case", ROPE_EDGE + [(700, 8, 2, 128, "causal"), (333, 8, 1, 64, "causal"),
                                              (513, 16, 2, 64, "docs")],
                         ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
def test_f16_rope_edge_shapes(case, with_o):
    S, H, KV, d, kind = case
    rng = np.random.default_rng(8500 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    init = [rng.standard_normal(p[k].shape).astype(np.float32) for k in ("Q", "K", "V")]
    check_full(p, "edge f16 rope " + "S%dH%dKV%dd%d_%s" % case, init=init, with_o=with_o,
               f16=True, rope=(500.0, 13), f16_bound=True)


def test_f16_rope_large_offset():
    check_full(make_inputs(3), "workload 3 f16 rope offset 1e6", f16=True, rope=(10000.0, 1_000_000))


@pytest.mark.parametrize("case", [(257, 4, 2, 192, "docs"), (161, 4, 2, 256, "docs"),
                                  (129, 4, 1, 128, "causal")],
                         ids=lambda c: "S%dH%dKV%dd%d_%s" % c)
def test_f16_rope_large_offset_wide_heads(case):
    # positions near 2^31 at the head dims whose dQ write-back rotates whole
    # 16-byte row chunks: angles up to ~2e9 rad in the fp64 sincos
    S, H, KV, d, kind = case
    rng = np.random.default_rng(8600 + S + d)
    p = random_problem(rng, S, H, KV, d, seg=make_seg(rng, S, kind))
    check_full(p, "f16 rope offset 2^31-S-1 " + "S%dH%dKV%dd%d_%s" % case, f16=True,
               rope=(10000.0, 2**31 - S - 1), f16_bound=True)


@pytest.mark.parametrize("wid", [4, 5])
def test_f16_rope_fullsize_whole_tensor(wid):
    x, _, lse, _ = reference(wid)
    ref = rope_reference(wid, 10000.0, 0)
    w = x["workload"]
    say(f"[gpu] workload {wid}: attn_bwd_f16_rope S={w.S} H={w.H} KV={w.KV} d={w.d}, every element")
    got = gpu_bwd(x, lse, use_seg=bool(np.any(x["seg"])), f16=True, rope=(10000.0, 0))
    errs = rel_errs(got, ref)
    say(f"[gpu] workload {wid} f16 rope: rel err " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= TOL, f"workload {wid} f16 rope: {name} rel err {e:.3e} > {TOL}"
