"""Argument errors of every backward entry point are status codes returned on
the host before any HIP call, so they are checked here without a GPU.  The
tensor pointers are placeholders that no failing (or empty) call reads: an
aligned non-NULL address, NULL, or a misaligned one."""
import math

import pytest

from causal_gqa_attention_bwd_amd import binding

OK, INVALID, UNSUPPORTED = binding.ATTN_OK, binding.ATTN_ERR_INVALID_ARG, binding.ATTN_ERR_UNSUPPORTED
A = 0x10000        # an aligned placeholder address
MIS = 0x10004      # a misaligned one


def bwd_args(S=8, H=2, KV=1, d=64, scale=0.125, null=None, mis=None, with_o=True):
    """Q, K, V, O, dO, LSE, seg, dQ, dK, dV, S, H, KV, d, scale, stream."""
    names = ["Q", "K", "V", "O", "dO", "LSE", "seg", "dQ", "dK", "dV"]
    ptrs = {n: A for n in names}
    if not with_o:
        ptrs["O"] = None
    if null:
        ptrs[null] = None
    if mis:
        ptrs[mis] = MIS
    return [ptrs[n] for n in names] + [S, H, KV, d, scale, None]


def decode_args(T=8, H=2, KV=1, d=64, scale=0.125, null=(), mis=None):
    """q, K, V, P, dO, dq, dK, dV, T, H, KV, d, scale, stream."""
    names = ["q", "K", "V", "P", "dO", "dq", "dK", "dV"]
    ptrs = {n: A for n in names}
    for n in null:
        ptrs[n] = None
    if mis:
        ptrs[mis] = MIS
    return [ptrs[n] for n in names] + [T, H, KV, d, scale, None]


CASES = [
    # attn_bwd_short
    ("attn_bwd_short", bwd_args(null="Q"), INVALID, "NULL"),
    ("attn_bwd_short", bwd_args(H=3, KV=2), INVALID, "multiple"),
    ("attn_bwd_short", bwd_args(scale=math.inf), INVALID, "scale"),
    ("attn_bwd_short", bwd_args(S=1025), UNSUPPORTED, "1024"),
    ("attn_bwd_short", bwd_args(d=272), UNSUPPORTED, "head_dim"),
    ("attn_bwd_short", bwd_args(d=24), UNSUPPORTED, "head_dim"),
    ("attn_bwd_short", bwd_args(mis="dK"), UNSUPPORTED, "aligned"),
    ("attn_bwd_short", bwd_args(S=1024, H=16384, KV=1, d=64), UNSUPPORTED, "2^31"),
    ("attn_bwd_short", bwd_args(S=0), OK, ""),
    ("attn_bwd_short", bwd_args(S=0, with_o=False), OK, ""),
    # attn_bwd_decode
    ("attn_bwd_decode", decode_args(null=("q",)), INVALID, "NULL"),
    ("attn_bwd_decode", decode_args(null=("K",)), INVALID, "NULL"),
    ("attn_bwd_decode", decode_args(T=-1), INVALID, "negative"),
    ("attn_bwd_decode", decode_args(H=4, KV=3), INVALID, "multiple"),
    ("attn_bwd_decode", decode_args(d=250), UNSUPPORTED, "head_dim"),
    ("attn_bwd_decode", decode_args(mis="P"), UNSUPPORTED, "aligned"),
    ("attn_bwd_decode", decode_args(T=0, null=("K", "V", "P", "dK", "dV")), OK, ""),
    # attn_bwd_f16
    ("attn_bwd_f16", bwd_args(null="dV"), INVALID, "NULL"),
    ("attn_bwd_f16", bwd_args(d=8), UNSUPPORTED, "head_dim"),
    ("attn_bwd_f16", bwd_args(mis="seg"), UNSUPPORTED, "aligned"),
    ("attn_bwd_f16", bwd_args(S=0, with_o=False), OK, ""),
    # attn_bwd_noalloc (Q, K, V, dO, LSE, seg, dQ, dK, dV: no O)
    ("attn_bwd_noalloc", [A] * 5 + [None] + [A] * 3 + [262144, 64, 8, 64, 0.125, None],
     UNSUPPORTED, "scratch"),
    ("attn_bwd_noalloc", [A] * 5 + [None] + [A, A, None] + [8, 2, 1, 64, 0.125, None], INVALID,
     "NULL"),
    ("attn_bwd_noalloc", [A] * 5 + [None] + [A] * 3 + [8, 3, 2, 64, 0.125, None], INVALID,
     "multiple"),
    ("attn_bwd_noalloc", [A] * 5 + [None] + [A] * 3 + [0, 2, 1, 64, 0.125, None], OK, ""),
    # attn_bwd_o
    ("attn_bwd_o", bwd_args(null="O"), INVALID, "NULL"),
    ("attn_bwd_o", bwd_args(S=-4), INVALID, "negative"),
    ("attn_bwd_o", bwd_args(S=0), OK, ""),
]


@pytest.mark.parametrize("entry,args,status,text", CASES,
                         ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_entry_rejects_bad_arguments_on_the_host(entry, args, status, text):
    lib = binding.load()
    st = getattr(lib, entry)(*args)
    assert st == status, (st, binding.last_error())
    if status != OK:
        assert text in binding.last_error(), binding.last_error()
    else:
        assert binding.last_error() == ""


@pytest.mark.parametrize("base,pos,text", [(0.0, 0, "rope_base"), (math.nan, 0, "rope_base"),
                                           (1e4, -1, "pos_offset"), (1e4, 2**31 - 4, "pos_offset")])
@pytest.mark.parametrize("entry", ["attn_bwd_rope", "attn_bwd_f16_rope"])
def test_rope_entry_rejects_bad_rotation_arguments(base, pos, text, entry):
    lib = binding.load()
    args = bwd_args(S=8)[:-1] + [base, pos, None]
    st = getattr(lib, entry)(*args)
    assert st == INVALID, (st, binding.last_error())
    assert text in binding.last_error() or "pos" in binding.last_error()


def _host_problem(S=8, H=2, KV=1, d=16):
    import torch
    z = lambda *s: torch.zeros(*s, dtype=torch.float32)  # noqa: E731
    return dict(Q=z(S, H, d), K=z(S, KV, d), V=z(S, KV, d), O=z(S, H, d), dO=z(S, H, d),
                LSE=z(S, H), dQ=z(S, H, d), dK=z(S, KV, d), dV=z(S, KV, d))


@pytest.mark.parametrize("entry", ["attn_bwd", "attn_bwd_o", "attn_bwd_rope", "attn_bwd_f16",
                                   "attn_bwd_f16_rope", "attn_bwd_short", "attn_bwd_noalloc",
                                   "attn_fwd_lse", "attn_bwd_decode"])
def test_binding_rejects_host_tensors_before_any_launch(entry):
    # host tensors carry host addresses; handed to a kernel they would fault
    # the GPU, so the binding refuses them with ValueError and calls nothing
    t = _host_problem()
    calls = {
        "attn_bwd": lambda: binding.attn_bwd(t["Q"], t["K"], t["V"], t["dO"], t["LSE"], None,
                                             t["dQ"], t["dK"], t["dV"], 0.25),
        "attn_bwd_o": lambda: binding.attn_bwd_o(t["Q"], t["K"], t["V"], t["O"], t["dO"],
                                                 t["LSE"], None, t["dQ"], t["dK"], t["dV"], 0.25),
        "attn_bwd_rope": lambda: binding.attn_bwd_rope(t["Q"], t["K"], t["V"], None, t["dO"],
                                                       t["LSE"], None, t["dQ"], t["dK"], t["dV"],
                                                       0.25, 1e4, 0),
        "attn_bwd_f16": lambda: binding.attn_bwd_f16(t["Q"], t["K"], t["V"], None, t["dO"],
                                                     t["LSE"], None, t["dQ"], t["dK"], t["dV"],
                                                     0.25),
        "attn_bwd_f16_rope": lambda: binding.attn_bwd_f16_rope(t["Q"], t["K"], t["V"], None,
                                                               t["dO"], t["LSE"], None, t["dQ"],
                                                               t["dK"], t["dV"], 0.25, 1e4, 0),
        "attn_bwd_short": lambda: binding.attn_bwd_short(t["Q"], t["K"], t["V"], None, t["dO"],
                                                         t["LSE"], None, t["dQ"], t["dK"],
                                                         t["dV"], 0.25),
        "attn_bwd_noalloc": lambda: binding.attn_bwd_noalloc(t["Q"], t["K"], t["V"], t["dO"],
                                                             t["LSE"], None, t["dQ"], t["dK"],
                                                             t["dV"], 0.25),
        "attn_fwd_lse": lambda: binding.attn_fwd_lse(t["Q"], t["K"], t["V"], None, None, t["LSE"],
                                                     0.25),
        "attn_bwd_decode": lambda: binding.attn_bwd_decode(t["Q"][0], t["K"], t["V"],
                                                           t["LSE"].T.contiguous(), t["dO"][0],
                                                           t["dQ"][0], t["dK"], t["dV"], 0.25),
    }
    with pytest.raises(ValueError, match="GPU tensors only"):
        calls[entry]()
