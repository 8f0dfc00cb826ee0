"""The C-ABI library loads and exports every entry point include/attnbwd.h
declares (no compute call: this runs without a GPU)."""
import ctypes
import os
import re

import pytest

from causal_gqa_attention_bwd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "attnbwd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} is declared but not exported"


def test_argument_errors_need_no_gpu():
    # invalid arguments are rejected on the host before any HIP call
    lib = binding.load()
    null = None
    st = lib.attn_bwd(null, null, null, null, null, null, null, null, null, 8, 2, 1, 64,
                      ctypes.c_float(0.125), null)
    assert st == binding.ATTN_ERR_INVALID_ARG
    assert "NULL" in binding.last_error()


def causal_pairs(nblk):
    return nblk * (nblk + 1) // 2


def up(n):
    return (n + 255) // 256 * 256


@pytest.fixture
def limit():
    saved = []

    def set_limit(nbytes):
        prev = binding.set_scratch_limit(int(nbytes))
        if not saved:
            saved.append(prev)

    yield set_limit
    if saved:
        binding.set_scratch_limit(saved[0])


DEFAULT_LIMIT = 32 << 30


def test_plan_sizes_the_workspace(limit):
    # host-only query: D [S,H], block metadata, and the P / P*dP tile scratch
    # (two 32x32 fp32 tiles per (query block, key block, head) of the causal
    # triangle), each part 256-byte aligned, then -- the most a call takes is
    # an unpaired one -- the partial dK, dV of the key-major head splits: 64
    # key tiles x 8 KV heads = 512 workgroups, so the 4 heads of a group go
    # to 4 workgroups (about 2048 in all); the first adds into dK, dV, each
    # of the other 3 writes an [S, KV, d] slice of dK and one of dV
    limit(DEFAULT_LIMIT)
    S, H = 4096, 32
    nblk = S // 32
    meta = up(up(up(S * H * 4) + 2 * nblk * 4) + (nblk + 1) * 8)
    part = 2 * 3 * S * 8 * 128 * 4
    assert binding.bwd_plan_heads(S, H, 8, 128) == (meta + causal_pairs(nblk) * H * 8192 + part, H)
    # a group of one head cannot split
    assert binding.bwd_plan(S, 8, 8, 128) == (
        up(up(up(S * 8 * 4) + 2 * nblk * 4) + (nblk + 1) * 8) + causal_pairs(nblk) * 8 * 8192, True)
    limit(0)
    assert binding.bwd_plan_heads(S, H, 8, 128) == (meta, 0)


def test_plan_takes_head_chunks_below_the_limit(limit):
    # 16384 rows, 16 heads in 2 groups of 8: all tiles need 16.03 GiB, within
    # the default limit; below it the tiles are stored for as many whole
    # groups as fit, else for the largest divisor of a group's 8 heads that
    # fits, else not at all (recomputed scores: D and the metadata only)
    S, H, KV, d = 16384, 16, 2, 256
    per_head = causal_pairs(S // 32) * 8192
    limit(DEFAULT_LIMIT)
    nbytes, heads = binding.bwd_plan_heads(S, H, KV, d)
    assert heads == H and nbytes > H * per_head
    for fit, chunk in ((16, 16), (15, 8), (8, 8), (7, 4), (4, 4), (3, 2), (2, 2), (1, 1)):
        limit(fit * per_head)
        nbytes, heads = binding.bwd_plan_heads(S, H, KV, d)
        assert heads == chunk, (fit, heads)
        assert chunk * per_head < nbytes < chunk * per_head + (S * H * 4 + (1 << 20)) + \
            2 * 7 * S * KV * d * 4
    limit(per_head - 1)
    nbytes, heads = binding.bwd_plan_heads(S, H, KV, d)
    assert heads == 0 and nbytes < 2 * S * H * 4
    # whole groups of a GQA 4:1 problem, with a smaller last chunk
    limit(9 * causal_pairs(128) * 8192)
    assert binding.bwd_plan_heads(4096, 32, 8, 128)[1] == 8


def test_plan_rejects_bad_shapes():
    for args in ((8, 3, 2, 64), (8, 2, 1, 250), (-1, 2, 1, 64)):
        try:
            binding.bwd_plan(*args)
        except binding.AttnError as e:
            assert e.status in (binding.ATTN_ERR_INVALID_ARG, binding.ATTN_ERR_UNSUPPORTED)
        else:
            raise AssertionError(f"bwd_plan{args} accepted")
    assert binding.bwd_plan(0, 2, 1, 64) == (0, False)
