"""The C-ABI library loads and exports every entry point include/attnbwd.h
declares (no compute call: this runs without a GPU)."""
import ctypes
import os
import re

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


def test_plan_sizes_the_workspace(monkeypatch):
    # host-only query: D [S,H], block metadata, and the P / P*dP tile scratch
    # (two 32x32 fp32 tiles per (query block, key block, head) of the causal
    # triangle), each part 256-byte aligned, then -- the most a call takes is
    # an unpaired one -- the partial dK, dV of the key-major head splits: 64
    # key tiles x 8 KV heads = 512 workgroups, so the 4 heads of a group go
    # to 2 workgroups; the first adds into dK, dV, the second writes an
    # [S, KV, d] slice of dK and one of dV
    monkeypatch.delenv("ATTNBWD_SCRATCH_MB", raising=False)
    S, H = 4096, 32
    nblk = S // 32
    meta = up(up(up(S * H * 4) + 2 * nblk * 4) + (nblk + 1) * 8)
    part = 2 * 1 * S * 8 * 128 * 4
    assert binding.bwd_plan(S, H, 8, 128) == (meta + causal_pairs(nblk) * H * 8192 + part, True)
    # a group of one head cannot split
    assert binding.bwd_plan(S, 8, 8, 128) == (
        up(up(up(S * 8 * 4) + 2 * nblk * 4) + (nblk + 1) * 8) + causal_pairs(nblk) * 8 * 8192, True)
    monkeypatch.setenv("ATTNBWD_SCRATCH_MB", "0")
    assert binding.bwd_plan(S, H, 8, 128) == (meta, False)


def test_plan_recomputes_above_the_budget(monkeypatch):
    # 16384 rows, 16 heads: the tiles need 16.03 GiB, within the default
    # budget; a smaller budget switches to recomputed scores
    monkeypatch.delenv("ATTNBWD_SCRATCH_MB", raising=False)
    S, H = 16384, 16
    need = causal_pairs(S // 32) * H * 8192
    nbytes, stored = binding.bwd_plan(S, H, 2, 256)
    assert stored and nbytes > need
    monkeypatch.setenv("ATTNBWD_SCRATCH_MB", repr(need / 2**20))
    assert binding.bwd_plan(S, H, 2, 256)[1]
    monkeypatch.setenv("ATTNBWD_SCRATCH_MB", repr((need - 1) / 2**20))
    nbytes, stored = binding.bwd_plan(S, H, 2, 256)
    assert not stored and nbytes < 2 * S * H * 4


def test_plan_rejects_bad_shapes():
    for args in ((8, 3, 2, 64), (8, 2, 1, 250), (-1, 2, 1, 64)):
        try:
            binding.bwd_plan(*args)
        except binding.AttnError as e:
            assert e.status in (binding.ATTN_ERR_INVALID_ARG, binding.ATTN_ERR_UNSUPPORTED)
        else:
            raise AssertionError(f"bwd_plan{args} accepted")
    assert binding.bwd_plan(0, 2, 1, 64) == (0, False)
