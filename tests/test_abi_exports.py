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
