"""Thin ctypes binding over libattnbwd.so (C ABI declared in include/attnbwd.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattnbwd.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
EXPORTED = ("attn_bwd", "attn_bwd_decode", "attn_bwd_f16", "attn_bwd_f16_rope", "attn_bwd_noalloc",
            "attn_bwd_o",
            "attn_bwd_plan",
            "attn_bwd_rope", "attn_bwd_short", "attn_fwd_lse", "attn_last_error",
            "attn_profile_begin", "attn_profile_end", "attn_set_scratch_limit")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str, msg: str):
        super().__init__(f"{what} failed with status {status}: {msg}")
        self.status = status


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, P]
    lib.attn_bwd.restype = I
    lib.attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, P]
    lib.attn_bwd_noalloc.restype = I
    lib.attn_bwd_o.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, P]
    lib.attn_bwd_o.restype = I
    lib.attn_bwd_rope.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, F, I, P]
    lib.attn_bwd_rope.restype = I
    lib.attn_bwd_f16.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, P]
    lib.attn_bwd_f16.restype = I
    lib.attn_bwd_f16_rope.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, F, I, P]
    lib.attn_bwd_f16_rope.restype = I
    lib.attn_bwd_short.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, P]
    lib.attn_bwd_short.restype = I
    lib.attn_bwd_decode.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, F, P]
    lib.attn_bwd_decode.restype = I
    lib.attn_bwd_plan.argtypes = [I, I, I, I, ctypes.POINTER(ctypes.c_size_t),
                                  ctypes.POINTER(ctypes.c_int)]
    lib.attn_bwd_plan.restype = I
    lib.attn_set_scratch_limit.argtypes = [ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_set_scratch_limit.restype = I
    lib.attn_fwd_lse.argtypes = [P, P, P, P, P, P, I, I, I, I, F, P]
    lib.attn_fwd_lse.restype = I
    lib.attn_profile_begin.argtypes = []
    lib.attn_profile_begin.restype = I
    lib.attn_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    lib.attn_profile_end.restype = I
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().attn_last_error().decode()


def _raise_on(status: int, what: str):
    if status != ATTN_OK:
        raise AttnError(status, what, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check_tensors(named, dev):
    """Every tensor must be a contiguous GPU tensor of an accepted dtype on the
    current HIP device: the C ABI takes device pointers, and a host pointer
    handed to a kernel would fault the GPU.  Raises ValueError before any
    launch otherwise."""
    import torch
    for name, t, dtypes in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} is on {t.device}: the library takes GPU tensors only")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
        if t.dtype not in dtypes:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _device_of(first):
    """The device every tensor of a call must be on: the current HIP device
    (kernels are launched there), checked against the first tensor's."""
    import torch
    if first.device.type != "cuda":
        raise ValueError(f"tensors are on {first.device}: the library takes GPU tensors only")
    cur = torch.device("cuda", torch.cuda.current_device())
    if first.device != cur:
        raise ValueError(f"tensors are on {first.device} but the current device is {cur}")
    return cur


def _dims(Q, K):
    if Q.dim() != 3 or K.dim() != 3:
        raise ValueError("Q must be [S, H, d] and K [S, KV, d]")
    S, H, d = Q.shape
    if K.shape[0] != S or K.shape[2] != d:
        raise ValueError(f"Q {tuple(Q.shape)} and K {tuple(K.shape)} disagree")
    return S, H, K.shape[1], d


def _bwd_args(Q, K, V, O, dO, LSE, seg, dQ, dK, dV):
    import torch
    S, H, KV, d = _dims(Q, K)
    f32 = (torch.float32,)
    _check_tensors([("Q", Q, f32), ("K", K, f32), ("V", V, f32), ("O", O, f32), ("dO", dO, f32),
                    ("LSE", LSE, f32), ("seg", seg, (torch.int32, torch.uint32)),
                    ("dQ", dQ, f32), ("dK", dK, f32), ("dV", dV, f32)], _device_of(Q))
    for name, t, shape in (("V", V, K.shape), ("O", O, Q.shape), ("dO", dO, Q.shape),
                           ("LSE", LSE, (S, H)), ("dQ", dQ, Q.shape), ("dK", dK, K.shape),
                           ("dV", dV, K.shape)):
        if t is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if seg is not None and tuple(seg.shape) != (S,):
        raise ValueError(f"seg has shape {tuple(seg.shape)}, expected ({S},)")
    return S, H, KV, d


def attn_bwd(Q, K, V, dO, LSE, seg, dQ, dK, dV, scale, stream=None):
    """dQ += ..., dK += ..., dV += ... (the C ABI's attn_bwd) on torch device tensors.

    Q, dO, dQ [S,H,d]; K, V, dK, dV [S,KV,d]; LSE [S,H] float32; seg [S]
    int32/uint32 document starts or None (plain causal).
    """
    S, H, KV, d = _bwd_args(Q, K, V, None, dO, LSE, seg, dQ, dK, dV)
    st = load().attn_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(LSE), _ptr(seg),
                         _ptr(dQ), _ptr(dK), _ptr(dV), S, H, KV, d, float(scale),
                         _stream(stream))
    _raise_on(st, "attn_bwd")


def attn_bwd_noalloc(Q, K, V, dO, LSE, seg, dQ, dK, dV, scale, stream=None):
    """attn_bwd on the library's fixed 32 MiB device workspace, allocating
    nothing (the C ABI's attn_bwd_noalloc); calls that overlap on one device
    race on that workspace."""
    S, H, KV, d = _bwd_args(Q, K, V, None, dO, LSE, seg, dQ, dK, dV)
    st = load().attn_bwd_noalloc(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(LSE), _ptr(seg),
                                 _ptr(dQ), _ptr(dK), _ptr(dV), S, H, KV, d, float(scale),
                                 _stream(stream))
    _raise_on(st, "attn_bwd_noalloc")


def attn_bwd_o(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, scale, stream=None):
    """attn_bwd with the forward output O [S,H,d] given (the C ABI's attn_bwd_o):
    the row term is read off it, D = dO . O."""
    if O is None:
        raise ValueError("attn_bwd_o needs the forward output O")
    S, H, KV, d = _bwd_args(Q, K, V, O, dO, LSE, seg, dQ, dK, dV)
    st = load().attn_bwd_o(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(seg),
                           _ptr(dQ), _ptr(dK), _ptr(dV), S, H, KV, d, float(scale),
                           _stream(stream))
    _raise_on(st, "attn_bwd_o")


def attn_bwd_rope(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, scale, rope_base, pos_offset,
                  stream=None):
    """attn_bwd (O None) or attn_bwd_o (O given), then the RoPE backward on dQ and
    dK fused into the write-back (the C ABI's attn_bwd_rope): dQ <- R^T(dQ + g)."""
    S, H, KV, d = _bwd_args(Q, K, V, O, dO, LSE, seg, dQ, dK, dV)
    st = load().attn_bwd_rope(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(seg),
                              _ptr(dQ), _ptr(dK), _ptr(dV), S, H, KV, d, float(scale),
                              float(rope_base), int(pos_offset), _stream(stream))
    _raise_on(st, "attn_bwd_rope")


def attn_bwd_f16(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, scale, stream=None):
    """The backward with fp16 matrix-core operands and fp32 accumulation (the C
    ABI's attn_bwd_f16); O is the forward output or None (row term computed)."""
    S, H, KV, d = _bwd_args(Q, K, V, O, dO, LSE, seg, dQ, dK, dV)
    st = load().attn_bwd_f16(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(seg),
                             _ptr(dQ), _ptr(dK), _ptr(dV), S, H, KV, d, float(scale),
                             _stream(stream))
    _raise_on(st, "attn_bwd_f16")


def attn_bwd_f16_rope(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, scale, rope_base, pos_offset,
                      stream=None):
    """attn_bwd_f16 with the RoPE backward on dQ and dK fused into the
    write-back (the C ABI's attn_bwd_f16_rope): dQ <- R^T(dQ + g)."""
    S, H, KV, d = _bwd_args(Q, K, V, O, dO, LSE, seg, dQ, dK, dV)
    st = load().attn_bwd_f16_rope(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE),
                                  _ptr(seg), _ptr(dQ), _ptr(dK), _ptr(dV), S, H, KV, d,
                                  float(scale), float(rope_base), int(pos_offset),
                                  _stream(stream))
    _raise_on(st, "attn_bwd_f16_rope")


def attn_bwd_short(Q, K, V, O, dO, LSE, seg, dQ, dK, dV, scale, stream=None):
    """The short-sequence backward (the C ABI's attn_bwd_short; seq_len <= 1024,
    head_dim <= 128): one launch when O (the forward output) is given, two when
    O is None."""
    S, H, KV, d = _bwd_args(Q, K, V, O, dO, LSE, seg, dQ, dK, dV)
    st = load().attn_bwd_short(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(seg),
                               _ptr(dQ), _ptr(dK), _ptr(dV), S, H, KV, d, float(scale),
                               _stream(stream))
    _raise_on(st, "attn_bwd_short")


def attn_bwd_decode(q, K, V, P, dO, dq, dK, dV, scale, stream=None):
    """Single-query backward over a KV history (the C ABI's attn_bwd_decode):
    q, dO, dq [H,d]; K, V, dK, dV [T,KV,d]; P [H,T] the forward's
    probabilities; dq, dK, dV accumulate."""
    import torch
    H, d = q.shape
    T, KV, d2 = K.shape
    if d2 != d:
        raise ValueError(f"q {tuple(q.shape)} and K {tuple(K.shape)} disagree")
    f32 = (torch.float32,)
    _check_tensors([("q", q, f32), ("K", K, f32), ("V", V, f32), ("P", P, f32), ("dO", dO, f32),
                    ("dq", dq, f32), ("dK", dK, f32), ("dV", dV, f32)], _device_of(q))
    for name, t, shape in (("V", V, K.shape), ("P", P, (H, T)), ("dO", dO, q.shape),
                           ("dq", dq, q.shape), ("dK", dK, K.shape), ("dV", dV, K.shape)):
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    st = load().attn_bwd_decode(_ptr(q), _ptr(K), _ptr(V), _ptr(P), _ptr(dO), _ptr(dq), _ptr(dK),
                                _ptr(dV), T, H, KV, d, float(scale), _stream(stream))
    _raise_on(st, "attn_bwd_decode")


def attn_fwd_lse(Q, K, V, seg, O, LSE, scale, stream=None):
    """O, LSE = forward of the masked attention (the C ABI's attn_fwd_lse); O may be None."""
    import torch
    S, H, KV, d = _dims(Q, K)
    f32 = (torch.float32,)
    _check_tensors([("Q", Q, f32), ("K", K, f32), ("V", V, f32),
                    ("seg", seg, (torch.int32, torch.uint32)), ("O", O, f32), ("LSE", LSE, f32)],
                   _device_of(Q))
    if tuple(LSE.shape) != (S, H) or (O is not None and tuple(O.shape) != tuple(Q.shape)):
        raise ValueError("O must be [S,H,d] and LSE [S,H]")
    st = load().attn_fwd_lse(_ptr(Q), _ptr(K), _ptr(V), _ptr(seg), _ptr(O), _ptr(LSE),
                             S, H, KV, d, float(scale), _stream(stream))
    _raise_on(st, "attn_fwd_lse")


def bwd_plan_heads(seq_len, n_heads, n_kv_heads, head_dim):
    """(workspace bytes, heads per stored-tile chunk) of one attn_bwd call; 0
    heads: the key-major pass recomputes the scores (nothing stored)."""
    nbytes = ctypes.c_size_t(0)
    heads = ctypes.c_int(0)
    _raise_on(load().attn_bwd_plan(seq_len, n_heads, n_kv_heads, head_dim, ctypes.byref(nbytes),
                                   ctypes.byref(heads)), "attn_bwd_plan")
    return int(nbytes.value), int(heads.value)


def bwd_plan(seq_len, n_heads, n_kv_heads, head_dim):
    """(workspace bytes, stored probability tiles?) of one attn_bwd call."""
    nbytes, heads = bwd_plan_heads(seq_len, n_heads, n_kv_heads, head_dim)
    return nbytes, heads > 0


def set_scratch_limit(nbytes):
    """Set the most bytes of stored probability tiles one call may take
    (process-wide; the C ABI's attn_set_scratch_limit).  Returns the previous
    limit."""
    prev = ctypes.c_size_t(0)
    _raise_on(load().attn_set_scratch_limit(int(nbytes), ctypes.byref(prev)),
              "attn_set_scratch_limit")
    return int(prev.value)


class scratch_limit:
    """Context manager: run a block with another scratch limit, then restore it."""

    def __init__(self, nbytes):
        self.nbytes = int(nbytes)

    def __enter__(self):
        self.prev = set_scratch_limit(self.nbytes)
        return self

    def __exit__(self, *exc):
        set_scratch_limit(self.prev)
        return False


def profile_begin():
    """Start recording per-kernel HIP events inside attn_bwd (calling thread only)."""
    _raise_on(load().attn_profile_begin(), "attn_profile_begin")


def profile_end():
    """Stop recording; returns (ms of the query-major pass, of the key-major pass,
    of the dQ pass, n_calls), the times summed over the recorded calls."""
    ms = (ctypes.c_double * 3)()
    n = ctypes.c_int(0)
    _raise_on(load().attn_profile_end(ms, ctypes.byref(n)), "attn_profile_end")
    return float(ms[0]), float(ms[1]), float(ms[2]), int(n.value)
