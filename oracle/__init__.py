"""CPU oracle for causal GQA attention (forward LSE and backward) -- test infrastructure.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product library never loads it, and it shares
no code with the HIP path.  The arithmetic lives in ``attn_oracle.c`` (plain C,
fp64); this module only builds that file and marshals numpy arrays to it.

Definitions followed (page "llm.istanbul -- 10_backward_attention.wgsl",
header comment and kernel attention_backward, Pass A / Pass B / Final):
P = exp(scale*q.k - LSE), dP = dO.v, D = sum_j P*dP, dS = scale*P*(dP - D),
dQ += dS.K, dK += dS^T.Q, dV += P^T.dO summed over each KV group, with key j
visible to query s iff seg[s] <= j <= s.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile attn_oracle.c into liboracle.so next to it (gcc, -O2, no fast-math)."""
    stale = (not os.path.exists(_LIB_PATH)
             or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-pthread",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_attn_fwd_f64.argtypes = [P, P, P, P, P, P, I, I, I, I, ctypes.c_double, I]
    lib.oracle_attn_bwd_f64.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I,
                                        ctypes.c_double, I]
    lib.oracle_attn_bwd_o_f64.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I,
                                          ctypes.c_double, I]
    lib.oracle_attn_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, ctypes.c_float, I]
    lib.oracle_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, ctypes.c_float, I]
    lib.oracle_attn_bwd_o.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, ctypes.c_float, I]
    lib.oracle_attn_bwd_rows.argtypes = [P, P, P, P, P, P, P, I, P, I, P, P, P, I, I, I, I,
                                         ctypes.c_float, I]
    lib.oracle_attn_bwd_rows_o.argtypes = [P, P, P, P, P, P, P, P, I, P, I, P, P, P, I, I, I, I,
                                           ctypes.c_float, I]
    lib.oracle_attn_fwd_rows.argtypes = [P, P, P, P, P, I, P, P, I, I, I, I, ctypes.c_float, I]
    lib.oracle_rope_f64.argtypes = [P, I, I, I, ctypes.c_double, ctypes.c_long, I]
    lib.oracle_attn_bwd_decode_f64.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I,
                                               ctypes.c_double]
    lib.oracle_attn_bwd_decode.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, ctypes.c_float]
    lib.oracle_attn_bwd_rope.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, ctypes.c_float,
                                         ctypes.c_double, ctypes.c_long, I]
    for f in (lib.oracle_attn_fwd_f64, lib.oracle_attn_bwd_f64, lib.oracle_attn_bwd_o_f64,
              lib.oracle_attn_fwd, lib.oracle_attn_bwd, lib.oracle_attn_bwd_o,
              lib.oracle_attn_bwd_rows, lib.oracle_attn_bwd_rows_o, lib.oracle_attn_fwd_rows,
              lib.oracle_rope_f64, lib.oracle_attn_bwd_rope):
        f.restype = I
    _lib = lib
    return lib


class _use_library:
    """Context manager that points this module at another build of the oracle
    (used only by the test that plants mistakes in a copy of attn_oracle.c)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = None
        saved_path = globals()["_LIB_PATH"]
        globals()["_LIB_PATH"] = self.path
        try:
            _load()
        finally:
            globals()["_LIB_PATH"] = saved_path
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _seg(seg, S):
    if seg is None:
        return None
    seg = np.ascontiguousarray(seg, dtype=np.uint32)
    assert seg.shape == (S,)
    return seg


def _dims(Q, K):
    S, H, d = Q.shape
    S2, KV, d2 = K.shape
    assert S == S2 and d == d2, "Q [S,H,d] and K [S,KV,d] disagree"
    return S, H, KV, d


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (status {rc})")


def attn_fwd_f64(Q, K, V, seg, scale, nthreads=0):
    """fp64 forward: returns (O [S,H,d], LSE [S,H]) as float64."""
    Q, K, V = (np.ascontiguousarray(x, dtype=np.float64) for x in (Q, K, V))
    S, H, KV, d = _dims(Q, K)
    seg = _seg(seg, S)
    O = np.zeros((S, H, d), np.float64)
    LSE = np.zeros((S, H), np.float64)
    _check(_load().oracle_attn_fwd_f64(_ptr(Q), _ptr(K), _ptr(V), _ptr(seg), _ptr(O), _ptr(LSE),
                                       S, H, KV, d, float(scale), nthreads), "attn_fwd_f64")
    return O, LSE


def attn_bwd_f64(Q, K, V, dO, LSE, seg, scale, nthreads=0, debug=False, O=None):
    """fp64 backward gradients of this call (no accumulation).

    With ``O`` (the forward output [S,H,d]) the row term is D = dO . O instead
    of sum_j P * dP.  Returns (dQ, dK, dV), plus (D, rowsum_dS) [S,H] when
    ``debug``.
    """
    Q, K, V, dO, LSE = (np.ascontiguousarray(x, dtype=np.float64) for x in (Q, K, V, dO, LSE))
    O = None if O is None else np.ascontiguousarray(O, dtype=np.float64)
    S, H, KV, d = _dims(Q, K)
    seg = _seg(seg, S)
    dQ = np.zeros((S, H, d), np.float64)
    dK = np.zeros((S, KV, d), np.float64)
    dV = np.zeros((S, KV, d), np.float64)
    D = np.zeros((S, H), np.float64)
    rs = np.zeros((S, H), np.float64)
    if O is not None:
        assert O.shape == Q.shape
    _check(_load().oracle_attn_bwd_o_f64(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE),
                                         _ptr(seg), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(D),
                                         _ptr(rs), S, H, KV, d, float(scale), nthreads),
           "attn_bwd_f64")
    if debug:
        return dQ, dK, dV, D, rs
    return dQ, dK, dV


def attn_fwd(Q, K, V, seg, scale, nthreads=0, want_o=True):
    """fp32 forward: returns (O or None, LSE) as float32 (fp64 math, rounded once)."""
    Q, K, V = (np.ascontiguousarray(x, dtype=np.float32) for x in (Q, K, V))
    S, H, KV, d = _dims(Q, K)
    seg = _seg(seg, S)
    O = np.zeros((S, H, d), np.float32) if want_o else None
    LSE = np.zeros((S, H), np.float32)
    _check(_load().oracle_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(seg), _ptr(O), _ptr(LSE),
                                   S, H, KV, d, np.float32(scale), nthreads), "attn_fwd")
    return O, LSE


def rope_f64(X, base, pos_offset, backward):
    """The page's RoPE rotation of interleaved column pairs of X [S, NH, d]
    (forward, or its transpose when ``backward``); returns a new float64 array."""
    X = np.array(X, dtype=np.float64, order="C")
    S, NH, d = X.shape
    _check(_load().oracle_rope_f64(_ptr(X), S, NH, d, float(base), int(pos_offset),
                                   1 if backward else 0), "rope_f64")
    return X


def attn_bwd(Q, K, V, dO, LSE, seg, scale, dQ=None, dK=None, dV=None, nthreads=0, O=None,
             rope=None):
    """fp32 backward with "+=" semantics on dQ, dK, dV (zeros when not given).

    With ``O`` (the forward output) the row term is D = dO . O.  With ``rope``
    = (base, pos_offset) the page's RoPE backward then rotates dQ and dK in
    place (Q, K are the rotated inputs).  Returns the (updated) float32
    arrays (dQ, dK, dV).
    """
    Q, K, V, dO, LSE = (np.ascontiguousarray(x, dtype=np.float32) for x in (Q, K, V, dO, LSE))
    O = None if O is None else np.ascontiguousarray(O, dtype=np.float32)
    S, H, KV, d = _dims(Q, K)
    seg = _seg(seg, S)
    dQ = np.zeros((S, H, d), np.float32) if dQ is None else np.array(dQ, np.float32, order="C")
    dK = np.zeros((S, KV, d), np.float32) if dK is None else np.array(dK, np.float32, order="C")
    dV = np.zeros((S, KV, d), np.float32) if dV is None else np.array(dV, np.float32, order="C")
    if O is not None:
        assert O.shape == Q.shape
    if rope is not None:
        _check(_load().oracle_attn_bwd_rope(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                                            _ptr(LSE), _ptr(seg), _ptr(dQ), _ptr(dK), _ptr(dV),
                                            S, H, KV, d, np.float32(scale), float(rope[0]),
                                            int(rope[1]), nthreads), "attn_bwd_rope")
        return dQ, dK, dV
    _check(_load().oracle_attn_bwd_o(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE),
                                     _ptr(seg), _ptr(dQ), _ptr(dK), _ptr(dV), S, H, KV, d,
                                     np.float32(scale), nthreads), "attn_bwd")
    return dQ, dK, dV


def _decode_dims(q, K, P):
    H, d = q.shape
    T, KV, d2 = K.shape
    assert d == d2 and P.shape == (H, T), "q [H,d], K [T,KV,d], P [H,T] disagree"
    return T, H, KV, d


def attn_bwd_decode_f64(q, K, V, P, dO, scale, debug=False):
    """Single-query backward over a KV history (page "rullama 0.5.0", pass 1
    and 2 of 2), fp64, no accumulation: q, dO [H,d]; K, V [T,KV,d]; P the
    forward's probabilities [H,T].  Returns (dq, dK, dV), plus the score
    gradients dS [H,T] when ``debug``."""
    q, K, V, P, dO = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, K, V, P, dO))
    T, H, KV, d = _decode_dims(q, K, P)
    dq = np.zeros((H, d), np.float64)
    dK = np.zeros((T, KV, d), np.float64)
    dV = np.zeros((T, KV, d), np.float64)
    dS = np.zeros((H, T), np.float64)
    _check(_load().oracle_attn_bwd_decode_f64(_ptr(q), _ptr(K), _ptr(V), _ptr(P), _ptr(dO),
                                              _ptr(dq), _ptr(dK), _ptr(dV), _ptr(dS), T, H, KV,
                                              d, float(scale)), "attn_bwd_decode_f64")
    return (dq, dK, dV, dS) if debug else (dq, dK, dV)


def attn_bwd_decode(q, K, V, P, dO, scale, dq=None, dK=None, dV=None):
    """fp32 single-query backward with "+=" semantics (zeros when not given);
    returns the (updated) float32 arrays (dq, dK, dV)."""
    q, K, V, P, dO = (np.ascontiguousarray(x, dtype=np.float32) for x in (q, K, V, P, dO))
    T, H, KV, d = _decode_dims(q, K, P)
    dq = np.zeros((H, d), np.float32) if dq is None else np.array(dq, np.float32, order="C")
    dK = np.zeros((T, KV, d), np.float32) if dK is None else np.array(dK, np.float32, order="C")
    dV = np.zeros((T, KV, d), np.float32) if dV is None else np.array(dV, np.float32, order="C")
    _check(_load().oracle_attn_bwd_decode(_ptr(q), _ptr(K), _ptr(V), _ptr(P), _ptr(dO), _ptr(dq),
                                          _ptr(dK), _ptr(dV), T, H, KV, d, np.float32(scale)),
           "attn_bwd_decode")
    return dq, dK, dV


def attn_bwd_rows(Q, K, V, dO, LSE, seg, scale, q_rows, k_rows, nthreads=0, O=None):
    """fp64 gradients for selected rows only (with ``O``: D = dO . O).

    Returns (dQ_sel [nq,H,d], dK_sel [nk,KV,d], dV_sel [nk,KV,d]).
    """
    Q, K, V, dO, LSE = (np.ascontiguousarray(x, dtype=np.float32) for x in (Q, K, V, dO, LSE))
    O = None if O is None else np.ascontiguousarray(O, dtype=np.float32)
    S, H, KV, d = _dims(Q, K)
    seg = _seg(seg, S)
    q_rows = np.ascontiguousarray(q_rows, dtype=np.int32)
    k_rows = np.ascontiguousarray(k_rows, dtype=np.int32)
    dQ = np.zeros((len(q_rows), H, d), np.float64)
    dK = np.zeros((len(k_rows), KV, d), np.float64)
    dV = np.zeros((len(k_rows), KV, d), np.float64)
    if O is not None:
        assert O.shape == Q.shape
    _check(_load().oracle_attn_bwd_rows_o(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE),
                                          _ptr(seg), _ptr(q_rows), len(q_rows), _ptr(k_rows),
                                          len(k_rows), _ptr(dQ), _ptr(dK), _ptr(dV), S, H, KV, d,
                                          np.float32(scale), nthreads), "attn_bwd_rows")
    return dQ, dK, dV


def attn_fwd_rows(Q, K, V, seg, scale, rows, nthreads=0, want_o=False):
    """fp32 forward for selected query rows: returns (O_sel or None, LSE_sel [n,H])."""
    Q, K, V = (np.ascontiguousarray(x, dtype=np.float32) for x in (Q, K, V))
    S, H, KV, d = _dims(Q, K)
    seg = _seg(seg, S)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    O = np.zeros((len(rows), H, d), np.float32) if want_o else None
    LSE = np.zeros((len(rows), H), np.float32)
    _check(_load().oracle_attn_fwd_rows(_ptr(Q), _ptr(K), _ptr(V), _ptr(seg), _ptr(rows),
                                        len(rows), _ptr(O), _ptr(LSE), S, H, KV, d,
                                        np.float32(scale), nthreads), "attn_fwd_rows")
    return O, LSE


def rows_needed(seg, S, q_rows, k_rows):
    """Query rows whose LSE the selected-row backward reads: the selected query
    rows plus every query that sees one of the selected keys."""
    segv = np.zeros(S, np.int64) if seg is None else np.asarray(seg, np.int64)
    need = np.zeros(S, bool)
    need[np.asarray(q_rows, np.int64)] = True
    s = np.arange(S)
    for j in np.asarray(k_rows, np.int64):
        need |= (s >= j) & (segv <= j)
    return np.nonzero(need)[0].astype(np.int32)
