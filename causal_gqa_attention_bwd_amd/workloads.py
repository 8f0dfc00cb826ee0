"""Seeded synthetic inputs for the five attention-backward workloads.

This module only draws random tensors and lays out documents; it holds none
of the attention arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it.

Recipe (numpy PCG64, ``default_rng(1000 + workload id)``): draw Q [S,H,d],
K [S,KV,d], V [S,KV,d], dO [S,H,d] as float32 standard normals in that order
(the S=4096 workload scales dO by 0.1 in float32), then the document layout.
``seg[s]`` is the index of the first token of the document holding token s,
so key j is visible to query s iff seg[s] <= j <= s.  scale = float32(1/sqrt(d)).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    S: int
    H: int
    KV: int
    d: int
    docs: str          # "single" | "split" | "uniform" | "geometric"
    do_std: float = 1.0

    @property
    def scale(self) -> np.float32:
        return np.float32(1.0 / np.sqrt(self.d))


WORKLOADS = {
    1: Workload(1, "s64_h2_kv1_d16_causal", 64, 2, 1, 16, "single"),
    2: Workload(2, "s512_h4_kv2_d32_two_docs", 512, 4, 2, 32, "split"),
    3: Workload(3, "s1024_h8_kv8_d64_docs_u64_512", 1024, 8, 8, 64, "uniform"),
    4: Workload(4, "s4096_h32_kv8_d128_causal", 4096, 32, 8, 128, "single", 0.1),
    5: Workload(5, "s16384_h16_kv2_d256_docs_geom2048", 16384, 16, 2, 256, "geometric"),
    # the S=4096 workload's heads at eight times the length: its stored tiles
    # (137 GB for all heads) exceed any scratch limit, so it measures the head
    # chunks; not one of the five parity workloads
    6: Workload(6, "s32768_h32_kv8_d128_causal", 32768, 32, 8, 128, "single", 0.1),
}


def seg_from_lengths(lengths, S: int) -> np.ndarray:
    """Lay documents of the given lengths out from token 0, truncating the last at S."""
    seg = np.zeros(S, dtype=np.uint32)
    start = 0
    for L in lengths:
        if start >= S:
            break
        end = min(S, start + int(L))
        seg[start:end] = start
        start = end
    if start < S:  # lengths ran out: the rest is one more document
        seg[start:] = start
    return seg


def draw_lengths(rng: np.random.Generator, S: int, kind: str) -> list:
    """Document lengths until they cover S tokens (the last one is truncated by the caller)."""
    out, total = [], 0
    while total < S:
        if kind == "uniform":
            L = int(rng.integers(64, 513))          # U{64..512}
        elif kind == "geometric":
            L = 15 + int(rng.geometric(1.0 / 2033))  # min 16, mean 2048
        else:
            raise ValueError(kind)
        out.append(L)
        total += L
    return out


def make_seg(rng: np.random.Generator, w: Workload) -> np.ndarray:
    if w.docs == "single":
        return np.zeros(w.S, dtype=np.uint32)
    if w.docs == "split":
        p = int(rng.integers(64, 449))               # U{64..448}
        return seg_from_lengths([p, w.S - p], w.S)
    return seg_from_lengths(draw_lengths(rng, w.S, w.docs), w.S)


def make_inputs(wid: int, seed: int | None = None) -> dict:
    """Q, K, V, dO (float32), seg (uint32) and scale (float32) of one workload."""
    w = WORKLOADS[wid]
    rng = np.random.default_rng(1000 + wid if seed is None else seed)
    Q = rng.standard_normal((w.S, w.H, w.d), dtype=np.float32)
    K = rng.standard_normal((w.S, w.KV, w.d), dtype=np.float32)
    V = rng.standard_normal((w.S, w.KV, w.d), dtype=np.float32)
    dO = rng.standard_normal((w.S, w.H, w.d), dtype=np.float32)
    if w.do_std != 1.0:
        dO *= np.float32(w.do_std)
    seg = make_seg(rng, w)
    return dict(Q=Q, K=K, V=V, dO=dO, seg=seg, scale=w.scale, workload=w)


def random_problem(rng: np.random.Generator, S: int, H: int, KV: int, d: int,
                   seg=None, dtype=np.float32) -> dict:
    """Small ad-hoc problem for tests: N(0,1) tensors and the given (or causal) seg."""
    Q = rng.standard_normal((S, H, d)).astype(dtype)
    K = rng.standard_normal((S, KV, d)).astype(dtype)
    V = rng.standard_normal((S, KV, d)).astype(dtype)
    dO = rng.standard_normal((S, H, d)).astype(dtype)
    seg = np.zeros(S, np.uint32) if seg is None else np.asarray(seg, np.uint32)
    return dict(Q=Q, K=K, V=V, dO=dO, seg=seg, scale=np.float32(1.0 / np.sqrt(d)))


# The single-query (decode-step) backward over a KV history: one query per head
# and a history of T keys, with the forward's probabilities given.  Llama-like
# heads (32 query heads in 8 KV groups of 128 columns) over a 32768-position
# history.
DECODE_WORKLOAD = dict(name="decode_t32768_h32_kv8_d128", T=32768, H=32, KV=8, d=128)


def make_decode_inputs(T: int, H: int, KV: int, d: int, seed: int = 1100) -> dict:
    """q, dO [H,d], K, V [T,KV,d] float32 standard normals (drawn in that order
    from ``default_rng(seed)``), and probabilities P [H,T]: each row
    normalises exp of standard-normal logits (the diffuse attention of an
    untrained model), in float64 then rounded to float32.  scale = 1/sqrt(d)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d)).astype(np.float32)
    K = rng.standard_normal((T, KV, d)).astype(np.float32)
    V = rng.standard_normal((T, KV, d)).astype(np.float32)
    dO = rng.standard_normal((H, d)).astype(np.float32)
    e = np.exp(rng.standard_normal((H, T)))
    P = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return dict(q=q, K=K, V=V, dO=dO, P=P, scale=np.float32(1.0 / np.sqrt(d)))
