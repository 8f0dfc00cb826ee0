#!/usr/bin/env python3
"""Benchmark of the attention backward on one MI355X.

One step = one attn_bwd call (the whole hot path: the small block-metadata
kernel; the query-major pass, which forms P, P*dP and the row term D and
stores the tiles; the key-major dK/dV pass, which also forms dS; the dQ pass)
on the S=4096, H=32, KV=8, d=128 plain-causal workload, fp32 inputs already
resident in HBM.  The LSE
input is produced beforehand on the GPU by attn_fwd_lse (untimed).

Metric: credited TFLOP/s = 10 * d * H * N_valid / time per step, where
N_valid is the number of visible (query, key) pairs (five contractions of 2*d
flops per visible pair and head).  Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_MFMA = 157.3   # TFLOP/s, MI355X dense fp32 matrix
PEAK_FP16_MFMA = 2516.6  # TFLOP/s, MI355X dense fp16/bf16 matrix
PEAK_HBM = 8.0           # TB/s
CSRC = os.path.join(ROOT, "causal_gqa_attention_bwd_amd", "csrc")
F16_KERNELS = ("k_cvt16", "k_kv16", "k_q16", "k_dqs16")
DEC_KERNELS = ("k_dec_dp", "k_dec_kv", "k_dec_dq")
SHORT_KERNELS = ("k_short", "k_short_rowterm")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def valid_pairs(seg):
    import numpy as np
    s = np.arange(len(seg), dtype=np.int64)
    return int(np.sum(np.maximum(s - np.asarray(seg, np.int64) + 1, 0)))


def source_sha(kname):
    """Hash of the source file holding kernel `kname` and the shared header."""
    base = kname.split("<")[0]
    src = ("attnbwd_f16.hip" if base in F16_KERNELS else
           "attnbwd_decode.hip" if base in DEC_KERNELS else
           "attnbwd_short.hip" if base in SHORT_KERNELS else "attnbwd.hip")
    h = hashlib.sha256()
    for name in (src, "common.h"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kname, workload):
    """HBM bytes per launch of kernel `kname` on `workload` from the committed
    rocprofv3 counter summary, or None when it is missing or was taken on a
    different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kname}_{workload}_traffic.txt")
    if not os.path.exists(path):
        log(f"traffic: no counter summary {path}; reporting null")
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_sha(kname):
        log(f"traffic: {path} was taken on another kernel source; reporting null")
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(x, groups, with_o=False, rope=None):
    """The oracle's backward on a bounded sample (the first `groups` KV groups:
    all S rows, `groups` KV heads and their query heads), timed on host cores.
    Returns (the baseline record, the sample's inputs with the oracle's LSE
    (and O when with_o), the oracle's gradients of the sample)."""
    import numpy as np
    import oracle
    w = x["workload"]
    g = w.H // w.KV
    groups = min(groups, w.KV)
    nh = g * groups
    Q = np.ascontiguousarray(x["Q"][:, :nh])
    dO = np.ascontiguousarray(x["dO"][:, :nh])
    K = np.ascontiguousarray(x["K"][:, :groups])
    V = np.ascontiguousarray(x["V"][:, :groups])
    # the machine's CPU share for one GPU is 16 threads (its OMP_NUM_THREADS)
    threads = min(16, len(os.sched_getaffinity(0)))
    O, lse = oracle.attn_fwd(Q, K, V, x["seg"], x["scale"], nthreads=threads, want_o=with_o)
    t0 = time.perf_counter()
    ref = oracle.attn_bwd(Q, K, V, dO, lse, x["seg"], x["scale"], nthreads=threads, O=O,
                          rope=rope)
    dt = time.perf_counter() - t0
    flops = 10.0 * w.d * nh * valid_pairs(x["seg"])
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"oracle attn_bwd (fp64 C, {threads} threads) on KV heads 0..{groups - 1} "
                     f"({nh} of {w.H} query heads, all {w.S} rows) of the same workload; "
                     f"{dt:.2f} s wall; {cpu_model}",
           "seconds": dt}
    sample = dict(Q=Q, K=K, V=V, dO=dO, seg=x["seg"], scale=x["scale"], LSE=lse, O=O)
    return rec, sample, ref


def parity_errors(sample, ref, entry, with_o, rope=None):
    """The timed entry once more on the oracle's sample, on zeroed outputs and
    the oracle's LSE (and O): max|gpu - oracle| / max|oracle| per gradient."""
    import numpy as np
    import torch
    from causal_gqa_attention_bwd_amd import binding
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(np.ascontiguousarray(sample[k])).to(dev)
         for k in ("Q", "K", "V", "dO", "LSE")}
    O = torch.from_numpy(sample["O"]).to(dev) if with_o else None
    seg = (None if not np.any(sample["seg"]) else
           torch.from_numpy(sample["seg"].astype(np.int32)).to(dev))
    out = [torch.zeros_like(t["Q"]), torch.zeros_like(t["K"]), torch.zeros_like(t["V"])]
    sc = float(sample["scale"])
    args = (t["Q"], t["K"], t["V"])
    if entry == "attn_bwd":
        binding.attn_bwd(*args, t["dO"], t["LSE"], seg, *out, sc)
    elif entry == "attn_bwd_o":
        binding.attn_bwd_o(*args, O, t["dO"], t["LSE"], seg, *out, sc)
    elif entry.endswith("_rope"):
        getattr(binding, entry)(*args, O, t["dO"], t["LSE"], seg, *out, sc, rope[0], rope[1])
    else:
        getattr(binding, entry)(*args, O, t["dO"], t["LSE"], seg, *out, sc)
    torch.cuda.synchronize()
    errs = {}
    for name, g, r in zip(("dQ", "dK", "dV"), out, ref):
        g = g.cpu().numpy().astype(np.float64)
        errs[name] = float(np.max(np.abs(g - r))) / max(float(np.max(np.abs(r))), 1e-30)
    return errs


def time_entry(wid, entry, with_o, steps, warmup, calib_copy_mb):
    """Time `steps` calls of one backward entry on workload `wid` (inputs in
    HBM, LSE and O from attn_fwd_lse beforehand, untimed) between HIP events;
    the library's measurement hooks give each pass's device time.  Returns the
    figures of the step and of its dominant kernel."""
    import numpy as np
    import torch

    from causal_gqa_attention_bwd_amd import binding
    from causal_gqa_attention_bwd_amd.workloads import make_inputs

    dev = torch.device("cuda:0")
    x = make_inputs(wid)
    w = x["workload"]
    log(f"bench: workload {w.name}: S={w.S} H={w.H} KV={w.KV} d={w.d}, {entry}")
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev) for k in ("Q", "K", "V", "dO")}
    seg_np = x["seg"]
    seg = None if not np.any(seg_np) else torch.from_numpy(seg_np.astype(np.int32)).to(dev)
    scale = float(x["scale"])
    lse = torch.empty((w.S, w.H), dtype=torch.float32, device=dev)
    O = torch.empty_like(t["Q"]) if with_o else None
    binding.attn_fwd_lse(t["Q"], t["K"], t["V"], seg, O, lse, scale)
    ws_bytes, heads = binding.bwd_plan_heads(w.S, w.H, w.KV, w.d)
    stored = heads > 0
    dpad = next(p for p in (32, 64, 96, 128, 192, 256) if p >= w.d)
    f16_ws = (2 * w.H + 2 * w.KV) * ((w.S + 127) // 128 * 128) * dpad * 2 + 2 * w.S * w.H * 4
    # the fp16 path's stored dS/scale tiles (2 KiB per slot of the causal
    # bound and head), when they fit the library's current scratch limit
    # (read back by setting it to itself)
    nblk = (w.S + 31) // 32
    ds_bytes = nblk * (nblk + 1) // 2 * w.H * 2048
    limit = binding.set_scratch_limit(0)
    binding.set_scratch_limit(limit)
    ds_stored = ds_bytes <= limit
    if ds_stored:
        f16_ws += ds_bytes
    if entry.startswith("attn_bwd_f16"):
        log(f"bench: {entry}, workspace {f16_ws / 2**30:.2f} GiB (fp16 copies"
            + (", stored dS tiles)" if ds_stored else "; dS formed again by the query-major pass)"))
    elif entry != "attn_bwd_short":
        log(f"bench: workspace at most {ws_bytes / 2**30:.2f} GiB (attn_bwd_plan), "
            + (f"stored probability tiles for {heads} heads at a time" if stored
               else "recomputed probability tiles"))
    dQ = torch.zeros_like(t["Q"])
    dK = torch.zeros_like(t["K"])
    dV = torch.zeros_like(t["V"])
    torch.cuda.synchronize()
    a = (t["Q"], t["K"], t["V"])

    def step():
        if entry == "attn_bwd":
            binding.attn_bwd(*a, t["dO"], lse, seg, dQ, dK, dV, scale)
        elif entry == "attn_bwd_o":
            binding.attn_bwd_o(*a, O, t["dO"], lse, seg, dQ, dK, dV, scale)
        elif entry.endswith("_rope"):
            getattr(binding, entry)(*a, O, t["dO"], lse, seg, dQ, dK, dV, scale, 10000.0, 0)
        else:
            getattr(binding, entry)(*a, O, t["dO"], lse, seg, dQ, dK, dV, scale)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    calibration_copy(calib_copy_mb, dev)

    binding.profile_begin()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_q, ms_k, ms_s, ncalls = binding.profile_end()
    ms_step = e0.elapsed_time(e1) / steps
    assert ncalls == steps, (ncalls, steps)
    if not (torch.isfinite(dQ).all() and torch.isfinite(dK).all() and torch.isfinite(dV).all()):
        raise RuntimeError("non-finite gradients")

    npairs = valid_pairs(seg_np)
    flops = 10.0 * w.d * w.H * npairs
    tflops = flops / (ms_step * 1e-3) / 1e12
    # the passes, with the algorithmic flops per visible (pair, head) of each
    # (2*d per contraction): with stored tiles k_dq forms S = Q.K^T and
    # dP = dO.V^T (k_dqw above 128 columns), k_dkdv_p P^T.dO and dS^T.Q, k_dqs dS.K; recomputing, k_dq
    # forms Q.K^T, dO.V^T and dS.K (with the row term), k_dkdv all four
    # (the O entry's row-term kernel, k_rowdot, runs before the first pass and
    # is in ms_per_step only)
    # attn_bwd_f16: the fp16 copies plus the row term (S and dP once more when
    # no forward output is given), k_kv16 (S, dP, P^T.dO, dS^T.Q, storing dS)
    # and k_dqs16 (dS.K from the stored tiles), or k_q16 (S, dP, dS.K) when
    # the tiles do not fit the scratch limit
    # attn_bwd_short: one launch whose key-role workgroups form S, dP, P^T.dO,
    # dS^T.Q and whose query-role workgroups form S, dP, dS.K (14 d per pair
    # and head together), after a row-term launch (S, dP) when no O is given
    if entry == "attn_bwd_short":
        passes = ([("k_short", ms_q, 14.0)] if with_o else
                  [("k_short_rowterm", ms_q, 4.0), ("k_short", ms_k, 14.0)])
    elif entry.startswith("attn_bwd_f16"):
        passes = [("k_cvt16", ms_q, 0.0 if with_o else 4.0), ("k_kv16", ms_k, 8.0),
                  ("k_dqs16", ms_s, 2.0) if ds_stored else ("k_q16", ms_s, 6.0)]
    elif stored:
        # above 128 columns the query-major pass that stores the tiles is k_dqw
        passes = [("k_dqw" if w.d > 128 else "k_dq", ms_q, 4.0), ("k_dkdv_p", ms_k, 4.0),
                  ("k_dqs", ms_s, 2.0)]
    else:
        passes = [("k_dq", ms_q, 6.0), ("k_dkdv", ms_k, 8.0)]
    kernel_ms = {n: round(tt / ncalls, 4) for n, tt, _ in passes}

    # dominant kernel: algorithmic flops per launch / its measured average
    # duration; with stored tiles in head chunks each pass launches once per
    # chunk, and a launch covers that chunk's heads (the average is taken)
    f16 = entry.startswith("attn_bwd_f16")
    launches = (w.H + heads - 1) // heads if stored and not f16 and entry != "attn_bwd_short" else 1
    kname, kms_sum, per_pair = max(passes, key=lambda p: p[1])
    kms = kms_sum / (ncalls * launches)
    kflops = per_pair * w.d * w.H * npairs / launches
    kach = kflops / (kms * 1e-3) / 1e12
    peak = PEAK_FP16_MFMA if entry.startswith("attn_bwd_f16") else PEAK_FP32_MFMA
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(kach, 3),
                "peak": peak, "unit": "TFLOP/s", "frac": round(kach / peak, 4),
                "traffic": (None if f16 and not ds_stored else read_traffic(kname, w.name)), "avg_launch_ms": round(kms, 4),
                "launches_per_step": launches}
    # general path: attn_bwd_plan's figure, the most a call of this size takes
    # (with a seg: head-split partial sums); fp16: the operand copies, D,
    # LSE*log2e and the stored dS tiles, before any partial sums; short: the
    # row term D
    ws_key = ("row_term_bytes" if entry == "attn_bwd_short" else
              "f16_workspace_bytes" if f16 else "workspace_bytes_max")
    ws_val = (0 if entry == "attn_bwd_short" and with_o else
              w.S * w.H * 4 if entry == "attn_bwd_short" else
              f16_ws if f16 else ws_bytes)
    del t, dQ, dK, dV, lse, O
    torch.cuda.empty_cache()
    return dict(workload=w, inputs=x, ms_step=ms_step, tflops=tflops, flops=flops, npairs=npairs,
                kernel_ms=kernel_ms, roofline=roofline, peak=peak,
                stored=None if f16 or entry == "attn_bwd_short" else stored,
                ws_key=ws_key, ws_bytes=ws_val)


def calibration_copy(mb, dev):
    """One device copy of mb MiB (nothing when mb is 0): a kernel of known
    traffic whose FETCH_SIZE and WRITE_SIZE counters scale those of the
    backward kernels to bytes."""
    import torch
    if not mb:
        return
    n = mb * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"bench: calibration copy of {mb} MiB done")


def bench_decode(args):
    """attn_bwd_decode on the decode workload: HBM-bound, so the roofline is
    bytes.  Algorithmic bytes per call: K and V read, dK and dV read and
    written, P read (q, dO, dq are a few KB): 4 (6 T KV d + H T)."""
    import numpy as np
    import torch

    import oracle
    from causal_gqa_attention_bwd_amd import binding
    from causal_gqa_attention_bwd_amd.workloads import DECODE_WORKLOAD, make_decode_inputs

    wl = DECODE_WORKLOAD
    T, H, KV, d = wl["T"], wl["H"], wl["KV"], wl["d"]
    x = make_decode_inputs(T, H, KV, d)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(dev) for k in ("q", "K", "V", "P", "dO")}
    dq, dK, dV = torch.zeros_like(t["q"]), torch.zeros_like(t["K"]), torch.zeros_like(t["V"])
    scale = float(x["scale"])
    log(f"bench: decode workload {wl['name']}: T={T} H={H} KV={KV} d={d}")

    def step():
        binding.attn_bwd_decode(t["q"], t["K"], t["V"], t["P"], t["dO"], dq, dK, dV, scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    calibration_copy(args.calib_copy_mb, dev)
    binding.profile_begin()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms1, ms2, ms3, ncalls = binding.profile_end()
    ms_step = e0.elapsed_time(e1) / args.steps
    assert ncalls == args.steps, (ncalls, args.steps)
    if not (torch.isfinite(dq).all() and torch.isfinite(dK).all() and torch.isfinite(dV).all()):
        raise RuntimeError("non-finite gradients")
    kv_bytes = 4.0 * T * KV * d
    total = 6 * kv_bytes + 4.0 * H * T
    # per kernel: its share of the algorithmic bytes (k_dec_dp: V and P;
    # k_dec_kv: K, dK and dV read and written, P; k_dec_dq: dq)
    passes = [("k_dec_dp", ms1, kv_bytes + 4.0 * H * T), ("k_dec_kv", ms2, 5 * kv_bytes + 4.0 * H * T),
              ("k_dec_dq", ms3, 8.0 * H * d)]
    kernel_ms = {n: round(tt / ncalls, 4) for n, tt, _ in passes}
    kname, kms_sum, kbytes = max(passes, key=lambda p: p[1])
    kms = kms_sum / ncalls
    kach = kbytes / (kms * 1e-3) / 1e9
    value = total / (ms_step * 1e-3) / 1e9
    log(f"bench: {ms_step:.4f} ms/step, " + ", ".join(f"{n} {v:.4f} ms" for n, v in kernel_ms.items())
        + f", {value:.1f} GB/s algorithmic")
    cpu = None
    if args.cpu_groups > 0:
        log("bench: timing the oracle on the host ...")
        t0 = time.perf_counter()
        oracle.attn_bwd_decode(x["q"], x["K"], x["V"], x["P"], x["dO"], x["scale"])
        dt = time.perf_counter() - t0
        cpu = {"value": round(total / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"oracle attn_bwd_decode (fp64 C, one thread) on the whole workload; "
                         f"{dt:.2f} s wall"}
    out = {
        "metric": "single-query attention-backward HBM throughput (algorithmic bytes)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl["name"], "history_len": T, "n_heads": H, "n_kv_heads": KV,
                   "head_dim": d, "entry": "attn_bwd_decode", "algorithmic_bytes_per_step": total,
                   "kernel_ms": kernel_ms},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(kach, 1),
                     "peak": PEAK_HBM * 1000.0, "unit": "GB/s",
                     "frac": round(kach / (PEAK_HBM * 1000.0), 4),
                     "traffic": read_traffic(kname, wl["name"]), "avg_launch_ms": round(kms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4, help="workload id (default: the headline one)")
    ap.add_argument("--cpu-groups", type=int, default=8,
                    help="KV groups in the oracle's timed sample (0: skip the CPU baseline)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--o-entry", action="store_true",
                    help="time attn_bwd_o (row term read off the forward output O) instead")
    ap.add_argument("--rope", action="store_true",
                    help="time attn_bwd_rope (RoPE backward fused into the write-back, base 1e4)")
    ap.add_argument("--decode", action="store_true",
                    help="time attn_bwd_decode (single-query backward over a 32768-key history, "
                         "stored probabilities) instead; reported against HBM bandwidth")
    ap.add_argument("--short", action="store_true",
                    help="time attn_bwd_short (the single-launch short-sequence backward, "
                         "seq_len <= 1024; with --o-entry the forward output is passed)")
    ap.add_argument("--f16", action="store_true",
                    help="time attn_bwd_f16 (fp16 matrix-core operands, fp32 accumulation; with "
                         "--o-entry the forward output is passed)")
    ap.add_argument("--scratch-limit-mb", type=float, default=None,
                    help="set the library's stored-tile scratch limit (MiB; 0: recompute the "
                         "scores) before timing")
    ap.add_argument("--no-extra", dest="extra", action="store_false",
                    help="skip the extra timings (S=16384 documents in fp32, S=4096 with fp16 "
                         "operands) that the default run adds to config.extra")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    if args.decode:
        bench_decode(args)
        return

    import numpy as np
    import torch

    if args.scratch_limit_mb is not None:
        from causal_gqa_attention_bwd_amd import binding
        binding.set_scratch_limit(int(args.scratch_limit_mb * (1 << 20)))

    entry = ("attn_bwd_short" if args.short else
             ("attn_bwd_f16_rope" if args.rope else "attn_bwd_f16") if args.f16 else
             "attn_bwd_rope" if args.rope else "attn_bwd_o" if args.o_entry else "attn_bwd")
    r = time_entry(args.workload, entry, args.o_entry, args.steps, args.warmup, args.calib_copy_mb)
    w, x = r["workload"], r["inputs"]
    log(f"bench: {r['ms_step']:.3f} ms/step, "
        + ", ".join(f"{n} {t:.3f} ms" for n, t in r["kernel_ms"].items())
        + f", {r['tflops']:.2f} TFLOP/s credited")

    cpu = errs = None
    if args.cpu_groups > 0:
        log("bench: timing the oracle on the host ...")
        rope = (10000.0, 0) if args.rope else None
        cpu, sample, ref = cpu_baseline(x, args.cpu_groups, with_o=args.o_entry, rope=rope)
        log(f"bench: oracle {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads "
            f"({cpu['seconds']:.1f} s)")
        cpu = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in cpu.items()
               if k != "seconds"}
        errs = parity_errors(sample, ref, entry, args.o_entry, rope)
        log("bench: parity against the oracle on the same sample: "
            + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))

    extra = None
    if args.extra and entry == "attn_bwd" and args.workload == 4:
        extra = {}
        for key, wid, ent in (("s16384_h16_kv2_d256_docs_geom2048_f32", 5, "attn_bwd"),
                              ("s4096_h32_kv8_d128_causal_f16", 4, "attn_bwd_f16")):
            log(f"bench: extra: {ent} on workload {wid}")
            e = time_entry(wid, ent, False, max(5, args.steps // 2), args.warmup, 0)
            extra[key] = {"entry": ent, "ms_per_step": round(e["ms_step"], 4),
                          "tflops_credited": round(e["tflops"], 3),
                          "pct_of_peak_dtype": round(100.0 * e["tflops"] / e["peak"], 2),
                          "kernel_ms": e["kernel_ms"],
                          "dominant_kernel": e["roofline"]["kernel"],
                          "dominant_kernel_frac": e["roofline"]["frac"]}
            log(f"bench: extra: {e['ms_step']:.3f} ms/step, {e['tflops']:.2f} TFLOP/s, "
                f"{e['roofline']['kernel']} frac {e['roofline']['frac']:.3f}")
            del e

    tflops, ms_step = r["tflops"], r["ms_step"]
    out = {
        "metric": "attention-backward TFLOP/s (causal FLOPs) and % of MI355X matrix peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if args.f16 else "f32",
        "data": "synthetic",
        "pct_of_peak_fp32_matrix": round(100.0 * tflops / PEAK_FP32_MFMA, 2),
        "pct_of_peak_fp16_matrix": round(100.0 * tflops / PEAK_FP16_MFMA, 3),
        "err_dq": None if errs is None else errs["dQ"],
        "err_dk": None if errs is None else errs["dK"],
        "err_dv": None if errs is None else errs["dV"],
        "config": {"workload": w.name, "seq_len": w.S, "n_heads": w.H, "n_kv_heads": w.KV,
                   "head_dim": w.d, "mask": "causal" if not np.any(x["seg"]) else "documents",
                   "valid_pairs": r["npairs"], "credited_flops_per_step": r["flops"],
                   # the same time counted on all causal pairs (labelled; differs from value
                   # only under a document mask)
                   "tflops_on_causal_pairs": round(
                       10.0 * w.d * w.H * (w.S * (w.S + 1) // 2) / (ms_step * 1e-3) / 1e12, 3),
                   "device_compute_units": torch.cuda.get_device_properties(0).multi_processor_count,
                   "entry": entry,
                   "operands": ("fp16, fp32 accumulation" if args.f16 else "fp32"),
                   "forward_output_given": bool(args.o_entry),
                   "stored_tiles": r["stored"],
                   # errors: max|gpu - oracle| / max|oracle| per gradient over the oracle's
                   # sample (cpu_baseline.sample), on zeroed outputs and the oracle's LSE
                   "parity_sample": None if cpu is None else cpu["sample"].split(";")[0],
                   r["ws_key"]: r["ws_bytes"],
                   "kernel_ms": r["kernel_ms"],
                   "extra": extra},
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
