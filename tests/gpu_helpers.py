"""Shared helpers of the GPU tests: move seeded numpy inputs to cuda:0, call the
HIP path through the C ABI, compare with the oracle."""
import numpy as np
import torch

from causal_gqa_attention_bwd_amd import binding

TOL = 2e-3  # max|gpu - oracle| <= TOL * max|oracle|, per output tensor


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def seg_dev(seg):
    return None if seg is None else to_dev(np.asarray(seg, np.uint32).astype(np.int32))


def gpu_bwd(p, lse, init=None, seg=None, use_seg=True, O=None, rope=None, f16=False,
            short=False):
    """Run attn_bwd (attn_bwd_o when the forward output O is given; attn_bwd_rope
    when rope = (base, pos_offset); attn_bwd_f16, with or without O, when f16;
    attn_bwd_short, with or without O, when short) on the GPU.  Returns numpy
    (dQ, dK, dV)."""
    t = {k: to_dev(p[k]) for k in ("Q", "K", "V", "dO")}
    if init is None:
        out = [torch.zeros_like(t["Q"]), torch.zeros_like(t["K"]), torch.zeros_like(t["V"])]
    else:
        out = [to_dev(x.copy()) for x in init]
    s = seg_dev(p["seg"] if seg is None else seg) if use_seg else None
    L = to_dev(lse.astype(np.float32))
    if short:
        binding.attn_bwd_short(t["Q"], t["K"], t["V"],
                               None if O is None else to_dev(O.astype(np.float32)), t["dO"], L, s,
                               *out, float(p["scale"]))
    elif f16 and rope is not None:
        binding.attn_bwd_f16_rope(t["Q"], t["K"], t["V"],
                                  None if O is None else to_dev(O.astype(np.float32)), t["dO"], L,
                                  s, *out, float(p["scale"]), float(rope[0]), int(rope[1]))
    elif f16:
        binding.attn_bwd_f16(t["Q"], t["K"], t["V"],
                             None if O is None else to_dev(O.astype(np.float32)), t["dO"], L, s,
                             *out, float(p["scale"]))
    elif rope is not None:
        binding.attn_bwd_rope(t["Q"], t["K"], t["V"],
                              None if O is None else to_dev(O.astype(np.float32)), t["dO"], L, s,
                              *out, float(p["scale"]), float(rope[0]), int(rope[1]))
    elif O is None:
        binding.attn_bwd(t["Q"], t["K"], t["V"], t["dO"], L, s, *out, float(p["scale"]))
    else:
        binding.attn_bwd_o(t["Q"], t["K"], t["V"], to_dev(O.astype(np.float32)), t["dO"], L, s,
                           *out, float(p["scale"]))
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def gpu_fwd(p, want_o=True):
    t = {k: to_dev(p[k]) for k in ("Q", "K", "V")}
    S, H, d = p["Q"].shape
    O = torch.empty_like(t["Q"]) if want_o else None
    LSE = torch.empty((S, H), dtype=torch.float32, device=dev())
    binding.attn_fwd_lse(t["Q"], t["K"], t["V"], seg_dev(p["seg"]), O, LSE, float(p["scale"]))
    torch.cuda.synchronize()
    return (None if O is None else O.cpu().numpy()), LSE.cpu().numpy()


def rel_err(got, want):
    want = np.asarray(want, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - want))) / max(
        float(np.max(np.abs(want))), 1e-30)
