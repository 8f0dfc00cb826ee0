"""Element-wise error bounds for the backward with fp16 product operands
(attn_bwd_f16), derived up front from the rounding model rather than fitted
to measurements.

Model (first order in the unit roundoff u = 2^-11; every sum in fp32):
Q, K, V, dO, P and dS/scale are rounded to fp16 before their products.  For
a visible pair (s, j) of head h:
  score:  |d(scale q.k)| <= a = 2u scale sum_i |q_i k_i|
  dP:     |d(dO.v)|      <= b = 2u sum_i |dO_i v_i|
  P:      |dP_|          <= P (a + u)                 (exponent, then rounding)
  D:      sum_j (|dP_sj| |P_sj dP - ...|): |dD| <= sum_j (|dP_| |dP| + P b)
          (zero when D is read off the forward output O, up to fp32 rounding)
  dS/scale = P (dP - D): |d| <= |dP_| |dP - D| + P (b + |dD|) + u |dS/scale|
then the three products, each with its own rounded operands:
  dQ_s  = scale sum_j dS/scale K_j:  scale sum_j (|d dS| + u |dS|) |K_j|
  dK_j  = scale sum_s,h dS/scale Q:  scale sum_s,h (|d dS| + u |dS|) |Q_s|
  dV_j  = sum_s,h P dO:              sum_s,h (|dP_| + u P) |dO_s|
and the fp32 sums add at most n 2^-24 of the sum of absolute terms (n keys
or queries).  The tests allow twice the first-order bound.

This module computes those sums densely in numpy for the small shapes the
edge tests use; it holds no attention result the tests compare against (that
is the oracle's job), only the size of the rounding error."""
import numpy as np

U16 = 2.0 ** -11
U32 = 2.0 ** -24


def f16_bounds(p, lse, O=None):
    """(bound dQ [S,H,d], bound dK [S,KV,d], bound dV [S,KV,d]) for the inputs
    p (Q, K, V, dO, seg, scale), the row log-sum-exp lse [S,H] and, when the
    row term is read off the forward output, O [S,H,d]."""
    Q, K, V, dO = (np.asarray(p[k], np.float64) for k in ("Q", "K", "V", "dO"))
    S, H, d = Q.shape
    KV = K.shape[1]
    g = H // KV
    sc = float(p["scale"])
    seg = np.zeros(S, np.int64) if p["seg"] is None else np.asarray(p["seg"], np.int64)
    s_idx, j_idx = np.arange(S)[:, None], np.arange(S)[None, :]
    vis = (j_idx <= s_idx) & (j_idx >= seg[:, None])            # [S, S]
    L = np.asarray(lse, np.float64)
    bQ, bK, bV = np.zeros((S, H, d)), np.zeros((S, KV, d)), np.zeros((S, KV, d))
    for h in range(H):
        kv = h // g
        q, k, v, go = Q[:, h], K[:, kv], V[:, kv], dO[:, h]
        x = sc * (q @ k.T)
        with np.errstate(over="ignore", invalid="ignore"):
            P = np.where(vis, np.exp(np.where(vis, x - L[:, h:h + 1], -np.inf)), 0.0)
        dp = go @ v.T
        a = 2 * U16 * sc * (np.abs(q) @ np.abs(k).T)
        b = 2 * U16 * (np.abs(go) @ np.abs(v).T)
        dPe = np.where(vis, P * (a + U16), 0.0)                  # |error of P|
        if O is None:
            D = np.sum(P * dp, axis=1, keepdims=True)
            dD = np.sum(dPe * np.abs(dp) + P * b, axis=1, keepdims=True)
        else:
            D = np.sum(go * np.asarray(O, np.float64)[:, h], axis=1, keepdims=True)
            dD = U32 * d * np.sum(np.abs(go * np.asarray(O, np.float64)[:, h]), axis=1,
                                  keepdims=True)
        ds = np.where(vis, P * (dp - D), 0.0)
        dse = np.where(vis, dPe * np.abs(dp - D) + P * (b + dD) + U16 * np.abs(ds), 0.0)
        n = vis.sum(axis=1, keepdims=True)                      # keys per row
        bQ[:, h] = sc * ((dse + U16 * np.abs(ds)) @ np.abs(k)) \
            + sc * U32 * n * (np.abs(ds) @ np.abs(k))
        bK[:, kv] += sc * ((dse + U16 * np.abs(ds)).T @ np.abs(q)) \
            + sc * U32 * S * (np.abs(ds).T @ np.abs(q))
        bV[:, kv] += (dPe + U16 * P).T @ np.abs(go) + U32 * S * (P.T @ np.abs(go))
    return bQ, bK, bV


def rotated(bound, d):
    """The bound after the RoPE backward turns each column pair: a rotation
    mixes the two columns, so each gets the sum of the pair's bounds."""
    b = np.asarray(bound)
    pair = b.reshape(*b.shape[:-1], d // 2, 2).sum(axis=-1)
    return np.repeat(pair, 2, axis=-1)
