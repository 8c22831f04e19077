"""Plain fp64 reference for the gradients of the flexible-mask attention forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Both pages present the forward as a training operator (MagiAttention
quickstart, "Single-GPU Flex-Flash-Attention": out is differentiated through
autograd; FlagAttention user guide, "FlashAttention": the operator supports
backward).  What the backward computes is the derivative of the forward
definition in ``oracle.fwd``: for a loss with upstream gradient dout = dL/dout,
and with P[i,h,j] = exp(s_ij - lse[i,h]) the attention weight of visible key j
(0 for masked keys and for rows that see nothing),

    dv[j,g]    = sum_{h in group g} sum_i P[i,h,j] dout[i,h]
    dP[i,h,j]  = dout[i,h] . v[j,g]
    dS[i,h,j]  = P[i,h,j] (dP[i,h,j] - sum_j' P[i,h,j'] dP[i,h,j'])   (softmax Jacobian)
    dq[i,h]    = scale * sum_j dS[i,h,j] k[j,g]
    dk[j,g]    = scale * sum_{h in group g} sum_i dS[i,h,j] q[i,h]

with g = h // (Hq // Hkv).  Everything is evaluated in float64 from the exact
input values, a block of query rows at a time, restricted (exactly) to the key
columns some row of the block sees.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .fwd import _as_f64, capped_scores, mask_rows, sink_logits


def attend_backward(q, k, v, dout, q_ranges, k_ranges, mask_types, softmax_scale: Optional[float] = None,
                    block_rows: int = 256, sink=None, sink_layout: str = "sh", softcap: float = 0.0):
    """Returns (dq [Tq,Hq,D], dk [Tk,Hkv,D], dv [Tk,Hkv,D]) in float64, and dsink
    (shaped like `sink`) as a fourth result when `sink` is given.

    Sinks (oracle.fwd.sink_logits) only add terms to the denominator: P keeps
    its definition with the full lse, and a sink's own weight
    Ps[i,s,h] = exp(sink - lse[i,h]) has dP = 0 (no value), so
    d sink = -sum_i Ps[i,s,h] * sum_j P[i,h,j] dP[i,h,j] (summed over rows for
    the shared layout "sh").  Soft-capping multiplies dS by the derivative of
    softcap * tanh(x / softcap), 1 - tanh(x / softcap)^2, before the products
    with k and q.
    """
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if dout.shape != q.shape or v.shape != k.shape or hq % hkv != 0:
        raise ValueError("shape mismatch")
    grp = hq // hkv
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsink = np.zeros(np.shape(sink)) if sink is not None else None
    for b0 in range(0, tq, block_rows):
        rb = np.arange(b0, min(tq, b0 + block_rows))
        sinks = sink_logits(sink, sink_layout, rb, hq)
        mask = mask_rows(rb, q_ranges, k_ranges, mask_types, tk)
        cols = np.nonzero(mask.any(axis=0))[0]
        if cols.size == 0:
            continue  # nothing visible: every gradient of these rows is 0 (out = 0, so Dd = 0)
        mk = mask[:, cols]
        for g in range(hkv):
            kg, vg = k[cols, g, :], v[cols, g, :]
            for hh in range(grp):
                h = g * grp + hh
                raw = (q[rb, h, :] @ kg.T) * scale
                s = np.where(mk, capped_scores(raw, softcap), -np.inf)
                sk = sinks[:, :, h] if sinks is not None else np.zeros((rb.shape[0], 0))
                mx = np.maximum(s.max(axis=1), sk.max(axis=1, initial=-np.inf))
                safe = np.where(np.isfinite(mx), mx, 0.0)
                e = np.exp(s - safe[:, None])
                es = np.exp(sk - safe[:, None])
                den = e.sum(axis=1) + es.sum(axis=1)
                p = e / np.where(den > 0, den, 1.0)[:, None]  # rows that see nothing: all zeros
                do = dout[rb, h, :]
                dv[cols, g, :] += p.T @ do
                dp = do @ vg.T
                dd = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - dd)
                if softcap and softcap > 0:
                    ds = ds * (1.0 - np.tanh(raw / softcap) ** 2)
                dq[rb, h, :] = scale * (ds @ kg)
                dk[cols, g, :] += scale * (ds.T @ q[rb, h, :])
                if sink is not None:
                    ps = es / np.where(den > 0, den, 1.0)[:, None]  # [B, S]
                    contrib = -ps * dd  # [B, S]
                    if sink_layout == "sh":
                        dsink[:, h] += contrib.sum(axis=0)
                    else:
                        dsink[rb, :, h] = contrib
    if sink is not None:
        return dq, dk, dv, dsink
    return dq, dk, dv
