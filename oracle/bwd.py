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

from .fwd import _as_f64, mask_rows


def attend_backward(q, k, v, dout, q_ranges, k_ranges, mask_types, softmax_scale: Optional[float] = None,
                    block_rows: int = 256):
    """Returns (dq [Tq,Hq,D], dk [Tk,Hkv,D], dv [Tk,Hkv,D]) in float64."""
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
    for b0 in range(0, tq, block_rows):
        rb = np.arange(b0, min(tq, b0 + block_rows))
        mask = mask_rows(rb, q_ranges, k_ranges, mask_types, tk)
        cols = np.nonzero(mask.any(axis=0))[0]
        if cols.size == 0:
            continue
        mk = mask[:, cols]
        for g in range(hkv):
            kg, vg = k[cols, g, :], v[cols, g, :]
            for hh in range(grp):
                h = g * grp + hh
                s = np.where(mk, (q[rb, h, :] @ kg.T) * scale, -np.inf)
                mx = s.max(axis=1)
                safe = np.where(np.isfinite(mx), mx, 0.0)
                e = np.exp(s - safe[:, None])
                den = e.sum(axis=1)
                p = e / np.where(den > 0, den, 1.0)[:, None]  # rows that see nothing: all zeros
                do = dout[rb, h, :]
                dv[cols, g, :] += p.T @ do
                dp = do @ vg.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[rb, h, :] = scale * (ds @ kg)
                dk[cols, g, :] += scale * (ds.T @ q[rb, h, :])
    return dq, dk, dv
