"""Plain fp64 reference for the flexible-mask attention forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (MagiAttention quickstart, "Single-GPU Flex-Flash-Attention";
FlagAttention user guide, "FlashAttention"):

  For query token i and query head h, with key/value head g = h // (Hq // Hkv)
  (contiguous GQA groups; the pages only require Hq % Hkv == 0):

    V(i)      = union over slices s with qs <= i < qe of the keys
                  j in [ks, ke)                                   FULL      (type 0)
                  j in [ks, ke - (qe - 1 - i))                    CAUSAL    (type 1)
                  j in [ks + (i - qs), ke)                        INVCAUSAL (type 2)
                  j in [ks + (i - qs), ke - (qe - 1 - i))         BICAUSAL  (type 3)
                (the kv-interval formula of the MagiAttention blog page
                 "Calculate KV Interval Boundaries for Mask Types": bit 1 of the
                 type moves the start by the row's offset from qs, bit 0 moves the
                 end back by its distance to qe - 1; so causal is bottom-right
                 aligned -- local row m of an M x N slice sees local keys
                 n <= N - M + m -- and inverse causal is top-left aligned)
    s_ij      = scale * sum_d q[i,h,d] * k[j,g,d]          scale defaults to 1/sqrt(D)
    lse[i,h]  = ln sum_{j in V(i)} exp(s_ij)                -inf when V(i) is empty
    out[i,h]  = sum_{j in V(i)} exp(s_ij - lse[i,h]) v[j,g]  0 when V(i) is empty

Ranges are half-open [start, end).  Slices may overlap here (the mask is the
union); the HIP library rejects overlapping slices instead.

The computation materialises the explicit boolean mask for a block of query
rows, restricts the key axis to columns that some row of the block can see
(exact: the others are zero in the mask), and evaluates softmax attention in
float64 with numpy BLAS.  The row max is subtracted before exp only to avoid
overflow; that is rounding order, not a different result.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

FULL = 0
CAUSAL = 1
INVCAUSAL = 2
BICAUSAL = 3


def slice_row_interval(i: int, qs: int, qe: int, ks: int, ke: int, mask_type: int) -> Tuple[int, int]:
    """Keys [a, b) that query row i sees through one slice (empty: a >= b).

    FULL: every key of the slice.  CAUSAL: bottom-right aligned, so the last
    query row of the slice sees every key and each earlier row one key fewer.
    INVCAUSAL: top-left aligned, so the first row sees every key and each later
    row starts one key later.  BICAUSAL: both bounds move, a band.
    """
    if not (qs <= i < qe):
        return (0, 0)
    if mask_type not in (FULL, CAUSAL, INVCAUSAL, BICAUSAL):
        raise ValueError(f"unknown mask type {mask_type}")
    a = ks + (i - qs) if mask_type in (INVCAUSAL, BICAUSAL) else ks
    b = ke - (qe - 1 - i) if mask_type in (CAUSAL, BICAUSAL) else ke
    return (a, b)


def mask_rows(rows: Sequence[int], q_ranges, k_ranges, mask_types, total_k: int) -> np.ndarray:
    """Explicit boolean mask [len(rows), total_k]; True = key visible."""
    rows = np.asarray(rows, dtype=np.int64)
    m = np.zeros((rows.shape[0], total_k), dtype=bool)
    cols = np.arange(total_k, dtype=np.int64)[None, :]
    for (qs, qe), (ks, ke), t in zip(np.asarray(q_ranges).tolist(), np.asarray(k_ranges).tolist(),
                                     np.asarray(mask_types).tolist()):
        inside = (rows >= qs) & (rows < qe)
        if not inside.any():
            continue
        if t not in (FULL, CAUSAL, INVCAUSAL, BICAUSAL):
            raise ValueError(f"unknown mask type {t}")
        start = ks + (rows - qs) if t in (INVCAUSAL, BICAUSAL) else np.full(rows.shape, ks, dtype=np.int64)
        end = ke - (qe - 1 - rows) if t in (CAUSAL, BICAUSAL) else np.full(rows.shape, ke, dtype=np.int64)
        vis = (cols >= start[:, None]) & (cols < end[:, None]) & inside[:, None]
        m |= vis
    return m


def dense_mask(q_ranges, k_ranges, mask_types, total_q: int, total_k: int) -> np.ndarray:
    """The whole [total_q, total_k] boolean mask (small problems only)."""
    return mask_rows(np.arange(total_q), q_ranges, k_ranges, mask_types, total_k)


def count_visible_pairs(q_ranges, k_ranges, mask_types, total_q: int, total_k: int) -> int:
    """Number of visible (query, key) pairs per head: the size of the union of intervals, row by row."""
    total = 0
    qr = np.asarray(q_ranges).tolist()
    kr = np.asarray(k_ranges).tolist()
    ty = np.asarray(mask_types).tolist()
    # rows only change their interval set at slice q boundaries; walk rows explicitly
    # but skip rows no slice covers.
    covered = np.zeros(total_q, dtype=bool)
    for (qs, qe) in qr:
        covered[max(qs, 0):min(qe, total_q)] = True
    for i in np.nonzero(covered)[0].tolist():
        ivs = []
        for (qs, qe), (ks, ke), t in zip(qr, kr, ty):
            a, b = slice_row_interval(i, qs, qe, ks, ke, t)
            a, b = max(a, 0), min(b, total_k)
            if b > a:
                ivs.append((a, b))
        if not ivs:
            continue
        ivs.sort()
        cur_a, cur_b = ivs[0]
        for a, b in ivs[1:]:
            if a > cur_b:
                total += cur_b - cur_a
                cur_a, cur_b = a, b
            else:
                cur_b = max(cur_b, b)
        total += cur_b - cur_a
    return total


def _as_f64(x) -> np.ndarray:
    """bf16/float torch tensor or numpy array -> float64 numpy (exact for bf16)."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to(torch.float64).cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def sink_logits(sink, sink_layout: str, rows: np.ndarray, hq: int) -> Optional[np.ndarray]:
    """Sink logits per selected row: [R, S_sink, Hq] float64, or None.

    The MagiAttention quickstart passes `sink` as float32 [S_sink, Hq] (layout
    "sh": the same logits for every query row) or [Tq, S_sink, Hq] ("ssh": per
    row) ("Single-GPU Flex-Flash-Attention" and the sink examples of the
    extension functions).  Reading: each sink logit is one more term of the
    row's softmax denominator, exp(sink), with no value vector; it is not scaled
    by softmax_scale and not soft-capped.
    """
    if sink is None:
        return None
    sk = _as_f64(sink)
    if sink_layout == "sh":
        if sk.ndim != 2 or sk.shape[1] != hq:
            raise ValueError("sink layout 'sh' needs [S_sink, Hq]")
        return np.broadcast_to(sk[None], (rows.shape[0],) + sk.shape)
    if sink_layout == "ssh":
        if sk.ndim != 3 or sk.shape[2] != hq:
            raise ValueError("sink layout 'ssh' needs [Tq, S_sink, Hq]")
        return sk[rows]
    raise ValueError(f"unknown sink layout {sink_layout!r}")


def capped_scores(raw: np.ndarray, softcap: float) -> np.ndarray:
    """Soft-capped scores: softcap * tanh(raw / softcap) for softcap > 0, else raw.

    Reading (the quickstart lists `softcap`, default 0, without defining it): the
    usual logit soft-capping applied to the scaled scores before the mask and
    the softmax; 0 disables it.
    """
    if softcap and softcap > 0:
        return softcap * np.tanh(raw / softcap)
    return raw


def attend(q, k, v, q_ranges, k_ranges, mask_types, softmax_scale: Optional[float] = None,
           rows: Optional[Sequence[int]] = None, block_rows: int = 256, sink=None, sink_layout: str = "sh",
           softcap: float = 0.0):
    """Reference forward.  Returns (out [R,Hq,D] float64, lse [R,Hq] float64).

    q [Tq,Hq,D], k/v [Tk,Hkv,D] (torch or numpy, any float dtype; converted
    exactly to float64).  `rows` selects query rows (default: all).  With
    `sink`, lse is the log of the full denominator (keys and sinks) and a row
    that sees no key has out 0 and lse = ln sum exp(sink).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    if dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    grp = hq // hkv
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    rows = np.arange(tq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    sinks = sink_logits(sink, sink_layout, rows, hq)  # [R, S, Hq] or None
    out = np.zeros((rows.shape[0], hq, d), dtype=np.float64)
    lse = np.full((rows.shape[0], hq), -np.inf, dtype=np.float64)
    for b0 in range(0, rows.shape[0], block_rows):
        rb = rows[b0:b0 + block_rows]
        nb = rb.shape[0]
        mask = mask_rows(rb, q_ranges, k_ranges, mask_types, tk)
        cols = np.nonzero(mask.any(axis=0))[0]
        mk = mask[:, cols]  # [B, C]
        for g in range(hkv):
            kg = k[cols, g, :]  # [C, D]
            vg = v[cols, g, :]
            for hh in range(grp):
                h = g * grp + hh
                s = capped_scores((q[rb, h, :] @ kg.T) * scale, softcap)  # [B, C]
                s = np.where(mk, s, -np.inf)
                sk = sinks[b0:b0 + nb, :, h] if sinks is not None else np.zeros((nb, 0))  # [B, S]
                mx = np.maximum(s.max(axis=1, initial=-np.inf), sk.max(axis=1, initial=-np.inf))
                safe = np.where(np.isfinite(mx), mx, 0.0)
                p = np.exp(s - safe[:, None])  # masked entries -> exp(-inf) = 0
                den = p.sum(axis=1) + np.exp(sk - safe[:, None]).sum(axis=1)
                nonempty = den > 0
                l = np.where(nonempty, safe + np.log(np.where(nonempty, den, 1.0)), -np.inf)
                o = (p @ vg) / np.where(nonempty, den, 1.0)[:, None]
                out[b0:b0 + nb, h, :] = np.where(nonempty[:, None], o, 0.0)
                lse[b0:b0 + nb, h] = l
    return out, lse


def total_attention(q, k, q_ranges, k_ranges, mask_types, softmax_scale: Optional[float] = None,
                    block_rows: int = 256, sink=None, sink_layout: str = "sh", softcap: float = 0.0):
    """Attention probabilities summed over the query axis: [Tk, Hq] float64.

    FlagAttention user guide, "FlashAttention": `total` [B, Hq, N] holds the
    attention probabilities summed over the query axis.  total[j, h] =
    sum_i P[i, h, j] with P[i, h, j] = exp(s_ij - lse[i, h]) on visible pairs
    (the weights `attend` uses; sinks only enter through lse, soft-capping
    through s).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = hq // hkv
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    tot = np.zeros((tk, hq))
    for b0 in range(0, tq, block_rows):
        rb = np.arange(b0, min(tq, b0 + block_rows))
        sinks = sink_logits(sink, sink_layout, rb, hq)
        mask = mask_rows(rb, q_ranges, k_ranges, mask_types, tk)
        cols = np.nonzero(mask.any(axis=0))[0]
        if cols.size == 0:
            continue
        mk = mask[:, cols]
        for g in range(hkv):
            kg = k[cols, g, :]
            for hh in range(grp):
                h = g * grp + hh
                s = np.where(mk, capped_scores((q[rb, h, :] @ kg.T) * scale, softcap), -np.inf)
                sk = sinks[:, :, h] if sinks is not None else np.zeros((rb.shape[0], 0))
                mx = np.maximum(s.max(axis=1), sk.max(axis=1, initial=-np.inf))
                safe = np.where(np.isfinite(mx), mx, 0.0)
                e = np.exp(s - safe[:, None])
                den = e.sum(axis=1) + np.exp(sk - safe[:, None]).sum(axis=1)
                p = e / np.where(den > 0, den, 1.0)[:, None]
                tot[cols, h] += p.sum(axis=0)
    return tot


def merge_partials(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Combine partial (out, lse) over disjoint key sets with a global logsumexp.

    FlagAttention user guide, "Split-KV and paged attention": each split gives a
    partial output and log-normalizer, and the partials merge through a global
    logsumexp:  lse = ln sum_j exp(lse_j);  out = sum_j exp(lse_j - lse) out_j.
    Partials whose lse is -inf (no visible key) carry no weight.
    """
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])  # [n, ...]
    O = np.stack([np.asarray(x, dtype=np.float64) for x in outs])  # [n, ..., D]
    mx = L.max(axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(L - safe)  # -inf -> 0
    den = w.sum(axis=0)
    ne = den > 0
    lse = np.where(ne, safe + np.log(np.where(ne, den, 1.0)), -np.inf)
    wn = np.where(ne, w / np.where(ne, den, 1.0), 0.0)
    out = (wn[..., None] * O).sum(axis=0)
    return out, lse
