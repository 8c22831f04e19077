"""The q = 0 closed form at the five workloads' full sizes, every row and every head.

With q = 0 every score is 0, so each visible key gets the same weight:
  lse[i, h] = ln |V(i)|          out[i, h] = mean of v[j, g(h)] over j in V(i)
and rows that see nothing get lse = -inf and out = 0.  |V(i)| and the key
intervals come from the slice formula itself (MagiAttention blog, "Calculate
KV Interval Boundaries for Mask Types": row i of a slice sees keys
[ks + (i - qs) if bit 1 of the type, else ks;  ke - (qe - 1 - i) if bit 0,
else ke)), so the check is independent of the oracle and of the kernels' own
tiling, skipping, edge masking, split and combine.  For the single causal
slices this is lse = ln(i + 1) (tiny causal, long context) and ln(2049 + m) at
local row m of the 2048 x 4096 bottom-right rectangles.

Each workload runs in the launch configuration the benchmark times (automatic
plan); the long-context and heterogeneous workloads also with forced split-K,
which sends every row through the logsumexp combine.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

LSE_ABS = 2e-5          # the closed form: only fp32 rounding of ln |V(i)| remains
OUT_MAX, OUT_MEAN = 2e-2, 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def key_intervals(p):
    """Per slice: (rows, a, b) with key interval [a, b) of each row (a <= b), numpy int64."""
    out = []
    for (qs, qe), (ks, ke), t in zip(p.q_ranges.tolist(), p.k_ranges.tolist(), p.mask_types.tolist()):
        rows = np.arange(qs, qe, dtype=np.int64)
        a = ks + (rows - qs) if t & 2 else np.full(rows.shape, ks, dtype=np.int64)
        b = ke - (qe - 1 - rows) if t & 1 else np.full(rows.shape, ke, dtype=np.int64)
        a = np.clip(a, ks, ke)
        b = np.clip(b, a, ke)
        out.append((rows, a, b))
    return out


def visible_counts(p, ivs):
    cnt = np.zeros(p.total_q, dtype=np.int64)
    for rows, a, b in ivs:
        cnt[rows] += b - a
    return cnt


def check_closed_form(gpu_lib, p, split_tiles, what):
    dev = torch.device("cuda", 0)
    log(f"  {what}: inputs on the device (q = 0)")
    q, k, v = W.make_qkv_device(p, dev, q_zero=True)
    log(f"  {what}: forward (split_tiles={split_tiles})")
    out, lse = gpu_lib.flex_flash_attn_fwd(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, split_tiles=split_tiles)
    torch.cuda.synchronize()
    plan = gpu_lib._plan_cache[next(reversed(gpu_lib._plan_cache))]
    del q
    ivs = key_intervals(p)
    cnt = visible_counts(p, ivs)
    # lse on every row and head
    with np.errstate(divide="ignore"):
        ref_lse = np.where(cnt > 0, np.log(np.maximum(cnt, 1)), -np.inf)
    l = lse.double().cpu().numpy()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse)[:, None].repeat(p.heads_q, 1)), \
        f"{what}: -inf pattern of lse"
    fin = cnt > 0
    lerr = np.abs(l[fin] - ref_lse[fin, None]).max() if fin.any() else 0.0
    # out on every row and head: mean of the visible v through prefix sums (fp64 on the device)
    ratio = p.heads_q // p.heads_kv
    S = torch.zeros((p.total_k + 1, p.heads_kv, p.head_dim), dtype=torch.float64, device=dev)
    S[1:] = torch.cumsum(v.double(), dim=0)
    num = torch.zeros((p.total_q, p.heads_kv, p.head_dim), dtype=torch.float64, device=dev)
    for rows, a, b in ivs:
        for c0 in range(0, rows.size, 16384):
            r = torch.from_numpy(rows[c0:c0 + 16384]).to(dev)
            num[r] += S[torch.from_numpy(b[c0:c0 + 16384]).to(dev)] - S[torch.from_numpy(a[c0:c0 + 16384]).to(dev)]
    cnt_d = torch.from_numpy(np.maximum(cnt, 1)).to(dev).double()
    omax, osum, n_el = 0.0, 0.0, 0
    for c0 in range(0, p.total_q, 8192):
        ref = (num[c0:c0 + 8192] / cnt_d[c0:c0 + 8192, None, None]).repeat_interleave(ratio, dim=1)
        e = (out[c0:c0 + 8192].double() - ref).abs()
        omax = max(omax, e.max().item())
        osum += e.sum().item()
        n_el += e.numel()
    empty = torch.from_numpy(cnt == 0).to(dev)
    assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item(), f"{what}: NaN"
    assert (out[empty] == 0).all().item(), f"{what}: rows without keys must be 0"
    log(f"  {what}: split items {plan.info['num_split_items']}, combine entries {plan.info['num_combine']} | "
        f"lse max err {lerr:.2e} | out max {omax:.2e} mean {osum / n_el:.2e}")
    assert lerr <= LSE_ABS, f"{what}: lse {lerr}"
    assert omax <= OUT_MAX and osum / n_el <= OUT_MEAN, f"{what}: out max {omax} mean {osum / n_el}"
    return cnt, plan


def test_closed_form_counts_match_the_single_slice_formulas():
    # the interval helper above against the closed forms of the single-slice workloads
    c1 = visible_counts(W.config(1), key_intervals(W.config(1)))
    assert (c1 == np.arange(1, 257)).all()
    c2 = visible_counts(W.config(2), key_intervals(W.config(2)))
    assert (c2 == np.tile(2049 + np.arange(2048), 2)).all()
    c5 = visible_counts(W.config(5), key_intervals(W.config(5)))
    assert (c5 == np.arange(1, 131073)).all()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_q_zero_full_size(gpu_lib, cfg):
    p = W.config(cfg)
    cnt, _ = check_closed_form(gpu_lib, p, 0, f"config {cfg} ({p.name})")
    assert int(cnt.sum()) == gpu_lib._plan_cache[next(reversed(gpu_lib._plan_cache))].info["visible_pairs"]


def test_q_zero_hetero_forced_split(gpu_lib):
    p = W.config(4)
    _, plan = check_closed_form(gpu_lib, p, 16, "config 4 forced split")
    assert plan.info["num_combine"] > 0


@pytest.mark.parametrize("split_tiles", [0, 256])
def test_q_zero_long_context_every_row(gpu_lib, split_tiles):
    # 131072 rows x 64 heads: lse = ln(i + 1) on every one; 256 tiles = chunks of 16384 keys
    p = W.config(5)
    _, plan = check_closed_form(gpu_lib, p, split_tiles, f"config 5 split_tiles={split_tiles}")
    if split_tiles:
        assert plan.info["num_split_items"] > 0 and plan.info["num_combine"] > 0
