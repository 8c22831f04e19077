"""Seeded synthetic workloads for flexible-mask attention.

This module only *describes* problems and draws their random inputs.  It holds
none of the attention arithmetic: no mask predicate, no softmax, no tiling.
Both the CPU oracle (``oracle/``) and the HIP path (``flexible_mask_flash_amd``)
are fed from here, and neither imports the other.

A problem is a set of slices ``(q_range, k_range, mask_type)`` over packed
token axes of lengths ``total_q`` / ``total_k`` (MagiAttention page, section
"Single-GPU Flex-Flash-Attention": q_ranges / k_ranges int32 [S,2], half-open,
attn_type_map 0 = full, 1 = causal).  q is [total_q, Hq, D], k and v are
[total_k, Hkv, D], all bfloat16.

Recipes (seed i for config i):
  1  tiny causal: one causal slice over 256 tokens, Hq = Hkv = 2, D = 64.
  2  rectangular causal + GQA: B = 2 batches packed, batch b is the slice
     q [2048b, 2048b+2048) x k [4096b, 4096b+4096), causal, Hq 16, Hkv 4, D 128
     (FlagAttention user guide, "FlashAttention" example shape).
  3  packed documents: 16384 tokens; document lengths round(lognormal(ln 1024,
     sigma 1)) clipped to [128, 8192], drawn one at a time from
     numpy.default_rng(3) until the total is reached, the last one trimmed;
     one causal slice per document; Hq 32, Hkv 8, D 128.
  4  heterogeneous mix: 32768 tokens; tokens [0, 512) are a shared prefix with
     a full self slice; documents of uniform-integer length in [512, 8192]
     (default_rng(4)) fill [512, 32768), the last one trimmed.  A document
     [s, e) with p = floor(L/4) gets: full q[s,s+p) x k[s,s+p); causal
     q[s+p,e) x k[s,e); full q[s,e) x k[0,512).  Hq 32, Hkv 8, D 128.
  5  long context: one causal slice over 131072 tokens, Hq 64, Hkv 8, D 128.

q, k, v are drawn as float32 N(0,1) with ``torch.Generator().manual_seed(seed)``
in the order q, k, v and rounded to bfloat16 (round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

FULL = 0
CAUSAL = 1
INVCAUSAL = 2
BICAUSAL = 3

CONFIG_NAMES = {
    1: "tiny_causal",
    2: "rect_causal_gqa",
    3: "packed_docs",
    4: "hetero_mask_mix",
    5: "long_context",
}


@dataclasses.dataclass
class Problem:
    """A flexible-mask attention problem: shapes plus the slice list."""

    name: str
    total_q: int
    total_k: int
    heads_q: int
    heads_kv: int
    head_dim: int
    q_ranges: np.ndarray  # int32 [S, 2]
    k_ranges: np.ndarray  # int32 [S, 2]
    mask_types: np.ndarray  # int32 [S]
    seed: int = 0
    docs: Optional[List[int]] = None

    @property
    def num_slices(self) -> int:
        return int(self.q_ranges.shape[0])

    def describe(self) -> dict:
        d = {
            "workload": self.name,
            "total_q": self.total_q,
            "total_k": self.total_k,
            "heads_q": self.heads_q,
            "heads_kv": self.heads_kv,
            "head_dim": self.head_dim,
            "slices": self.num_slices,
            "seed": self.seed,
        }
        if self.docs is not None:
            d["docs"] = list(self.docs)
        return d


def make_problem(name, total_q, total_k, hq, hkv, d, slices, seed=0, docs=None) -> Problem:
    qr = np.array([s[0] for s in slices], dtype=np.int32).reshape(-1, 2)
    kr = np.array([s[1] for s in slices], dtype=np.int32).reshape(-1, 2)
    ty = np.array([s[2] for s in slices], dtype=np.int32).reshape(-1)
    return Problem(name, total_q, total_k, hq, hkv, d, qr, kr, ty, seed, docs)


def draw_doc_lengths(seed: int, total: int, draw) -> List[int]:
    """Draw document lengths one at a time until `total` is covered; trim the last."""
    rng = np.random.default_rng(seed)
    out: List[int] = []
    s = 0
    while s < total:
        n = min(int(draw(rng)), total - s)
        out.append(n)
        s += n
    return out


def _lognormal_len(rng) -> int:
    return int(np.clip(round(rng.lognormal(np.log(1024.0), 1.0)), 128, 8192))


def _uniform_len(rng) -> int:
    return int(rng.integers(512, 8193))


def config(i: int) -> Problem:
    """The five seeded problems (see module docstring)."""
    if i == 1:
        return make_problem(CONFIG_NAMES[1], 256, 256, 2, 2, 64,
                            [((0, 256), (0, 256), CAUSAL)], seed=1)
    if i == 2:
        sl = [((2048 * b, 2048 * b + 2048), (4096 * b, 4096 * b + 4096), CAUSAL) for b in range(2)]
        return make_problem(CONFIG_NAMES[2], 4096, 8192, 16, 4, 128, sl, seed=2)
    if i == 3:
        docs = draw_doc_lengths(3, 16384, _lognormal_len)
        sl, s = [], 0
        for n in docs:
            sl.append(((s, s + n), (s, s + n), CAUSAL))
            s += n
        return make_problem(CONFIG_NAMES[3], 16384, 16384, 32, 8, 128, sl, seed=3, docs=docs)
    if i == 4:
        prefix = 512
        docs = draw_doc_lengths(4, 32768 - prefix, _uniform_len)
        sl = [((0, prefix), (0, prefix), FULL)]
        s = prefix
        for n in docs:
            e = s + n
            p = n // 4
            sl.append(((s, s + p), (s, s + p), FULL))
            sl.append(((s + p, e), (s, e), CAUSAL))
            sl.append(((s, e), (0, prefix), FULL))
            s = e
        return make_problem(CONFIG_NAMES[4], 32768, 32768, 32, 8, 128, sl, seed=4, docs=docs)
    if i == 5:
        return make_problem(CONFIG_NAMES[5], 131072, 131072, 64, 8, 128,
                            [((0, 131072), (0, 131072), CAUSAL)], seed=5)
    raise ValueError(f"no config {i}")


def scaled(i: int, factor: int) -> Problem:
    """Config `i` with every token coordinate divided by `factor` (for oracle-sized runs).

    Head counts and head_dim are kept; slice boundaries are floor-divided, which
    keeps the slices disjoint and the mask kinds unchanged.
    """
    p = config(i)
    f = int(factor)
    qr = (p.q_ranges // f).astype(np.int32)
    kr = (p.k_ranges // f).astype(np.int32)
    return Problem(f"{p.name}_div{f}", p.total_q // f, p.total_k // f, p.heads_q, p.heads_kv,
                   p.head_dim, qr, kr, p.mask_types.copy(), p.seed, None)


def random_problem(seed: int, total_q: int, total_k: int, hq: int, hkv: int, d: int,
                   max_slices: int = 6, n_types: int = 2) -> Problem:
    """Random disjoint slices for small property tests.

    Slices are built on a grid of q bands; each q band receives up to two slices
    whose k ranges do not overlap, so no (q, k) pair is covered twice.  Types are
    drawn from the first n_types codes (2: full / causal; 4: also inverse causal
    and bi-causal); empty ranges and rows with no slice occur by design.
    """
    rng = np.random.default_rng(seed)
    cuts = sorted(set([0, total_q] + list(rng.integers(0, total_q + 1, size=rng.integers(1, 4)))))
    slices = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if rng.random() < 0.15:
            continue  # a q band with no slice: its rows see nothing
        kcuts = sorted(rng.integers(0, total_k + 1, size=4).tolist())
        pairs = [(kcuts[0], kcuts[1]), (kcuts[2], kcuts[3])]
        for (ka, kb) in pairs[: rng.integers(1, 3)]:
            # occasionally shrink the q range inside the band (still disjoint)
            qa, qb = a, b
            if rng.random() < 0.3 and b - a > 2:
                qa = int(rng.integers(a, b))
                qb = int(rng.integers(qa, b + 1))
            slices.append(((int(qa), int(qb)), (int(ka), int(kb)), int(rng.integers(0, n_types))))
            if len(slices) >= max_slices:
                break
        if len(slices) >= max_slices:
            break
    if not slices:
        slices.append(((0, total_q), (0, total_k), FULL))
    return make_problem(f"random_{seed}", total_q, total_k, hq, hkv, d, slices, seed=seed)


def make_qkv(p: Problem, seed: Optional[int] = None, q_zero: bool = False, dtype=None):
    """Draw q, k, v (CPU, bfloat16 unless `dtype` says otherwise) for problem `p`.

    Returns torch tensors q [Tq,Hq,D], k [Tk,Hkv,D], v [Tk,Hkv,D].
    """
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype

    g = torch.Generator().manual_seed(p.seed if seed is None else seed)
    q = torch.randn(p.total_q, p.heads_q, p.head_dim, generator=g, dtype=torch.float32)
    k = torch.randn(p.total_k, p.heads_kv, p.head_dim, generator=g, dtype=torch.float32)
    v = torch.randn(p.total_k, p.heads_kv, p.head_dim, generator=g, dtype=torch.float32)
    if q_zero:
        q.zero_()
    return q.to(dtype), k.to(dtype), v.to(dtype)


def make_qkv_device(p: Problem, device, seed: Optional[int] = None, q_zero: bool = False, dtype=None):
    """Draw q, k, v for problem `p` directly on `device` (a seeded device generator; for
    full-size runs whose inputs are too large to draw on the CPU quickly).  The draws are
    N(0,1) in the order q, k, v, rounded to bfloat16 (or `dtype`); they are not the same
    numbers as make_qkv's CPU draws."""
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    g = torch.Generator(device=device).manual_seed(p.seed if seed is None else seed)
    shape_q = (p.total_q, p.heads_q, p.head_dim)
    if q_zero:
        q = torch.zeros(shape_q, dtype=dtype, device=device)
    else:
        q = torch.randn(shape_q, generator=g, dtype=torch.float32, device=device).to(dtype)
    k = torch.randn((p.total_k, p.heads_kv, p.head_dim), generator=g, dtype=torch.float32, device=device).to(dtype)
    v = torch.randn((p.total_k, p.heads_kv, p.head_dim), generator=g, dtype=torch.float32, device=device).to(dtype)
    return q, k, v


def sliding_window_problem(T, w, docs, hq, hkv, d, seed):
    """Per-document sliding window of w keys: row i sees keys [max(s, i - w + 1), i + 1).
    The first w - 1 rows of a document are a causal slice; the rest a bi-causal band."""
    sl = []
    for s0, e0 in zip(docs[:-1], docs[1:]):
        h = min(e0, s0 + w - 1)
        if h > s0:
            sl.append(((s0, h), (s0, h), CAUSAL))
        if e0 > h:
            sl.append(((h, e0), (h - w + 1, e0), BICAUSAL))
    return make_problem(f"window{w}", T, T, hq, hkv, d, sl, seed=seed)


def block_sparse_problem(total: int, q_block: int, k_block: int, keep: float, hq: int, hkv: int, d: int,
                         seed: int, name: Optional[str] = None) -> Problem:
    """Uniform block-sparse mask over `total` tokens (q = k axis).

    The query axis is cut into blocks of q_block rows and the key axis into blocks
    of k_block keys; every query block keeps the same number of key blocks,
    round(keep * number of key blocks) (at least 1), drawn without replacement
    from numpy.random.default_rng(seed); each kept (query block, key block) cell
    is one FULL slice.  The block-size pairs of the MagiAttention experiment
    notes (uniform block sparse: 64/64 and 128/128, small query blocks 8-32
    against 64-key blocks, small key blocks 1-64 against 64-row blocks) name the
    shapes; the kept fraction is not given there (a quarter is used here).
    """
    rng = np.random.default_rng(seed)
    nq, nk = -(-total // q_block), -(-total // k_block)
    n_keep = max(1, int(round(keep * nk)))
    sl = []
    for bq in range(nq):
        qs, qe = bq * q_block, min(total, (bq + 1) * q_block)
        for bk in sorted(rng.choice(nk, size=n_keep, replace=False).tolist()):
            sl.append(((qs, qe), (bk * k_block, min(total, (bk + 1) * k_block)), FULL))
    return make_problem(name or f"block_sparse_q{q_block}_k{k_block}", total, total, hq, hkv, d, sl, seed=seed)


# Extra workloads beyond the five configurations (by name): block-sparse planner
# stress cases at the packed-document head shape (Hq 32, Hkv 8, D 128).
EXTRA_WORKLOADS = {
    "block_sparse": lambda: block_sparse_problem(16384, 64, 64, 0.25, 32, 8, 128, 31, "block_sparse"),
    "block_sparse_k16": lambda: block_sparse_problem(16384, 64, 16, 0.25, 32, 8, 128, 32, "block_sparse_k16"),
    "block_sparse_q16": lambda: block_sparse_problem(16384, 16, 64, 0.25, 32, 8, 128, 33, "block_sparse_q16"),
    # sliding windows of 1024 keys over the packed documents (bi-causal bands)
    "sliding_window": lambda: _named(sliding_window_problem(16384, 1024, [0] + list(np.cumsum(config(3).docs)),
                                                            32, 8, 128, 3), "sliding_window"),
    "packed_docs_d64": lambda: _with_head_dim(config(3), 64, "packed_docs_d64"),
    "packed_docs_d32": lambda: _with_head_dim(config(3), 32, "packed_docs_d32"),
    "packed_docs_d16": lambda: _with_head_dim(config(3), 16, "packed_docs_d16"),
}


def _named(p: Problem, name: str) -> Problem:
    p.name = name
    return p


def _with_head_dim(p: Problem, d: int, name: str) -> Problem:
    """The same mask and head counts with another head_dim."""
    return make_problem(name, p.total_q, p.total_k, p.heads_q, p.heads_kv, d,
                        [((a, b), (c, e), t) for (a, b), (c, e), t in
                         zip(p.q_ranges.tolist(), p.k_ranges.tolist(), p.mask_types.tolist())], seed=p.seed)


def workload(name: str) -> Problem:
    """A configuration by name (CONFIG_NAMES) or an extra workload (EXTRA_WORKLOADS)."""
    for i, n in CONFIG_NAMES.items():
        if n == name:
            return config(i)
    if name in EXTRA_WORKLOADS:
        return EXTRA_WORKLOADS[name]()
    raise ValueError(f"unknown workload {name!r}")


def make_dout(p: Problem, seed: Optional[int] = None, dtype=None):
    """Draw an upstream gradient dout [Tq,Hq,D] (CPU, bfloat16 unless `dtype`) for problem `p`."""
    import torch

    g = torch.Generator().manual_seed((p.seed if seed is None else seed) + 7919)
    return torch.randn(p.total_q, p.heads_q, p.head_dim, generator=g, dtype=torch.float32).to(
        torch.bfloat16 if dtype is None else dtype)


def sample_rows(p: Problem, n: int, seed: int = 0) -> np.ndarray:
    """A seeded sample of query rows: slice boundaries +/- 1, first/last rows, and random rows."""
    rng = np.random.default_rng(1000 + seed)
    cand = {0, p.total_q - 1}
    for (a, b) in p.q_ranges.tolist():
        for r in (a - 1, a, a + 1, b - 2, b - 1, b):
            if 0 <= r < p.total_q:
                cand.add(int(r))
    extra = rng.integers(0, p.total_q, size=max(0, n - len(cand)))
    rows = sorted(cand | set(int(x) for x in extra))
    return np.array(rows[: max(n, len(cand))], dtype=np.int64)
