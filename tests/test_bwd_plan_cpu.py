"""Host-side checks of the backward worklists (no GPU, no compute calls).

The backward plan holds two worklists (include/ffa.h, FFA_PLAN_BACKWARD):
- dQ, query-major: the forward's items without split.  Rasterised with the
  kernels' visibility rule (key j of a tile is used by row i iff
  i + lo_base <= j < min(k_hi, i + edge_base)), it must cover every visible
  (row, head, key) of the oracle's mask exactly once.
- dK / dV, key-major: items (key block, kv head) over the transposed slices,
  whose runs walk query positions; the same rule with the key as the row.
  Visited once per query head of the kv head, it must cover the mask of every
  query head exactly once, too.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W

ffa = pytest.importorskip("flexible_mask_flash_amd")

HDR, REC, IREC, BWDHDR = 16, 8, 16, 8
NCU = 256


def make_plan(p, **kw):
    return ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, num_cus=kw.pop("num_cus", NCU), backward=True, **kw)


def parse_bwd(meta):
    off = int(meta[14])
    assert off > 0
    n_dq, n_dqr, n_kv, n_kvr, kv_rows, G = meta[off:off + 6]
    w = off + BWDHDR
    out = {"kv_rows": kv_rows, "G": G}
    for name, n_items, n_runs in (("dq", n_dq, n_dqr), ("kv", n_kv, n_kvr)):
        items = meta[w:w + n_items * IREC].reshape(n_items, IREC)
        w += n_items * IREC
        runs = meta[w:w + n_runs * REC].reshape(n_runs, REC)
        w += n_runs * REC
        has = items[:, 4] > 0
        assert (items[~has, 8:] == 0).all()
        if has.any():
            assert (items[has, 8:] == runs[items[has, 3]]).all()
        assert (items[:, 5] == -1).all(), "backward items never write partials"
        out[name] = (items[:, :8], runs)
    assert w == meta.size, "backward section does not end the metadata"
    return out


def raster(items, runs, n_rows, n_cols, bn=64):
    """(item, row, col) coverage: col j of a tile is used by row i iff
    i + lb <= j < min(khi, i + eb).  Returns {head field: count matrix}."""
    cover = {}
    for it in items:
        r0, nrows, h0, roff, nruns, _slot, tiles = it[:7]
        rows = np.arange(r0, r0 + nrows)
        assert sum(runs[roff + r][1] for r in range(nruns)) == tiles
        c = cover.setdefault(int(h0), np.zeros((n_rows, n_cols), np.int32))
        for r in range(nruns):
            k0, nt, nf, khi, eb, nl, lb = runs[roff + r][:7]
            assert nt >= 1 and nl >= 0 and nf >= 0 and nl + nf <= nt
            for t in range(nt):
                cols = np.arange(k0 + t * bn, k0 + (t + 1) * bn)
                vis = (cols[None, :] < np.minimum(khi, rows + eb)[:, None]) & (cols[None, :] >= (rows + lb)[:, None])
                if nl <= t < nl + nf:
                    assert vis.all(), "a tile marked full needs a mask"
                assert vis.any(), "an emitted tile is fully masked"
                kk = cols < n_cols
                c[np.ix_(rows, cols[kk])] += vis[:, kk]
    return cover


def check_bwd(p, **kw):
    plan = make_plan(p, **kw)
    b = parse_bwd(plan.meta_host())
    mask = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k)
    G, ratio = int(b["G"]), p.heads_q // p.heads_kv
    # dQ: per head group; each group field h0 covers heads h0 .. h0 + G - 1
    dq_items, dq_runs = b["dq"]
    cov = raster(dq_items, dq_runs, p.total_q, p.total_k)
    assert sorted(cov) == list(range(0, p.heads_q, G))
    for h0, c in cov.items():
        assert (c == mask).all(), f"dQ head group {h0}: coverage differs from the mask"
    # every query row of every head group is in exactly one dQ item
    rows = np.zeros((p.heads_q // G, p.total_q), np.int32)
    for it in dq_items:
        rows[it[2] // G, it[0]:it[0] + it[1]] += 1
    assert (rows == 1).all()
    # dK / dV: rows are keys, columns are queries; one item per (key block, kv head)
    kv_items, kv_runs = b["kv"]
    assert (kv_items[:, 1] <= b["kv_rows"]).all()
    cov = raster(kv_items, kv_runs, p.total_k, p.total_q)
    assert sorted(cov) == list(range(p.heads_kv))
    for hk, c in cov.items():
        assert (c == mask.T).all(), f"dK/dV kv head {hk}: coverage differs from the transposed mask"
    keys = np.zeros((p.heads_kv, p.total_k), np.int32)
    for it in kv_items:
        keys[it[2], it[0]:it[0] + it[1]] += 1
    assert (keys == 1).all()
    assert plan.info["num_dq_items"] == len(dq_items) and plan.info["num_kv_items"] == len(kv_items)
    assert plan.info["kv_tiles"] == int(kv_items[:, 6].sum()) * ratio
    assert plan.info["dq_tiles"] == int(dq_items[:, 6].sum())
    assert plan.info["bwd_workspace_bytes"] == 8 * p.heads_q * p.total_q
    return plan, b


@pytest.mark.parametrize("seed", range(16))
def test_backward_worklists_cover_mask_exactly_once(seed):
    rng = np.random.default_rng(700 + seed)
    tq, tk = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    p = W.random_problem(700 + seed, tq, tk, hq, hkv, 64, n_types=4)
    check_bwd(p)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_backward_worklists_scaled_configs(cfg):
    p = W.scaled(cfg, {1: 1, 2: 16, 3: 16}[cfg])
    p.heads_q, p.heads_kv = min(p.heads_q, 8), min(p.heads_kv, 2)
    check_bwd(p)


def test_sliding_window_backward_worklists():
    # a band of width 37 over 400 tokens: its transpose is a band with other offsets
    T, w = 400, 37
    p = W.make_problem("window", T, T, 2, 1, 64, [((0, w - 1), (0, w - 1), W.CAUSAL),
                                                    ((w - 1, T), (0, T), W.BICAUSAL)])
    check_bwd(p)


def test_rectangular_causal_transpose_has_a_moving_lower_bound():
    # causal, 100 queries over 300 keys (bottom-right): key j is seen by queries
    # i >= j - 200, so key blocks past 200 start their query runs late and key
    # blocks before 200 see every query
    p = W.make_problem("rect", 100, 300, 1, 1, 64, [((0, 100), (0, 300), W.CAUSAL)])
    plan, b = check_bwd(p)
    items, runs = b["kv"]
    for it in items:
        r = runs[it[3]]
        assert r[6] == 1 - (300 - 100 + 1), "transposed lower offset is 1 - edge_base"
        assert r[4] == 0x3FFFFFFF, "no upper bound after transposing a causal slice"


def test_forward_part_unchanged_by_backward_flag():
    p = W.random_problem(5, 257, 300, 4, 2, 128, n_types=4)
    a = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                 p.head_dim, num_cus=NCU).meta_host()
    b = make_plan(p).meta_host()
    assert a[14] == 0 and b[14] == a.size
    assert (b[:14] == a[:14]).all() and (b[15:a.size] == a[15:]).all()


def test_forward_only_plan_has_no_backward_section():
    plan = ffa.Plan([[0, 64]], [[0, 64]], [1], 64, 64, 2, 2, 128, num_cus=NCU)
    i = plan.info
    assert i["bwd_workspace_bytes"] == 0 and i["num_dq_items"] == 0 and i["num_kv_items"] == 0
    assert plan.meta_host()[14] == 0


def test_bwd_rejects_bad_arguments_without_launching():
    lib = ffa.load_library()
    fake = 1 << 20  # never dereferenced: validation fails first
    pb = make_plan(W.make_problem("c", 64, 64, 2, 2, 128, [((0, 64), (0, 64), W.CAUSAL)]))
    pf = ffa.Plan([[0, 64]], [[0, 64]], [1], 64, 64, 2, 2, 128, num_cus=NCU)
    wsb = pb.info["bwd_workspace_bytes"]

    def call(plan=pb, **kw):
        a = dict(meta=fake, batch=1, q=fake, k=fake, v=fake, out=fake, lse=fake, dout=fake, dq=fake, dk=fake,
                 dv=fake, st=2 * 128, sh=128, scale=0.1, ws=fake, wsb=wsb)
        a.update(kw)
        t = lambda n: (a[n], 0, a["st"], a["sh"])
        args = [*t("q"), *t("k"), *t("v"), *t("out"), a["lse"], 0, 2, 1, *t("dout"), *t("dq"), *t("dk"), *t("dv")]
        return lib.ffa_bwd(plan.handle if plan is not None else None, a["meta"], a["batch"], *args, a["scale"],
                           a.get("ex"), a["ws"], a["wsb"], None)

    assert call(plan=pf) == 11          # planned without FFA_PLAN_BACKWARD
    assert call(plan=None) == 1
    assert call(batch=0) == 11
    assert call(scale=float("inf")) == 11
    assert call(meta=None) == 1
    assert call(dout=None) == 1
    assert call(dk=None) == 1
    assert call(ws=None) == 7
    assert call(wsb=wsb - 4) == 7
    assert call(dq=fake + 4) == 10
    assert call(st=2 * 128 + 2) == 10
    assert call(st=(1 << 24) * 8) == 11  # token stride beyond the 32-bit tile addressing
    assert call(st=-256) == 11            # negative token strides (unsigned tile offsets)
    ex = ffa.AttnExtras()
    ex.n_sink = 1  # no sink pointer
    assert call(ex=ctypes.byref(ex)) == 1
    ex.n_sink, ex.softcap = 0, float("inf")
    assert call(ex=ctypes.byref(ex)) == 11
    # n_sink * heads_q beyond the d sink grid: refused before the first kernel is enqueued
    hq = 40000
    pbig = make_plan(W.make_problem("h", 32, 32, hq, 1, 16, [((0, 32), (0, 32), W.FULL)]))
    ex = ffa.AttnExtras()
    ex.n_sink, ex.sink, ex.dsink, ex.sink_ss, ex.sink_sh = 65536, fake, fake, hq, 1
    assert call(plan=pbig, st=hq * 16, sh=16, wsb=pbig.info["bwd_workspace_bytes"], ex=ctypes.byref(ex)) == 11
    assert "n_sink" in lib.ffa_last_error().decode()


@pytest.mark.parametrize("qb,kb", [(64, 64), (16, 64), (64, 16), (64, 1), (8, 64)])
def test_block_sparse_worklists_cover_mask_exactly_once(qb, kb):
    # uniform block-sparse masks: many tiny FULL slices (forward and both backward worklists)
    p = W.block_sparse_problem(256, qb, kb, 0.25, 4, 1, 64, seed=qb * 100 + kb)
    check_bwd(p)
    from tests.test_library_cpu import check_plan
    check_plan(p)


@pytest.mark.parametrize("name,qb,kb", [("block_sparse", 64, 64), ("block_sparse_k16", 64, 16),
                                         ("block_sparse_q16", 16, 64)])
def test_block_sparse_full_size_plans_quickly(name, qb, kb):
    # The visible-pair count (the FLOP count of the bench lines) against the closed form of
    # the construction: every kept (query block, key block) cell is a disjoint FULL slice of
    # qb x kb pairs (16384 is a multiple of both block sizes), and every query block keeps
    # round(nk / 4) of the nk key blocks.
    import time
    p = W.workload(name)
    nq, nk = 16384 // qb, 16384 // kb
    n_keep = round(0.25 * nk)
    assert p.num_slices == nq * n_keep
    cells = np.stack([p.q_ranges[:, 0] // qb, p.k_ranges[:, 0] // kb], axis=1)
    assert len({tuple(c) for c in cells.tolist()}) == p.num_slices  # no cell twice
    assert ((p.q_ranges[:, 1] - p.q_ranges[:, 0]) == qb).all() and ((p.k_ranges[:, 1] - p.k_ranges[:, 0]) == kb).all()
    t0 = time.perf_counter()
    plan = make_plan(p)
    dt = time.perf_counter() - t0
    assert plan.info["visible_pairs"] == nq * n_keep * qb * kb
    assert dt < 5.0, f"{name}: planning took {dt:.2f} s for {p.num_slices} slices"


def test_total_attention_rejects_bad_arguments_without_launching():
    lib = ffa.load_library()
    fake = 1 << 20  # never dereferenced: validation fails first
    pb = make_plan(W.make_problem("c", 64, 64, 2, 2, 128, [((0, 64), (0, 64), W.CAUSAL)]))
    pf = ffa.Plan([[0, 64]], [[0, 64]], [1], 64, 64, 2, 2, 128, num_cus=NCU)
    wsb = pb.info["bwd_workspace_bytes"]

    def call(plan=pb, **kw):
        a = dict(meta=fake, batch=1, q=fake, k=fake, lse=fake, tot=fake, st=2 * 128, sh=128, scale=0.1,
                 ws=fake, wsb=wsb, ex=None)
        a.update(kw)
        return lib.ffa_total_attention(plan.handle if plan is not None else None, a["meta"], a["batch"],
                                       a["q"], 0, a["st"], a["sh"], a["k"], 0, a["st"], a["sh"],
                                       a["lse"], 0, 2, 1, a["tot"], 0, 1, 64, a["scale"], a["ex"],
                                       a["ws"], a["wsb"], None)

    assert call(plan=pf) == 11          # no key-major worklist
    assert call(plan=None) == 1
    assert call(batch=0) == 11
    assert call(scale=0.0) == 11
    assert call(meta=None) == 1
    assert call(q=None) == 1
    assert call(tot=None) == 1
    assert call(ws=None) == 7
    assert call(wsb=wsb - 4) == 7
    assert call(k=fake + 2) == 10
    assert call(st=2 * 128 + 4) == 10
    assert call(st=-256) == 11            # negative token strides (unsigned tile offsets)
    ex = ffa.AttnExtras()
    ex.softcap = -2.0
    assert call(ex=ctypes.byref(ex)) == 11
