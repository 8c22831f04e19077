"""Host-side checks of libffa.so (no GPU, no compute calls).

- the library loads and exports every function include/ffa.h declares;
- the planner rejects every invalid input with the documented status;
- the worklist it emits, rasterised with the kernels' visibility rule
  (key j of a tile is used by row i iff j < min(k_hi, i + edge_base)), covers
  every visible (row, head, key) of the oracle's explicit mask exactly once and
  nothing else; tiles before n_full need no mask; split chunks are disjoint and
  their combine entries cover exactly the split rows;
- visible_pairs equals the oracle's count.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffa.h")

ffa = pytest.importorskip("flexible_mask_flash_amd")

HDR, REC, IREC = 16, 8, 16
NCU = 256


@pytest.fixture(scope="module")
def lib():
    return ffa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ffa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"ffa_plan", "ffa_fwd", "ffa_plan_upload", "ffa_plan_destroy"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ffa.h but not exported"
    bound = {s[0] for s in ffa._SIGNATURES}
    assert set(names) == bound, "binding and header disagree"


def test_extras_layout_matches_the_header():
    # ffa_attn_extras as include/ffa.h declares it (the binding's ctypes mirror): two
    # pointers, four int64 strides, n_sink, softcap, dtype and flags
    import ctypes as ct
    assert ct.sizeof(ffa.AttnExtras) == 2 * 8 + 4 * 8 + 4 * 4
    assert [f[0] for f in ffa.AttnExtras._fields_] == ["sink", "dsink", "sink_sb", "sink_st", "sink_ss", "sink_sh",
                                                       "n_sink", "softcap", "dtype", "flags"]
    assert ffa.EXTRAS_ROUNDED_NORM == 1


def test_abi_version_and_status_strings(lib):
    assert lib.ffa_abi_version() == 3
    for code in range(12):
        assert lib.ffa_status_string(code).decode() not in ("", "unknown status")
    assert lib.ffa_status_string(99).decode() == "unknown status"


def plan_status(qr, kr, ty, tq, tk, hq, hkv, d, num_cus=NCU):
    try:
        ffa.Plan(qr, kr, ty, tq, tk, hq, hkv, d, num_cus=num_cus)
        return 0
    except ffa.FFAError as e:
        return e.status


def test_validation_errors():
    ok = ([[0, 8]], [[0, 8]], [1])
    assert plan_status(*ok, 8, 8, 2, 2, 128) == 0
    assert plan_status(*ok, 8, 8, 2, 2, 96) == 2            # head_dim
    assert plan_status(*ok, 8, 8, 2, 2, 8) == 2
    assert plan_status(*ok, 8, 8, 2, 2, 16) == 0
    assert plan_status(*ok, 8, 8, 2, 2, 32) == 0
    assert plan_status(*ok, 8, 8, 0, 2, 128) == 2           # heads
    assert plan_status(*ok, -1, 8, 2, 2, 128) == 2          # total_q
    assert plan_status(*ok, 8, 8, 6, 4, 128) == 3           # GQA
    assert plan_status([[0, 9]], [[0, 8]], [1], 8, 8, 2, 2, 128) == 4   # q out of range
    assert plan_status([[5, 3]], [[0, 8]], [1], 8, 8, 2, 2, 128) == 4   # start > end
    assert plan_status([[0, 8]], [[-1, 8]], [0], 8, 8, 2, 2, 128) == 4
    assert plan_status([[0, 8]], [[0, 8]], [4], 8, 8, 2, 2, 128) == 5   # mask type
    assert plan_status([[0, 8]], [[0, 8]], [-1], 8, 8, 2, 2, 128) == 5
    assert plan_status([[0, 8]], [[0, 8]], [2], 8, 8, 2, 2, 128) == 0   # inverse causal
    assert plan_status([[0, 8]], [[0, 8]], [3], 8, 8, 2, 2, 128) == 0   # bi-causal (the diagonal)
    assert plan_status([[0, 8], [4, 8]], [[0, 8], [7, 8]], [0, 0], 8, 8, 2, 2, 128) == 6  # overlap
    # touching but disjoint: causal [0,8)x[0,8) and full rows [0,8) keys [8,12)
    assert plan_status([[0, 8], [0, 8]], [[0, 8], [8, 12]], [1, 0], 8, 12, 2, 2, 128) == 0
    # causal slices whose rectangles overlap but whose visible pairs do not
    # (row i of a 4x8 causal sees keys < 5 + i, so key 7 only from row 3 on)
    assert plan_status([[0, 4], [0, 3]], [[0, 8], [7, 8]], [1, 0], 4, 8, 1, 1, 64) == 0
    assert plan_status([[0, 4], [0, 4]], [[0, 8], [7, 8]], [1, 0], 4, 8, 1, 1, 64) == 6
    assert plan_status(*ok, 8, 8, 2, 2, 128, num_cus=-3) == 11
    # a band (row i sees keys [i, i + 3)) meets the FULL slice on key 5 only on
    # rows 3..5: neither the first nor the last shared row shows the overlap
    assert plan_status([[0, 10], [0, 10]], [[0, 12], [5, 6]], [3, 0], 10, 12, 1, 1, 64) == 6
    assert plan_status([[0, 10], [0, 3]], [[0, 12], [5, 6]], [3, 0], 10, 12, 1, 1, 64) == 0
    assert plan_status([[0, 10], [6, 10]], [[0, 12], [5, 6]], [3, 0], 10, 12, 1, 1, 64) == 0
    # inverse causal over keys [i, 10) next to causal over [0, i - 4): disjoint on every row
    assert plan_status([[0, 10], [0, 10]], [[0, 10], [0, 5]], [2, 1], 10, 10, 1, 1, 64) == 0
    # ... but a FULL slice on key 0 meets it on the first row only
    assert plan_status([[0, 10], [0, 10]], [[0, 10], [0, 1]], [2, 0], 10, 10, 1, 1, 64) == 6
    # zero slices is a valid (all-empty) problem
    assert plan_status(np.zeros((0, 2)), np.zeros((0, 2)), np.zeros(0), 8, 8, 2, 2, 64) == 0
    # empty slices are no-ops, even when their rectangle would overlap another slice
    assert plan_status([[0, 8], [2, 2]], [[0, 8], [0, 8]], [0, 0], 8, 8, 2, 2, 64) == 0


@pytest.mark.parametrize("seed", range(6))
def test_overlap_verdict_matches_mask_intersection(seed):
    # random pairs of slices of all four types: the planner rejects a pair iff the
    # oracle's masks of the two slices share a (row, key) pair
    rng = np.random.default_rng(900 + seed)
    for _ in range(150):
        T = int(rng.integers(1, 24))
        qr, kr = [], []
        for _s in range(2):
            a, b = sorted(rng.integers(0, T + 1, size=2).tolist())
            c, d = sorted(rng.integers(0, T + 1, size=2).tolist())
            qr.append([a, b]), kr.append([c, d])
        ty = rng.integers(0, 4, size=2).tolist()
        m0 = oracle.dense_mask([qr[0]], [kr[0]], [ty[0]], T, T)
        m1 = oracle.dense_mask([qr[1]], [kr[1]], [ty[1]], T, T)
        want = 6 if (m0 & m1).any() else 0
        assert plan_status(qr, kr, ty, T, T, 1, 1, 64) == want, (qr, kr, ty)


def test_last_error_names_the_slice(lib):
    with pytest.raises(ffa.FFAError) as ei:
        ffa.Plan([[0, 4], [0, 4], [1, 3]], [[0, 4], [4, 6], [5, 6]], [0, 0, 0], 4, 6, 1, 1, 64, num_cus=NCU)
    assert ei.value.status == 6
    assert "slices 1 and 2" in lib.ffa_last_error().decode()


def parse(meta):
    h = meta[:HDR]
    assert h[0] == 0x46464131
    n_items, n_runs, n_comb, G, rows, bn = h[2], h[3], h[4], h[5], h[6], h[7]
    items = meta[HDR:HDR + n_items * IREC].reshape(n_items, IREC)
    r0 = HDR + n_items * IREC
    runs = meta[r0:r0 + n_runs * REC].reshape(n_runs, REC)
    comb = meta[r0 + n_runs * REC:r0 + (n_runs + n_comb) * REC].reshape(n_comb, REC)
    # every item carries a copy of its first run record (zeros when it has none)
    has = items[:, 4] > 0
    assert (items[~has, 8:] == 0).all()
    if has.any():
        assert (items[has, 8:] == runs[items[has, 3]]).all(), "inline first run differs from runs[run_off]"
    return dict(G=G, rows=rows, bn=bn, items=items[:, :8], runs=runs, comb=comb, hdr=h)


def rasterise(p, plan):
    """Per head, count how often each (row, key) is used by the kernels."""
    m = parse(plan.meta_host())
    G, bn = m["G"], m["bn"]
    hq = p.heads_q
    cover = np.zeros((hq, p.total_q, p.total_k), dtype=np.int32)
    rows_written = np.zeros((hq, p.total_q), dtype=np.int32)      # final writes (main kernel)
    partial_slots = {}
    for it in m["items"]:
        q0, nrows, h0, roff, nruns, slot, tiles = it[:7]
        assert 1 <= nrows <= m["rows"] and h0 % G == 0
        rows = np.arange(q0, q0 + nrows)
        assert sum(m["runs"][roff + r][1] for r in range(nruns)) == tiles
        for r in range(nruns):
            k0, nt, nf, khi, eb, nl, lb = m["runs"][roff + r][:7]
            assert nt >= 1 and nl >= 0 and nf >= 0 and nl + nf <= nt
            for t in range(nt):
                keys = np.arange(k0 + t * bn, k0 + (t + 1) * bn)
                lim = np.minimum(khi, rows + eb)
                vis = (keys[None, :] < lim[:, None]) & (keys[None, :] >= (rows + lb)[:, None])
                if nl <= t < nl + nf:
                    assert vis.all(), "a tile marked full needs a mask"
                assert vis.any(), "an emitted tile is fully masked"
                kk = keys[keys < p.total_k]
                for g in range(G):
                    cover[h0 + g][np.ix_(rows, kk)] += vis[:, : kk.size]
        for g in range(G):
            if slot < 0:
                rows_written[h0 + g, rows] += 1
            else:
                for lr in range(nrows):
                    s = slot + lr * G + g
                    assert s not in partial_slots, "two items write one partial slot"
                    partial_slots[s] = (q0 + lr, h0 + g)
    combined = np.zeros((hq, p.total_q), dtype=np.int32)
    for c in m["comb"]:
        q0, nrows, h0, nch, slot0 = c[:5]
        for lr in range(nrows):
            for g in range(G):
                combined[h0 + g, q0 + lr] += 1
                for ch in range(nch):
                    assert partial_slots.pop(slot0 + ch * m["rows"] * G + lr * G + g) == (q0 + lr, h0 + g)
    assert not partial_slots, "partial slots nobody combines"
    # every (row, head) is finalised exactly once, by the main kernel or by the combine
    assert ((rows_written + combined) == 1).all()
    return cover, m


def check_plan(p, **kw):
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, num_cus=kw.pop("num_cus", NCU), **kw)
    cover, m = rasterise(p, plan)
    mask = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k)
    for h in range(p.heads_q):
        assert (cover[h] == mask).all(), f"head {h}: coverage differs from the mask"
    assert plan.info["visible_pairs"] == int(mask.sum())
    return plan, m


@pytest.mark.parametrize("seed", range(16))
def test_worklist_covers_mask_exactly_once(seed):
    rng = np.random.default_rng(seed)
    tq, tk = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    p = W.random_problem(seed, tq, tk, hq, hkv, 64, n_types=2 if seed < 10 else 4)
    check_plan(p)


@pytest.mark.parametrize("seed", range(4))
def test_sliding_window_bands_cover_mask_exactly_once(seed):
    # sliding windows written as bi-causal slices: rows [s, e) of a document see
    # the w keys ending at their own position (keys [i - w + 1, i + 1) clipped to
    # the document), i.e. a band slice q [s, e) x k [s - w + 1, e) cut at s
    rng = np.random.default_rng(300 + seed)
    T, w = int(rng.integers(200, 700)), int(rng.integers(1, 200))
    docs = [0] + sorted(rng.choice(np.arange(1, T), size=2, replace=False).tolist()) + [T]
    sl = []
    for s0, e0 in zip(docs[:-1], docs[1:]):
        # rows [s0, min(e0, s0 + w - 1)) see the document start: causal part
        h = min(e0, s0 + w - 1)
        if h > s0:
            sl.append(((s0, h), (s0, h), W.CAUSAL))
        if e0 > h:
            sl.append(((h, e0), (h - w + 1, e0), W.BICAUSAL))
    p = W.make_problem("window", T, T, 4, 1, 64, sl)
    check_plan(p)
    check_plan(p, split_tiles=2)


@pytest.mark.parametrize("seed", range(6))
def test_forced_split_covers_mask_exactly_once(seed):
    rng = np.random.default_rng(50 + seed)
    p = W.random_problem(50 + seed, int(rng.integers(40, 260)), int(rng.integers(200, 700)), 4, 1, 128)
    plan, m = check_plan(p, split_tiles=int(rng.integers(1, 4)), max_splits=int(rng.integers(2, 6)))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_scaled_configs_cover_mask(cfg):
    p = W.scaled(cfg, {1: 1, 2: 16, 3: 16, 4: 32}[cfg])
    p.heads_q, p.heads_kv = min(p.heads_q, 8), min(p.heads_kv, 2)
    check_plan(p)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_visible_pairs_match_oracle_at_full_size(cfg):
    p = W.config(cfg)
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, num_cus=NCU)
    if cfg == 5:
        expect = 131072 * 131073 // 2
    else:
        expect = oracle.count_visible_pairs(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k)
    assert plan.info["visible_pairs"] == expect
    assert plan.info["computed_pairs"] >= expect


def test_plan_meta_layout_and_order():
    p = W.config(3)
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, num_cus=NCU)
    i = plan.info
    assert i["meta_bytes"] == 4 * (HDR + IREC * i["num_items"] + REC * (i["num_runs"] + i["num_combine"]))
    m = parse(plan.meta_host())
    assert m["G"] == 4 and m["rows"] == 32 and m["bn"] == 64
    cost = m["items"][:, 6] + 2 * (m["items"][:, 4] > 0)
    # longest first, except that the second half of the first wave (items NCU .. 2 NCU - 1,
    # in q-tile blocks of Hq / G items) runs shortest first, pairing long and short items
    nb = p.heads_q // m["G"]
    assert (np.diff(cost[:NCU]) <= 0).all() and (np.diff(cost[2 * NCU:]) <= 0).all(), "not longest-first"
    blocks = cost[NCU:2 * NCU].reshape(-1, nb)
    assert (blocks == blocks[:, :1]).all(), "a q-tile block was split"
    assert (np.diff(blocks[:, 0]) >= 0).all(), "second half of the first wave is not shortest-first"
    assert cost[2 * NCU - 1] >= cost[2 * NCU], "the reversed wave must not reach into the tail"
    # per-document causal: one run per item, every row of the problem in some item
    assert (m["items"][:, 4] == 1).all()


def test_auto_split_only_when_items_cannot_fill_the_device():
    # one long causal sequence with few heads: items far longer than a fair share -> split
    p = W.make_problem("long_few", 256, 65536, 4, 1, 128, [((0, 256), (0, 65536), W.CAUSAL)])
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, num_cus=NCU)
    assert plan.info["num_split_items"] > 0 and plan.info["num_combine"] > 0
    assert plan.info["workspace_bytes"] > 0
    # the packed-document workload fills the device without splitting
    p3 = W.config(3)
    plan3 = ffa.Plan(p3.q_ranges, p3.k_ranges, p3.mask_types, p3.total_q, p3.total_k, p3.heads_q, p3.heads_kv,
                     p3.head_dim, num_cus=NCU)
    assert plan3.info["num_split_items"] == 0 and plan3.info["workspace_bytes"] == 0
    # never split below the minimum chunk
    plan_n = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                      p.head_dim, num_cus=NCU, split_tiles=-1)
    assert plan_n.info["num_split_items"] == 0


def test_auto_split_cost_model_cases():
    # Cases whose answer is fixed by the cost model's measured constants (about 1.8 us
    # per tile per slot, 3 tiles per item, 6 us + partial traffic for the combine):
    # (a) as many items as resident slots, each at most 64 tiles: splitting cannot pay
    #     for the combine pass -- the rectangular causal GQA workload stays unsplit;
    p2 = W.config(2)
    plan2 = ffa.Plan(p2.q_ranges, p2.k_ranges, p2.mask_types, p2.total_q, p2.total_k, p2.heads_q,
                     p2.heads_kv, p2.head_dim, num_cus=NCU)
    assert plan2.info["num_items"] == 512 and plan2.info["num_split_items"] == 0
    # (b) a quarter of the slots busy with items of up to 256 tiles: split;
    p = W.make_problem("one_head", 16384, 16384, 1, 1, 128, [((0, 16384), (0, 16384), W.CAUSAL)])
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, num_cus=NCU)
    assert plan.info["num_split_items"] > 0 and plan.info["num_items"] > 2 * NCU
    # (c) the same sequence on a device with 8 CUs already has 8x more work per slot
    #     than there are items to balance: no split.
    plan_s = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                      p.head_dim, num_cus=8)
    assert plan_s.info["num_split_items"] == 0


def test_fwd_rejects_bad_arguments_without_launching(lib):
    p = ffa.Plan([[0, 64]], [[0, 64]], [1], 64, 64, 2, 2, 128, num_cus=NCU)
    fake = 1 << 20  # never dereferenced: validation fails first
    def call(**kw):
        a = dict(meta=fake, batch=1, q=fake, k=fake, v=fake, out=fake, lse=fake, st=2 * 128, sh=128,
                 scale=0.1, ws=None, wsb=0)
        a.update(kw)
        return lib.ffa_fwd(p.handle, a["meta"], a["batch"], a["q"], 0, a["st"], a["sh"], a["k"], 0, a["st"],
                           a["sh"], a["v"], 0, a["st"], a["sh"], a["out"], 0, a["st"], a["sh"], a["lse"], 0, 2, 1,
                           a["scale"], a.get("ex"), a["ws"], a["wsb"], None)
    assert call(batch=0) == 11
    assert call(scale=float("nan")) == 11
    assert call(scale=0.0) == 11
    assert call(meta=None) == 1
    assert call(q=None) == 1
    assert call(k=None) == 1
    assert call(q=fake + 2) == 10
    assert call(st=2 * 128 + 4) == 10
    assert lib.ffa_fwd(None, fake, 1, fake, 0, 1, 1, fake, 0, 1, 1, fake, 0, 1, 1, fake, 0, 1, 1, fake, 0, 1, 1,
                       0.1, None, None, 0, None) == 1
    # sink / softcap arguments
    ex = ffa.AttnExtras()
    ex.softcap = -1.0
    assert call(ex=ctypes.byref(ex)) == 11
    ex.softcap = float("nan")
    assert call(ex=ctypes.byref(ex)) == 11
    ex.softcap, ex.n_sink = 0.0, -1
    assert call(ex=ctypes.byref(ex)) == 11
    ex.n_sink = 2  # sink pointer NULL
    assert call(ex=ctypes.byref(ex)) == 1
    ex.n_sink, ex.dtype = 0, 7  # unknown element type
    assert call(ex=ctypes.byref(ex)) == 11
    ex.n_sink, ex.dtype, ex.sink = 70000, 0, fake  # too many sink logits
    assert call(ex=ctypes.byref(ex)) == 11
    ex.n_sink, ex.sink, ex.flags = 0, None, 2  # unknown flag bit
    assert call(ex=ctypes.byref(ex)) == 11
    assert "flags" in lib.ffa_last_error().decode()
    # a split plan without workspace
    ps = ffa.Plan([[0, 32]], [[0, 8192]], [0], 32, 8192, 4, 1, 128, num_cus=NCU, split_tiles=16)
    assert ps.info["workspace_bytes"] > 0
    assert lib.ffa_fwd(ps.handle, fake, 1, fake, 0, 512, 128, fake, 0, 128, 128, fake, 0, 128, 128, fake, 0, 512,
                       128, fake, 0, 4, 1, 0.1, None, None, 0, None) == 7
    # negative k / v token strides: the kernels address a tile with unsigned offsets
    for ks_, vs_ in ((-256, 256), (256, -256)):
        assert lib.ffa_fwd(p.handle, fake, 1, fake, 0, 256, 128, fake, 0, ks_, 128, fake, 0, vs_, 128, fake, 0,
                           256, 128, fake, 0, 2, 1, 0.1, None, None, 0, None) == 11


def test_plan_sizes_match_plan_info(lib):
    for split in (-1, 16):
        p = ffa.Plan([[0, 32]], [[0, 8192]], [0], 32, 8192, 4, 1, 128, num_cus=NCU, split_tiles=split)
        assert p.sizes() == (p.info["meta_bytes"], p.info["workspace_bytes"])
        assert (p.info["workspace_bytes"] > 0) == (split > 0)
        mb = ctypes.c_size_t(0)
        assert lib.ffa_plan_sizes(p.handle, ctypes.byref(mb), None) == 0 and mb.value == p.info["meta_bytes"]
        assert lib.ffa_plan_sizes(p.handle, None, None) == 0
    assert lib.ffa_plan_sizes(None, None, None) == 1


def test_combine_rejects_bad_arguments_without_launching(lib):
    fake = 1 << 20  # never dereferenced: validation fails first
    ps = ffa.Plan([[0, 32]], [[0, 8192]], [0], 32, 8192, 4, 1, 128, num_cus=NCU, split_tiles=16)
    wsb = ps.info["workspace_bytes"]
    assert ps.info["num_combine"] > 0

    def call(plan=ps, **kw):
        a = dict(meta=fake, batch=1, out=fake, lse=fake, st=512, sh=128, ws=fake, wsb=wsb, ex=None)
        a.update(kw)
        return lib.ffa_combine(plan.handle if plan is not None else None, a["meta"], a["batch"], a["out"], 0,
                               a["st"], a["sh"], a["lse"], 0, 4, 1, a["ex"], a["ws"], a["wsb"], None)

    assert call(plan=None) == 1
    assert call(batch=0) == 11
    assert call(meta=None) == 1
    assert call(out=None) == 1
    assert call(lse=None) == 1
    assert call(ws=None) == 7
    assert call(wsb=wsb - 4) == 7
    assert call(batch=2) == 7            # the workspace holds one batch element
    assert call(out=fake + 2) == 10
    assert call(st=512 + 4) == 10
    ex = ffa.AttnExtras()
    ex.softcap = -1.0
    assert call(ex=ctypes.byref(ex)) == 11
    # a plan that splits nothing: nothing to merge, nothing enqueued
    pn = ffa.Plan([[0, 64]], [[0, 64]], [1], 64, 64, 2, 2, 128, num_cus=NCU)
    assert pn.info["num_combine"] == 0
    assert call(plan=pn, ws=None, wsb=0) == 0


def test_largest_key_axis_keeps_its_causal_edge():
    # With a key axis of 2^30 - 2 tokens a causal bound ke - qe + 1 stays below the
    # "no bound" sentinel, so the run keeps its masked trailing tile; one more token is
    # rejected (a bound could then equal the sentinel and read as "no bound").
    nk = (1 << 30) - 2
    p = ffa.Plan([[0, 2]], [[0, nk]], [1], 2, nk, 1, 1, 128, num_cus=NCU, split_tiles=-1)
    meta = p.meta_host()
    assert p.info["num_items"] == 1
    run = meta[HDR + IREC * 1: HDR + IREC * 1 + REC]
    k0, n_tiles, n_full, k_hi, edge_base = (int(x) for x in run[:5])
    assert (k0, k_hi, edge_base) == (0, nk, nk - 2 + 1)
    assert n_tiles == -(-nk // 64) and n_full == (nk - 1) // 64 < n_tiles
    assert plan_status([[0, 2]], [[0, 2]], [1], 2, nk + 1, 1, 1, 128) == 2
    assert plan_status([[0, 2]], [[0, 2]], [1], nk + 1, 2, 1, 1, 128) == 2


def test_head_groups_of_a_kv_head_share_a_dispatch_lane():
    """Hq 64 / Hkv 8 (two head groups of 4 per kv head): within every block of 8
    consecutive items (the XCDs the dispatcher cycles through) each item's kv head
    equals its position, so both groups of a kv head run on the same L2."""
    qr, kr = [[0, 4096]], [[0, 4096]]
    plan = ffa.Plan(qr, kr, [1], 4096, 4096, 64, 8, 128, num_cus=NCU)
    m = parse(plan.meta_host())
    assert m["G"] == 4
    kv = m["items"][:, 2] // 8  # h0 / (Hq / Hkv)
    assert len(kv) % 8 == 0
    assert (kv == np.arange(len(kv)) % 8).all()
    # every (q tile, head group) pair appears exactly once
    pairs = {(int(a), int(b)) for a, b in zip(m["items"][:, 0], m["items"][:, 2])}
    assert len(pairs) == len(kv) == (4096 // 32) * 16


def test_make_extras_fields():
    # the binding's extras builder: None for plain bf16 attention, the dtype code for fp16,
    # and the rounded-weight flag (no device tensors needed for these fields)
    import torch

    assert ffa.make_extras() is None
    assert ffa.make_extras(dtype=torch.bfloat16) is None
    ex = ffa.make_extras(dtype=torch.float16)
    assert ex.dtype == 1 and ex.flags == 0 and ex.n_sink == 0
    ex = ffa.make_extras(rounded_norm=True)
    assert ex.flags == ffa.EXTRAS_ROUNDED_NORM and ex.dtype == 0 and ex.softcap == 0.0
    ex = ffa.make_extras(softcap=5.0, rounded_norm=True, dtype=torch.float16)
    assert (ex.flags, ex.dtype, ex.softcap) == (1, 1, 5.0)
