"""Pins for the CPU oracle against things other than itself.

- brute force: pure-Python loops with math.exp / math.fsum over a visibility
  predicate written from the pages' interval formula (MagiAttention blog page
  "Calculate KV Interval Boundaries for Mask Types": start = k_start +
  (type & 2 ? q_idx - q_start : 0), end = k_end - (type & 1 ? q_end - q_idx - 1 : 0));
- the mask figures the MagiAttention quickstart prints (tests/golden/);
- torch's fp64 scaled_dot_product_attention for the special cases that it can
  express (no mask, square causal, bottom-right causal, per-document causal, GQA);
- closed forms (q = 0 gives lse = ln |V(i)|; constant v gives out = v; visible
  pair counts of the five workloads) and the split / merge identity of the
  FlagAttention split-KV combine.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers (test-side, independent)

def formula_visible(i, j, qs, qe, ks, ke, t):
    """The pages' interval formula, used literally as a predicate."""
    if not (qs <= i < qe):
        return False
    start = ks + ((i - qs) if (t & 2) else 0)
    end = ke - ((qe - i - 1) if (t & 1) else 0)
    return start <= j < end


def brute_force(q, k, v, slices, scale):
    """Pure-Python reference: loops, math.exp, math.fsum."""
    q = q.to(torch.float64).tolist()
    k = k.to(torch.float64).tolist()
    v = v.to(torch.float64).tolist()
    tq, hq, d = len(q), len(q[0]), len(q[0][0])
    tk, hkv = len(k), len(k[0])
    grp = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(tq)]
    lse = [[-math.inf] * hq for _ in range(tq)]
    for i in range(tq):
        vis = [j for j in range(tk) if any(formula_visible(i, j, *s) for s in slices)]
        if not vis:
            continue
        for h in range(hq):
            g = h // grp
            sc = {j: scale * math.fsum(q[i][h][x] * k[j][g][x] for x in range(d)) for j in vis}
            mx = max(sc.values())
            den = math.fsum(math.exp(sc[j] - mx) for j in vis)
            lse[i][h] = mx + math.log(den)
            for x in range(d):
                out[i][h][x] = math.fsum(math.exp(sc[j] - lse[i][h]) * v[j][g][x] for j in vis)
    return np.array(out), np.array(lse)


def slices_of(p):
    return [(int(a), int(b), int(c), int(e), int(t))
            for (a, b), (c, e), t in zip(p.q_ranges.tolist(), p.k_ranges.tolist(), p.mask_types.tolist())]


def load_golden(name):
    meta, rows, slices = {}, [], []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.rstrip("\n")
            if not line or line.startswith("#"):
                continue
            if line.startswith("slice:"):
                slices.append(tuple(int(x) for x in line.split()[1:]))
            elif ":" in line:
                key, val = line.split(":", 1)
                meta[key.strip()] = int(val)
            else:
                rows.append([c == "*" for c in line.split()])
    return meta, slices, np.array(rows)


def any_visible_cells(mask, cells):
    tq, tk = mask.shape
    return mask.reshape(cells, tq // cells, cells, tk // cells).any(axis=(1, 3))


# ---------------------------------------------------------------- mask geometry

@pytest.mark.parametrize("seed", range(16))
def test_mask_equals_interval_formula(seed):
    rng = np.random.default_rng(seed)
    tq, tk = int(rng.integers(1, 40)), int(rng.integers(1, 40))
    p = W.random_problem(seed, tq, tk, 1, 1, 8, n_types=2 if seed < 8 else 4)
    m = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, tq, tk)
    sl = slices_of(p)
    ref = np.array([[any(formula_visible(i, j, *s) for s in sl) for j in range(tk)] for i in range(tq)])
    assert (m == ref).all()


def test_golden_full_then_causal_picture():
    meta, slices, pic = load_golden("quickstart_full_then_causal_mask.txt")
    qr = [(s[0], s[1]) for s in slices]
    kr = [(s[2], s[3]) for s in slices]
    ty = [s[4] for s in slices]
    m = oracle.dense_mask(qr, kr, ty, meta["total_q"], meta["total_k"])
    cells = any_visible_cells(m, meta["cells"])
    assert cells.shape == pic.shape
    assert (cells == pic).all()


def test_golden_block_causal_picture():
    meta, slices, pic = load_golden("quickstart_block_causal_mask.txt")
    qr = [(s[0], s[1]) for s in slices]
    kr = [(s[2], s[3]) for s in slices]
    ty = [s[4] for s in slices]
    n = meta["cells"]
    # any-visible reduction, computed block of rows at a time (32768^2 mask is 1 GiB as bool)
    step = meta["total_q"] // n
    cells = np.zeros((n, n), dtype=bool)
    for r in range(n):
        rows = np.arange(r * step, (r + 1) * step, 64)  # FULL slices: rows in a block share intervals
        mk = oracle.mask_rows(rows, qr, kr, ty, meta["total_k"])
        cells[r] = mk.reshape(len(rows), n, -1).any(axis=(0, 2))
    # the picture's 2x2 blocks are uniform; reduce it to n x n
    f = pic.shape[0] // n
    blocks = pic.reshape(n, f, n, f)
    assert (blocks.all(axis=(1, 3)) == blocks.any(axis=(1, 3))).all()
    assert (blocks.any(axis=(1, 3)) == cells).all()


# ---------------------------------------------------------------- values vs brute force

@pytest.mark.parametrize("seed", range(12))
def test_oracle_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    tq, tk = int(rng.integers(1, 24)), int(rng.integers(1, 24))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2]))
    d = int(rng.choice([4, 8]))
    p = W.random_problem(seed, tq, tk, hq, hkv, d, n_types=2 if seed < 8 else 4)
    q, k, v = W.make_qkv(p, seed=seed)
    scale = float(rng.uniform(0.1, 1.0))
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, scale, block_rows=5)
    bo, bl = brute_force(q, k, v, slices_of(p), scale)
    assert np.array_equal(np.isinf(lse), np.isinf(bl))
    fin = np.isfinite(bl)
    assert np.allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)
    assert np.allclose(out, bo, rtol=0, atol=1e-12)


def test_empty_rows_give_zero_and_neg_inf():
    # rows 0..3 have no slice; rows 4..7 have a causal slice with M > N so the first rows see nothing
    p = W.make_problem("empty", 12, 6, 2, 1, 8, [((4, 12), (0, 3), W.CAUSAL)])
    q, k, v = W.make_qkv(p, seed=3)
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    # row i in [4,12) sees keys [0, 3 - (11 - i)) -> first visible row is i = 9
    assert np.isneginf(lse[:9]).all() and np.isfinite(lse[9:]).all()
    assert (out[:9] == 0).all()
    assert not np.isnan(out).any() and not np.isnan(lse).any()


# ---------------------------------------------------------------- special cases vs torch SDPA (fp64, CPU)

def sdpa(q, k, v, **kw):
    # q [T,H,D] -> [1,H,T,D]
    qq = q.to(torch.float64).permute(1, 0, 2).unsqueeze(0)
    kk = k.to(torch.float64).permute(1, 0, 2).unsqueeze(0)
    vv = v.to(torch.float64).permute(1, 0, 2).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, **kw)
    return o.squeeze(0).permute(1, 0, 2).numpy()


def test_full_slice_is_dense_attention():
    p = W.make_problem("full", 40, 56, 3, 3, 16, [((0, 40), (0, 56), W.FULL)])
    q, k, v = W.make_qkv(p, seed=5)
    out, _ = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    assert np.allclose(out, sdpa(q, k, v), rtol=0, atol=1e-10)


def test_square_causal_slice_is_causal_attention():
    p = W.make_problem("causal", 48, 48, 2, 2, 16, [((0, 48), (0, 48), W.CAUSAL)])
    q, k, v = W.make_qkv(p, seed=6)
    out, _ = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    assert np.allclose(out, sdpa(q, k, v, is_causal=True), rtol=0, atol=1e-10)


def test_rect_causal_is_bottom_right():
    from torch.nn.attention.bias import causal_lower_right

    M, N = 24, 56
    p = W.make_problem("rect", M, N, 2, 2, 16, [((0, M), (0, N), W.CAUSAL)])
    q, k, v = W.make_qkv(p, seed=7)
    out, _ = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    ref = sdpa(q, k, v, attn_mask=causal_lower_right(M, N))
    assert np.allclose(out, ref, rtol=0, atol=1e-10)
    # FlagAttention's piecewise-attention text gives the same alignment: row m,
    # key n is at signed offset N - M + m - n, visible when >= 0.
    m = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, M, N)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    assert (m == (N - M + mm - nn >= 0)).all()


def test_per_document_causal_is_per_document_sdpa():
    docs = [5, 17, 1, 9]
    sl, s = [], 0
    for n in docs:
        sl.append(((s, s + n), (s, s + n), W.CAUSAL))
        s += n
    p = W.make_problem("docs", s, s, 2, 1, 8, sl)
    q, k, v = W.make_qkv(p, seed=8)
    out, _ = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    s = 0
    kk = k.repeat_interleave(2, dim=1)
    vv = v.repeat_interleave(2, dim=1)
    for n in docs:
        ref = sdpa(q[s:s + n], kk[s:s + n], vv[s:s + n], is_causal=True)
        assert np.allclose(out[s:s + n], ref, rtol=0, atol=1e-10)
        s += n


def test_gqa_is_mha_with_repeated_kv():
    p = W.make_problem("gqa", 20, 30, 8, 2, 8, [((0, 20), (0, 30), W.CAUSAL)])
    q, k, v = W.make_qkv(p, seed=9)
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    k4 = k.repeat_interleave(4, dim=1)
    v4 = v.repeat_interleave(4, dim=1)
    p4 = W.make_problem("mha", 20, 30, 8, 8, 8, [((0, 20), (0, 30), W.CAUSAL)])
    out4, lse4 = oracle.attend(q, k4, v4, p4.q_ranges, p4.k_ranges, p4.mask_types)
    assert np.allclose(out, out4, atol=1e-13) and np.allclose(lse, lse4, atol=1e-13)
    # and head h uses kv head h // 4 (contiguous groups), not h % 2
    from torch.nn.attention.bias import causal_lower_right

    ref = sdpa(q, k4, v4, attn_mask=causal_lower_right(20, 30))
    assert np.allclose(out, ref, atol=1e-10)


# ---------------------------------------------------------------- closed forms and identities

@pytest.mark.parametrize("seed", range(4))
def test_q_zero_closed_form(seed):
    # q = 0: every score is 0, so lse = ln |V(i)| and out = mean of the visible v
    p = W.random_problem(200 + seed, 30, 26, 2, 1, 8)
    q, k, v = W.make_qkv(p, seed=seed, q_zero=True)
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    sl = slices_of(p)
    vv = v.to(torch.float64).numpy()
    for i in range(p.total_q):
        vis = [j for j in range(p.total_k) if any(formula_visible(i, j, *s) for s in sl)]
        for h in range(2):
            if not vis:
                assert lse[i, h] == -np.inf and (out[i, h] == 0).all()
            else:
                assert abs(lse[i, h] - math.log(len(vis))) < 1e-12
                assert np.allclose(out[i, h], vv[vis, 0].mean(axis=0), atol=1e-12)


def test_constant_v_gives_constant_out():
    p = W.random_problem(300, 33, 41, 4, 2, 8)
    q, k, _ = W.make_qkv(p, seed=1)
    v = torch.full_like(k, 0.375)
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    ne = np.isfinite(lse)
    assert np.allclose(out[ne], 0.375, atol=1e-13)
    assert (out[~ne] == 0).all()


@pytest.mark.parametrize("seed", range(4))
def test_lse_is_logsumexp_of_masked_scores(seed):
    p = W.random_problem(400 + seed, 25, 31, 2, 2, 8)
    q, k, v = W.make_qkv(p, seed=seed)
    _, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, softmax_scale=0.3)
    sl = slices_of(p)
    vis = torch.tensor([[any(formula_visible(i, j, *s) for s in sl) for j in range(p.total_k)]
                        for i in range(p.total_q)])
    for h in range(2):
        s = 0.3 * (q[:, h].double() @ k[:, h].double().T)
        s = s.masked_fill(~vis, -math.inf)
        ref = torch.logsumexp(s, dim=1).numpy()
        assert np.array_equal(np.isinf(ref), np.isinf(lse[:, h]))
        fin = np.isfinite(ref)
        assert np.allclose(lse[fin, h], ref[fin], atol=1e-12)


@pytest.mark.parametrize("kind", ["full", "causal"])
def test_split_and_merge_reproduces_single_slice(kind):
    M, N = 32, 64
    t = W.FULL if kind == "full" else W.CAUSAL
    p = W.make_problem("one", M, N, 2, 1, 16, [((0, M), (0, N), t)])
    q, k, v = W.make_qkv(p, seed=11)
    o, l = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    # split point: FULL anywhere; CAUSAL at kmid <= N - M + 1 so the left part is FULL for every row
    kmid = 23 if kind == "full" else N - M + 1
    left = ((0, M), (0, kmid), W.FULL)
    right = ((0, M), (kmid, N), t)
    pl = W.make_problem("l", M, N, 2, 1, 16, [left])
    pr = W.make_problem("r", M, N, 2, 1, 16, [right])
    o1, l1 = oracle.attend(q, k, v, pl.q_ranges, pl.k_ranges, pl.mask_types)
    o2, l2 = oracle.attend(q, k, v, pr.q_ranges, pr.k_ranges, pr.mask_types)
    om, lm = oracle.merge_partials([o1, o2], [l1, l2])
    assert np.allclose(om, o, atol=1e-12) and np.allclose(lm, l, atol=1e-12)
    # the two-slice problem gives the same result as the single slice
    p2 = W.make_problem("two", M, N, 2, 1, 16, [left, right])
    o3, l3 = oracle.attend(q, k, v, p2.q_ranges, p2.k_ranges, p2.mask_types)
    assert np.allclose(o3, o, atol=1e-12) and np.allclose(l3, l, atol=1e-12)


def test_square_inverse_causal_is_causal_on_reversed_sequences():
    # Row i of a square INVCAUSAL slice sees keys j >= i.  Reversing the order of
    # queries and keys turns that into j' <= i': torch's fp64 causal SDPA on the
    # flipped tensors, flipped back, must give the same out and lse.
    import torch.nn.functional as F
    T = 40
    p = W.make_problem("inv", T, T, 2, 1, 16, [((0, T), (0, T), W.INVCAUSAL)])
    q, k, v = W.make_qkv(p, seed=21)
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    qf, kf, vf = (x.double().flip(0) for x in (q, k, v))
    for h in range(2):
        ref = F.scaled_dot_product_attention(qf[:, h][None], kf[:, 0][None], vf[:, 0][None], is_causal=True)[0].flip(0)
        assert np.allclose(out[:, h], ref.numpy(), atol=1e-12)
        s = (qf[:, h] @ kf[:, 0].T) / math.sqrt(16)
        s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), -math.inf)
        assert np.allclose(lse[:, h], torch.logsumexp(s, dim=1).flip(0).numpy(), atol=1e-12)


def test_square_bicausal_sees_only_its_diagonal_key():
    # A square BICAUSAL slice leaves each row exactly one key, its own:
    # out = v[i], lse = scale * q[i] . k[i].
    T, D = 24, 8
    p = W.make_problem("bi", T, T, 2, 2, D, [((0, T), (0, T), W.BICAUSAL)])
    q, k, v = W.make_qkv(p, seed=22)
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    qd, kd, vd = q.double(), k.double(), v.double()
    assert np.allclose(out, vd.numpy(), atol=1e-12)
    assert np.allclose(lse, ((qd * kd).sum(-1) / math.sqrt(D)).numpy(), atol=1e-12)


def test_bicausal_band_splits_into_inverse_causal_and_causal():
    # A BICAUSAL slice of M queries over N >= 2M - 1 keys is a band of width
    # w = N - M + 1 >= M.  Cut its keys at kmid in [M - 1, w]: row i sees
    # [i, kmid) through the left part (INVCAUSAL over [0, kmid)) and
    # [kmid, N - (M - 1 - i)) through the right part (CAUSAL over [kmid, N)).
    # Merging the two by logsumexp must give the band.
    M, N = 12, 30
    p = W.make_problem("band", M, N, 2, 1, 16, [((0, M), (0, N), W.BICAUSAL)])
    q, k, v = W.make_qkv(p, seed=23)
    o, l = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    for kmid in (M - 1, 15, N - M + 1):
        pl = W.make_problem("l", M, N, 2, 1, 16, [((0, M), (0, kmid), W.INVCAUSAL)])
        pr = W.make_problem("r", M, N, 2, 1, 16, [((0, M), (kmid, N), W.CAUSAL)])
        o1, l1 = oracle.attend(q, k, v, pl.q_ranges, pl.k_ranges, pl.mask_types)
        o2, l2 = oracle.attend(q, k, v, pr.q_ranges, pr.k_ranges, pr.mask_types)
        om, lm = oracle.merge_partials([o1, o2], [l1, l2])
        assert np.allclose(om, o, atol=1e-12) and np.allclose(lm, l, atol=1e-12)
    # the band has exactly w keys on every row
    m = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, M, N)
    assert (m.sum(axis=1) == N - M + 1).all()


def test_merge_with_empty_partial():
    o1 = np.ones((3, 4))
    l1 = np.array([0.5, -np.inf, 1.0])
    o2 = np.zeros((3, 4))
    l2 = np.array([-np.inf, -np.inf, 1.0])
    o, l = oracle.merge_partials([o1, o2], [l1, l2])
    assert l[0] == 0.5 and np.isneginf(l[1]) and abs(l[2] - (1.0 + math.log(2))) < 1e-15
    assert np.allclose(o[0], 1) and (o[1] == 0).all() and np.allclose(o[2], 0.5)


# ---------------------------------------------------------------- visible-pair counts (FLOP metric)

def test_visible_pair_counts_closed_forms():
    c1 = W.config(1)
    assert oracle.count_visible_pairs(c1.q_ranges, c1.k_ranges, c1.mask_types, 256, 256) == 256 * 257 // 2
    c2 = W.config(2)
    # bottom-right causal 2048 x 4096: row m sees 2049 + m keys
    per_batch = sum(2049 + m for m in range(2048))
    assert oracle.count_visible_pairs(c2.q_ranges, c2.k_ranges, c2.mask_types, 4096, 8192) == 2 * per_batch
    c3 = W.config(3)
    assert sum(c3.docs) == 16384
    assert oracle.count_visible_pairs(c3.q_ranges, c3.k_ranges, c3.mask_types, 16384, 16384) == \
        sum(n * (n + 1) // 2 for n in c3.docs)
    c4 = W.config(4)
    assert sum(c4.docs) == 32768 - 512
    expect = 512 * 512
    for n in c4.docs:
        p = n // 4
        expect += p * p + (n * (n + 1) // 2 - p * (p + 1) // 2) + n * 512
    assert oracle.count_visible_pairs(c4.q_ranges, c4.k_ranges, c4.mask_types, 32768, 32768) == expect


def test_visible_pair_count_matches_mask_sum():
    for seed in range(6):
        p = W.random_problem(500 + seed, 37, 29, 1, 1, 4)
        m = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, 37, 29)
        assert oracle.count_visible_pairs(p.q_ranges, p.k_ranges, p.mask_types, 37, 29) == int(m.sum())
    # overlapping slices (the oracle's mask is their union): two 10 x 10 FULL squares that
    # share a 5 x 5 corner cover 175 pairs; a causal square under a FULL one covers the square
    assert oracle.count_visible_pairs([[0, 10], [5, 15]], [[0, 10], [5, 15]], [0, 0], 15, 15) == 175
    assert oracle.count_visible_pairs([[0, 8], [0, 8]], [[0, 8], [0, 8]], [1, 0], 8, 8) == 64
    rng = np.random.default_rng(77)
    for _ in range(20):
        qr = np.sort(rng.integers(0, 30, size=(4, 2)), axis=1)
        kr = np.sort(rng.integers(0, 25, size=(4, 2)), axis=1)
        ty = rng.integers(0, 4, size=4)
        m = oracle.dense_mask(qr, kr, ty, 30, 25)
        assert oracle.count_visible_pairs(qr, kr, ty, 30, 25) == int(m.sum())


def test_config_doc_lists():
    # the seeded generators give the document lists the workload recipe fixes
    assert W.config(3).docs == [7882, 128, 1556, 580, 651, 825, 136, 812, 431, 3383]
    assert W.config(4).docs == [6091, 7755, 7282, 4439, 6689]
