"""Pins of the fp64 backward oracle (``oracle.attend_backward``) against things other
than itself:

- central finite differences of the forward oracle's loss L = sum(out * dout) on tiny
  random problems with all four mask types (the backward is the derivative of the
  forward definition; the pages give no gradient formula of their own);
- torch's fp64 autograd through ``scaled_dot_product_attention`` for the masks it can
  express (no mask, square causal, bottom-right causal via ``causal_lower_right``,
  per-document causal, GQA by repeating kv heads);
- closed forms: rows that see nothing get dq = 0, keys nobody sees get dk = dv = 0,
  and since every visible row's weights sum to one, sum_j dv[j] = sum of dout over the
  rows that see something.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def loss_and_grads_fd(p, q, k, v, dout, eps=1e-6, n_probe=12, seed=0):
    """Central differences of L = sum(out * dout) for n_probe random entries of each input."""
    rng = np.random.default_rng(seed)
    res = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        probes = []
        for _ in range(n_probe):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            op, _ = oracle.attend(args["q"], args["k"], args["v"], p.q_ranges, p.k_ranges, p.mask_types)
            args[name] = xm
            om, _ = oracle.attend(args["q"], args["k"], args["v"], p.q_ranges, p.k_ranges, p.mask_types)
            probes.append((idx, float(((op - om) * dout).sum() / (2 * eps))))
        res[name] = probes
    return res


@pytest.mark.parametrize("seed", range(8))
def test_backward_matches_finite_differences(seed):
    rng = np.random.default_rng(500 + seed)
    tq, tk = int(rng.integers(1, 12)), int(rng.integers(1, 12))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2]))
    p = W.random_problem(500 + seed, tq, tk, hq, hkv, 4, n_types=4)
    q = rng.standard_normal((tq, hq, 4))
    k = rng.standard_normal((tk, hkv, 4))
    v = rng.standard_normal((tk, hkv, 4))
    dout = rng.standard_normal((tq, hq, 4))
    dq, dk, dv = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types, block_rows=3)
    fd = loss_and_grads_fd(p, q, k, v, dout, seed=seed)
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        for idx, val in fd[name]:
            assert abs(g[idx] - val) <= 1e-6 * (1 + abs(val)), (name, idx, g[idx], val)


def torch_grads(q, k, v, dout, fn):
    """fp64 autograd of sum(fn(q, k, v) * dout) with q [T,H,D] -> SDPA layout [1,H,T,D]."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = fn(qt, kt, vt)
    (out * torch.tensor(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def sdpa(qt, kt, vt, **kw):
    import torch.nn.functional as F
    rep = qt.shape[1] // kt.shape[1]
    kk = kt.repeat_interleave(rep, dim=1)
    vv = vt.repeat_interleave(rep, dim=1)
    o = F.scaled_dot_product_attention(qt.permute(1, 0, 2)[None], kk.permute(1, 0, 2)[None],
                                       vv.permute(1, 0, 2)[None], **kw)
    return o[0].permute(1, 0, 2)


def check_against(p, fn, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((p.total_q, p.heads_q, p.head_dim))
    k = rng.standard_normal((p.total_k, p.heads_kv, p.head_dim))
    v = rng.standard_normal((p.total_k, p.heads_kv, p.head_dim))
    dout = rng.standard_normal((p.total_q, p.heads_q, p.head_dim))
    got = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types, block_rows=7)
    ref = torch_grads(q, k, v, dout, fn)
    for g, r in zip(got, ref):
        assert np.allclose(g, r, atol=1e-11, rtol=0)


def test_full_slice_gradients_are_sdpa_gradients():
    p = W.make_problem("full", 20, 28, 4, 2, 8, [((0, 20), (0, 28), W.FULL)])
    check_against(p, lambda q, k, v: sdpa(q, k, v), 1)


def test_square_causal_gradients_are_sdpa_gradients():
    p = W.make_problem("causal", 24, 24, 2, 1, 8, [((0, 24), (0, 24), W.CAUSAL)])
    check_against(p, lambda q, k, v: sdpa(q, k, v, is_causal=True), 2)


def test_rect_causal_gradients_are_bottom_right_sdpa_gradients():
    from torch.nn.attention.bias import causal_lower_right
    M, N = 10, 26
    p = W.make_problem("rect", M, N, 2, 2, 8, [((0, M), (0, N), W.CAUSAL)])
    check_against(p, lambda q, k, v: sdpa(q, k, v, attn_mask=causal_lower_right(M, N)), 3)


def test_per_document_causal_gradients():
    docs = [0, 7, 19, 30]
    sl = [((a, b), (a, b), W.CAUSAL) for a, b in zip(docs[:-1], docs[1:])]
    p = W.make_problem("docs", 30, 30, 4, 1, 8, sl)

    def fn(q, k, v):
        return torch.cat([sdpa(q[a:b], k[a:b], v[a:b], is_causal=True) for a, b in zip(docs[:-1], docs[1:])])

    check_against(p, fn, 4)


def test_rows_and_keys_outside_the_mask_get_zero_gradient():
    # rows 0..3 have no slice; keys 10..11 are seen by nobody
    p = W.make_problem("gaps", 12, 12, 2, 1, 8, [((4, 12), (0, 10), W.CAUSAL)])
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal(s) for s in ((12, 2, 8), (12, 1, 8), (12, 1, 8)))
    dout = rng.standard_normal((12, 2, 8))
    dq, dk, dv = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types)
    # row i in [4, 12) sees keys [0, 10 - (11 - i)) = [0, i - 1): rows 4.. see 3.. keys
    assert (dq[:4] == 0).all() and np.abs(dq[4:]).min(axis=-1).min() > 0
    assert (dk[10:] == 0).all() and (dv[10:] == 0).all()


@pytest.mark.parametrize("seed", range(3))
def test_dv_sums_to_dout_of_visible_rows(seed):
    rng = np.random.default_rng(40 + seed)
    p = W.random_problem(40 + seed, 30, 30, 4, 2, 8, n_types=4)
    q, k, v = (rng.standard_normal(s) for s in ((30, 4, 8), (30, 2, 8), (30, 2, 8)))
    dout = rng.standard_normal((30, 4, 8))
    _, _, dv = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types)
    m = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, 30, 30)
    seen = m.any(axis=1)
    for g in range(2):
        want = dout[seen][:, 2 * g:2 * g + 2, :].sum(axis=(0, 1))
        assert np.allclose(dv[:, g, :].sum(axis=0), want, atol=1e-12)
