"""Pins of ``oracle.total_attention`` (FlagAttention's `total`: attention probabilities
summed over the query axis) against things other than itself: brute-force loops on tiny
inputs, the row-sum identity (every row that sees a key distributes exactly 1), and the
q = 0 closed form (each such row gives 1/|V(i)| to each of its keys)."""
import math

import numpy as np
import pytest

import oracle
import workloads as W


def brute_total(q, k, p):
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = hq // hkv
    scale = 1.0 / math.sqrt(d)
    tot = np.zeros((tk, hq))
    for i in range(tq):
        keys = set()
        for (qs, qe), (ks, ke), t in zip(p.q_ranges.tolist(), p.k_ranges.tolist(), p.mask_types.tolist()):
            a, b = oracle.slice_row_interval(i, qs, qe, ks, ke, t)
            keys.update(range(max(a, 0), min(b, tk)))
        if not keys:
            continue
        for h in range(hq):
            g = h // grp
            sc = {j: scale * sum(q[i, h, x] * k[j, g, x] for x in range(d)) for j in keys}
            den = sum(math.exp(v) for v in sc.values())
            for j, v in sc.items():
                tot[j, h] += math.exp(v) / den
    return tot


@pytest.mark.parametrize("seed", range(6))
def test_total_attention_matches_brute_force(seed):
    rng = np.random.default_rng(2000 + seed)
    tq, tk = int(rng.integers(1, 10)), int(rng.integers(1, 10))
    p = W.random_problem(2000 + seed, tq, tk, 2, 1, 3, n_types=4)
    q, k = rng.standard_normal((tq, 2, 3)), rng.standard_normal((tk, 1, 3))
    np.testing.assert_allclose(oracle.total_attention(q, k, p.q_ranges, p.k_ranges, p.mask_types),
                               brute_total(q, k, p), atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_total_attention_sums_to_rows_that_see_keys(seed):
    p = W.random_problem(2100 + seed, 60, 70, 4, 2, 8, n_types=4)
    q, k, _ = W.make_qkv(p)
    tot = oracle.total_attention(q, k, p.q_ranges, p.k_ranges, p.mask_types)
    seen = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, 60, 70).any(axis=1).sum()
    np.testing.assert_allclose(tot.sum(axis=0), np.full(4, float(seen)), rtol=1e-12)


def test_total_attention_q_zero_closed_form():
    p = W.random_problem(2200, 50, 40, 2, 1, 8, n_types=4)
    q, k, _ = W.make_qkv(p, q_zero=True)
    m = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, 50, 40)
    n = m.sum(axis=1)
    want = (m[n > 0] / n[n > 0, None]).sum(axis=0)
    tot = oracle.total_attention(q, k, p.q_ranges, p.k_ranges, p.mask_types)
    for h in range(2):
        np.testing.assert_allclose(tot[:, h], want, atol=1e-12)


def test_total_attention_with_sinks_loses_the_sink_mass():
    # with sinks each row distributes 1 - sum_s exp(sink_s - lse) over its keys
    p = W.random_problem(2300, 30, 30, 2, 2, 8, n_types=4)
    q, k, v = W.make_qkv(p)
    sink = np.array([[0.5, -0.3], [1.0, 0.2]])
    tot = oracle.total_attention(q, k, p.q_ranges, p.k_ranges, p.mask_types, sink=sink)
    _, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink)
    seen = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, 30, 30).any(axis=1)
    want = (1.0 - np.exp(sink[None, :, :] - lse[:, None, :]).sum(axis=1))[seen].sum(axis=0)
    np.testing.assert_allclose(tot.sum(axis=0), want, rtol=1e-12)


def test_pins_catch_total_attention_mutations(monkeypatch):
    import inspect
    import types

    import oracle.fwd as oracle_fwd

    mutations = {
        "unnormalised": ("tot[cols, h] += p.sum(axis=0)", "tot[cols, h] += e.sum(axis=0)"),
        "sinks_ignored": ("den = e.sum(axis=1) + np.exp(sk - safe[:, None]).sum(axis=1)", "den = e.sum(axis=1)"),
        "scale_dropped": ("s = np.where(mk, capped_scores((q[rb, h, :] @ kg.T) * scale, softcap), -np.inf)",
                          "s = np.where(mk, capped_scores((q[rb, h, :] @ kg.T), softcap), -np.inf)"),
    }
    src = inspect.getsource(oracle_fwd)
    for name, (old, new) in mutations.items():
        assert src.count(old) == 1, name
        mod = types.ModuleType("oracle_total_mutant")
        exec(compile(src.replace(old, new), "oracle_total_mutant", "exec"), mod.__dict__)
        monkeypatch.setattr(oracle, "total_attention", mod.total_attention)
        failed = 0
        for pin in (lambda: test_total_attention_matches_brute_force(0),
                    lambda: test_total_attention_sums_to_rows_that_see_keys(0),
                    test_total_attention_q_zero_closed_form,
                    test_total_attention_with_sinks_loses_the_sink_mass):
            try:
                pin()
            except AssertionError:
                failed += 1
        assert failed > 0, f"no pin caught {name}"
