"""Pins of the oracle's attention sink and soft-capping (``oracle.attend`` /
``oracle.attend_backward`` with ``sink`` / ``softcap``) against things other than
themselves.

Sink (reading: each sink logit is one more term exp(sink) of the row's softmax
denominator, with no value).  Pinned by construction against the oracle WITHOUT
sinks: a sink logit is exactly a key whose score is that logit and whose value is
zero.  With one extra head-dim coordinate per sink token, q'[i,h] = [q[i,h],
sink/scale] and a sink key k'_s = [0, e_s] with v = 0, visible from every row
(one FULL slice over the sink keys), gives score scale * q'.k'_s = sink.  So
out and lse with sinks equal those of the augmented problem, the gradients of
q, k, v equal its gradients on the original coordinates, and d sink =
d q'[extra] / scale (summed over rows for the shared layout).  MHA (Hq = Hkv)
keeps one kv head per query head.

Softcap (reading: score -> softcap * tanh(score / softcap), 0 = off): its two
limits are closed forms -- a cap far above every score leaves attention
unchanged, a cap near 0 flattens every visible score to 0 (out = mean of the
visible v, lse = ln |V(i)|) -- and its gradient is pinned by central
differences of the forward.  The exact form between the limits is the reading
itself (the quickstart names the argument without defining it).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W


def augmented(p, q, k, v, sink, layout, scale):
    """The problem without sinks that a sink must equal (see the module docstring)."""
    tq, hq, d = q.shape
    tk = k.shape[0]
    ns = sink.shape[-2] if layout == "ssh" else sink.shape[0]
    per_row = sink if layout == "ssh" else np.broadcast_to(sink[None], (tq, ns, hq))
    q2 = np.concatenate([q, np.transpose(per_row, (0, 2, 1)) / scale], axis=2)       # [Tq, Hq, D + S]
    k2 = np.zeros((tk + ns, hq, d + ns))
    k2[:tk, :, :d] = k
    for s in range(ns):
        k2[tk + s, :, d + s] = 1.0
    v2 = np.zeros((tk + ns, hq, d + ns))  # the oracle takes v shaped like k: extra coordinates 0
    v2[:tk, :, :d] = v
    qr = np.concatenate([p.q_ranges, [[0, tq]]]).astype(np.int32)
    kr = np.concatenate([p.k_ranges, [[tk, tk + ns]]]).astype(np.int32)
    ty = np.concatenate([p.mask_types, [oracle.FULL]]).astype(np.int32)
    return q2, k2, v2, qr, kr, ty


def sink_case(seed, layout):
    rng = np.random.default_rng(1300 + seed)
    tq, tk = int(rng.integers(1, 14)), int(rng.integers(1, 14))
    h, d, ns = int(rng.choice([1, 2])), 4, int(rng.integers(1, 4))
    p = W.random_problem(1300 + seed, tq, tk, h, h, d, n_types=4)
    q = rng.standard_normal((tq, h, d))
    k = rng.standard_normal((tk, h, d))
    v = rng.standard_normal((tk, h, d))
    dout = rng.standard_normal((tq, h, d))
    sink = 2.0 * rng.standard_normal((ns, h) if layout == "sh" else (tq, ns, h))
    return p, q, k, v, dout, sink


@pytest.mark.parametrize("layout", ["sh", "ssh"])
@pytest.mark.parametrize("seed", range(6))
def test_sink_is_a_zero_value_key(seed, layout):
    p, q, k, v, dout, sink = sink_case(seed, layout)
    scale = 1.0 / math.sqrt(q.shape[2])
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink, sink_layout=layout)
    q2, k2, v2, qr, kr, ty = augmented(p, q, k, v, sink, layout, scale)
    out2, lse2 = oracle.attend(q2, k2, v2, qr, kr, ty, softmax_scale=scale)
    np.testing.assert_allclose(out, out2[:, :, :q.shape[2]], atol=1e-12, rtol=1e-12)
    assert (out2[:, :, q.shape[2]:] == 0).all()
    np.testing.assert_allclose(lse, lse2, atol=1e-12, rtol=1e-12)
    assert np.isfinite(lse).all()  # every row sees its sinks
    dq, dk, dv, ds = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types, sink=sink,
                                            sink_layout=layout, block_rows=5)
    d = q.shape[2]
    dout2 = np.concatenate([dout, np.zeros(dout.shape[:2] + (q2.shape[2] - d,))], axis=2)
    dq2, dk2, dv2 = oracle.attend_backward(q2, k2, v2, dout2, qr, kr, ty, softmax_scale=scale, block_rows=5)
    np.testing.assert_allclose(dq, dq2[:, :, :d], atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(dk, dk2[:k.shape[0], :, :d], atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(dv, dv2[:k.shape[0], :, :d], atol=1e-12, rtol=1e-10)
    extra = np.transpose(dq2[:, :, d:], (0, 2, 1)) / scale  # [Tq, S, H]: q'[extra] = sink / scale
    want = extra.sum(axis=0) if layout == "sh" else extra
    np.testing.assert_allclose(ds, want, atol=1e-12, rtol=1e-10)


def test_sink_of_minus_infinity_is_no_sink():
    p, q, k, v, dout, _ = sink_case(3, "sh")
    sink = np.full((2, q.shape[1]), -np.inf)
    a = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink)
    b = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_row_without_keys_keeps_sink_normaliser():
    # rows 0-3 are in no slice: out 0, lse = logsumexp of the sinks; their gradients are 0
    p = W.make_problem("s", 8, 8, 1, 1, 4, [((4, 8), (0, 8), W.CAUSAL)])
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal(s) for s in ((8, 1, 4), (8, 1, 4), (8, 1, 4)))
    sink = np.array([[0.3], [-1.2]])
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink)
    assert (out[:4] == 0).all()
    np.testing.assert_allclose(lse[:4, 0], np.log(np.exp(0.3) + np.exp(-1.2)), rtol=1e-15)


def fd_check(p, q, k, v, dout, grads, fwd_kw, names, seed, eps=1e-6, n_probe=10):
    rng = np.random.default_rng(seed)
    inputs = {"q": q, "k": k, "v": v}
    if "sink" in fwd_kw:
        inputs["sink"] = fwd_kw["sink"]
    for name in names:
        x = inputs[name]
        for _ in range(n_probe):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            vals = []
            for sgn in (1, -1):
                xx = x.copy()
                xx[idx] += sgn * eps
                args = dict(inputs)
                args[name] = xx
                kw = dict(fwd_kw)
                if "sink" in kw:
                    kw["sink"] = args.pop("sink")
                o, _ = oracle.attend(args["q"], args["k"], args["v"], p.q_ranges, p.k_ranges, p.mask_types, **kw)
                vals.append((o * dout).sum())
            want = (vals[0] - vals[1]) / (2 * eps)
            got = grads[name][idx]
            assert abs(got - want) <= 2e-6 * (1 + abs(want)), (name, idx, got, want)


@pytest.mark.parametrize("seed", range(6))
def test_softcap_and_sink_gradients_match_finite_differences(seed):
    p, q, k, v, dout, sink = sink_case(seed, "sh" if seed % 2 == 0 else "ssh")
    layout = "sh" if seed % 2 == 0 else "ssh"
    cap = [0.7, 2.0, 5.0][seed % 3]
    q, k = 3 * q, 3 * k  # scores well inside the cap's curved part
    dq, dk, dv, ds = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types, sink=sink,
                                            sink_layout=layout, softcap=cap, block_rows=4)
    fd_check(p, q, k, v, dout, {"q": dq, "k": dk, "v": dv, "sink": ds},
             {"sink": sink, "sink_layout": layout, "softcap": cap}, ("q", "k", "v", "sink"), seed)


@pytest.mark.parametrize("seed", range(4))
def test_softcap_gradients_without_sink_match_finite_differences(seed):
    rng = np.random.default_rng(1400 + seed)
    tq, tk = int(rng.integers(1, 12)), int(rng.integers(1, 12))
    p = W.random_problem(1400 + seed, tq, tk, 2, 1, 4, n_types=4)
    q, k, v = (rng.standard_normal(s) for s in ((tq, 2, 4), (tk, 1, 4), (tk, 1, 4)))
    dout = rng.standard_normal((tq, 2, 4))
    q = 4 * q
    dq, dk, dv = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types, softcap=1.5)
    fd_check(p, q, k, v, dout, {"q": dq, "k": dk, "v": dv}, {"softcap": 1.5}, ("q", "k", "v"), seed)


def test_large_softcap_is_no_softcap():
    p = W.random_problem(7, 40, 50, 2, 1, 8, n_types=4)
    q, k, v = W.make_qkv(p)
    a = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, softcap=1e9)
    b = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types)
    np.testing.assert_allclose(a[0], b[0], atol=1e-10)
    np.testing.assert_allclose(a[1], b[1], atol=1e-10)


def test_tiny_softcap_flattens_scores():
    # cap -> 0: every visible capped score -> 0, so out = mean of the visible v and
    # lse = ln |V(i)| (the q = 0 closed form), up to O(cap)
    p = W.random_problem(8, 40, 50, 2, 1, 8, n_types=4)
    q, k, v = W.make_qkv(p)
    out, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, softcap=1e-9)
    m = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, 40, 50)
    n = m.sum(axis=1)
    vv = v.double().numpy()
    for i in range(40):
        if n[i] == 0:
            assert np.isneginf(lse[i]).all()
            continue
        np.testing.assert_allclose(lse[i], np.log(n[i]), atol=1e-7)
        np.testing.assert_allclose(out[i, 0], vv[m[i], 0].mean(axis=0), atol=1e-7)


def test_softcap_bounds_the_log_normaliser():
    # every capped score lies in (-cap, cap): ln|V(i)| - cap < lse < ln|V(i)| + cap
    p = W.random_problem(9, 30, 30, 1, 1, 16, n_types=4)
    q, k, v = W.make_qkv(p)
    q = q * 8
    cap = 0.5
    _, lse = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, softcap=cap)
    n = oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, 30, 30).sum(axis=1)
    ok = n > 0
    assert (np.abs(lse[ok, 0] - np.log(n[ok])) < cap).all()
