"""GPU parity of attention sink and soft-capping through the C ABI (forward and backward)
against the fp64 oracle (``oracle.attend`` / ``attend_backward`` with sink / softcap).

Forward tolerances as for plain attention: out max-abs <= 2e-2, mean-abs <= 2e-3,
lse abs <= 1e-3.  Backward: the FlagAttention rule of test_gpu_bwd (error at most
twice that of the same-precision PyTorch backward, plus 1e-3 of max(max|ref|, 0.01)),
for dq, dk, dv and d sink.  Sink layouts: "sh" [S_sink, Hq] (shared by every row) and
"ssh" [Tq, S_sink, Hq] (per row).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

OUT_MAX, OUT_MEAN, LSE_ABS = 2e-2, 2e-3, 1e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_sink(p, layout, n, seed):
    g = torch.Generator().manual_seed(seed)
    shape = (n, p.heads_q) if layout == "sh" else (p.total_q, n, p.heads_q)
    return 2.0 * torch.randn(shape, generator=g, dtype=torch.float32)


def fwd(ffa, p, q, k, v, sink, layout, cap, **kw):
    dev = torch.device("cuda", 0)
    out, lse = ffa.flex_flash_attn_fwd(q.to(dev), k.to(dev), v.to(dev), p.q_ranges, p.k_ranges, p.mask_types,
                                       sink=sink.to(dev) if sink is not None else None, sink_layout=layout,
                                       softcap=cap, **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def check_fwd(out, lse, ref_out, ref_lse, what):
    o = out.double().numpy()
    l = lse.double().numpy()
    assert not np.isnan(o).any() and not np.isnan(l).any(), f"{what}: NaN"
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), empty), f"{what}: -inf pattern of lse differs"
    err = np.abs(o - ref_out)
    lerr = np.abs(l[~empty] - ref_lse[~empty]) if (~empty).any() else np.zeros(1)
    log(f"  {what}: out max {err.max():.3e} mean {err.mean():.3e} | lse max {lerr.max():.3e}")
    assert err.max() <= OUT_MAX and err.mean() <= OUT_MEAN and lerr.max() <= LSE_ABS, what


CASES = [(layout, n, cap) for layout in ("sh", "ssh") for n, cap in ((1, 0.0), (3, 0.0), (2, 8.0))] + \
        [(None, 0, 8.0), (None, 0, 30.0)]


@pytest.mark.parametrize("layout,n,cap", CASES)
@pytest.mark.parametrize("seed", range(3))
def test_forward_sink_softcap_random_slices(gpu_lib, seed, layout, n, cap):
    rng = np.random.default_rng(1500 + seed)
    tq, tk = int(rng.integers(1, 500)), int(rng.integers(1, 500))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    p = W.random_problem(1500 + seed, tq, tk, hq, hkv, d, n_types=4)
    q, k, v = W.make_qkv(p)
    q = q * 3  # scores large enough for the cap to bend them
    sink = make_sink(p, layout, n, seed) if layout else None
    out, lse = fwd(gpu_lib, p, q, k, v, sink, layout or "sh", cap)
    ref = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink, sink_layout=layout or "sh",
                        softcap=cap)
    check_fwd(out, lse, *ref, f"seed {seed} sink {layout}/{n} cap {cap}")


@pytest.mark.parametrize("layout", ["sh", "ssh"])
def test_forward_sink_on_split_rows(gpu_lib, layout):
    # forced split-K: the sinks join in the combine kernel
    p = W.make_problem("split", 64, 6000, 4, 1, 128, [((0, 64), (0, 6000), W.CAUSAL)], seed=5)
    q, k, v = W.make_qkv(p)
    sink = make_sink(p, layout, 2, 7)
    out, lse = fwd(gpu_lib, p, q, k, v, sink, layout, 5.0, split_tiles=16)
    plan = gpu_lib._plan_cache[next(reversed(gpu_lib._plan_cache))]
    assert plan.info["num_split_items"] > 0
    ref = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink, sink_layout=layout, softcap=5.0)
    check_fwd(out, lse, *ref, f"split, sink {layout}")


def test_rows_without_keys_take_the_sink_normaliser(gpu_lib):
    p = W.make_problem("holes", 300, 300, 2, 1, 64, [((100, 200), (0, 150), W.CAUSAL)], seed=3)
    q, k, v = W.make_qkv(p)
    sink = make_sink(p, "sh", 2, 3)
    out, lse = fwd(gpu_lib, p, q, k, v, sink, "sh", 0.0)
    want = torch.logsumexp(sink.double(), dim=0).numpy()
    assert (out[:100] == 0).all() and (out[200:] == 0).all()
    np.testing.assert_allclose(lse[:100].double().numpy(), np.broadcast_to(want, (100, 2)), atol=1e-5)
    ref = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink)
    check_fwd(out, lse, *ref, "holes with sink")


def test_forward_full_size_packed_docs_sampled_with_sink_and_cap(gpu_lib):
    p = W.config(3)
    q, k, v = W.make_qkv(p)
    sink = make_sink(p, "sh", 4, 11)
    out, lse = fwd(gpu_lib, p, q, k, v, sink, "sh", 20.0)
    rows = W.sample_rows(p, 96, seed=9)
    ref = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, rows=rows, sink=sink, softcap=20.0)
    check_fwd(out[rows], lse[rows], *ref, "packed docs, sampled rows")


# ---------------------------------------------------------------- backward

def torch_bf16_grads(p, q, k, v, dout, sink, layout, cap):
    """Same-precision PyTorch backward on the CPU: bf16 autograd with the oracle's mask,
    the cap as cap*tanh(s/cap) and the sinks as extra score columns with zero value."""
    mask = torch.from_numpy(oracle.dense_mask(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k))
    has = mask.any(1)
    rep = p.heads_q // p.heads_kv
    sc = 1.0 / p.head_dim ** 0.5
    qq, kk, vv = (x.clone().requires_grad_(True) for x in (q, k, v))
    sk = sink.clone().requires_grad_(True) if sink is not None else None
    a = qq.permute(1, 0, 2)
    b = kk.repeat_interleave(rep, 1).permute(1, 2, 0).contiguous()
    c = vv.repeat_interleave(rep, 1).permute(1, 0, 2).contiguous()
    s = torch.matmul(a, b) * sc
    if cap:
        s = cap * torch.tanh(s / cap)
    if sk is not None:
        s = s.masked_fill(~mask[None], float("-inf"))
        extra = (sk.t()[:, None, :].expand(-1, p.total_q, -1) if layout == "sh" else sk.permute(2, 0, 1))
        full = torch.cat([s, extra.to(torch.bfloat16)], dim=-1)
        pr = torch.softmax(full, dim=-1)[..., :p.total_k]
        o = torch.matmul(pr, c)
    else:
        m2 = mask | ~has[:, None]
        s = s.masked_fill(~m2[None], float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), c) * has[None, :, None]
    (o.permute(1, 0, 2).float() * dout.float()).sum().backward()
    res = [x.grad.double().numpy() for x in (qq, kk, vv)]
    if sk is not None:
        res.append(sk.grad.double().numpy())
    return res


@pytest.mark.parametrize("layout,n,cap", [("sh", 2, 0.0), ("ssh", 1, 0.0), (None, 0, 6.0), ("sh", 3, 6.0)])
@pytest.mark.parametrize("seed", range(3))
def test_backward_sink_softcap(gpu_lib, seed, layout, n, cap):
    rng = np.random.default_rng(1600 + seed)
    tq, tk = int(rng.integers(1, 400)), int(rng.integers(1, 400))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    p = W.random_problem(1600 + seed, tq, tk, hq, hkv, d, n_types=4)
    q, k, v = W.make_qkv(p)
    q = q * 3
    dout = W.make_dout(p)
    sink = make_sink(p, layout, n, seed) if layout else None
    dev = torch.device("cuda", 0)
    qd, kd, vd, dd = q.to(dev), k.to(dev), v.to(dev), dout.to(dev)
    sd = sink.to(dev) if sink is not None else None
    lay = layout or "sh"
    out, lse = gpu_lib.flex_flash_attn_fwd(qd, kd, vd, p.q_ranges, p.k_ranges, p.mask_types, sink=sd,
                                           sink_layout=lay, softcap=cap)
    g = gpu_lib.flex_flash_attn_bwd(dd, qd, kd, vd, out, lse, p.q_ranges, p.k_ranges, p.mask_types, sink=sd,
                                    sink_layout=lay, softcap=cap)
    torch.cuda.synchronize()
    ref = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types, sink=sink, sink_layout=lay,
                                 softcap=cap)
    tb = torch_bf16_grads(p, q, k, v, dout, sink, lay, cap)
    names = ("dq", "dk", "dv", "dsink")[:len(ref)]
    for name, x, r, t in zip(names, g, ref, tb):
        xn = x.double().cpu().numpy()
        assert not np.isnan(xn).any(), name
        err, et = np.abs(xn - r), np.abs(t - r)
        allow = 1e-3 * max(np.abs(r).max(), 1e-2)
        log(f"  seed {seed} sink {layout}/{n} cap {cap} {name}: max {err.max():.3e} (torch bf16 {et.max():.3e}) "
            f"mean {err.mean():.3e} (torch bf16 {et.mean():.3e})")
        if name == "dsink":
            check_dsink(xn, r, out, lse, dout, sink, lay, p, q, k, v, cap, err, et, allow)
            continue
        assert err.max() <= 2.0 * et.max() + allow, name
        assert err.mean() <= 2.0 * et.mean() + allow, name


def check_dsink(got, ref, out, lse, dout, sink, layout, p, q, k, v, cap, err, et, allow):
    """d sink = -sum_i exp(sink - lse_i) Dd_i with Dd_i = rowsum(dout_i * out_i) formed from
    the stored (bf16) out, as the backward defines it (test_dsink_follows_its_definition
    pins that sum).  PyTorch's autograd reaches the sink gradient without the rounded
    out, so on some seeds (3 of 100 in a sweep) the kernel's error exceeds twice
    PyTorch's while being the forward's output rounding carried into Dd.  Accepted when
    either (a) the same-precision rule holds, or (b) the distance to the oracle stays
    within the forward's output error propagated through that sum:
    sum_i exp(sink - lse_i) sum_d |dout_id| |out_id - out_exact_id|."""
    if err.max() <= 2.0 * et.max() + allow and err.mean() <= 2.0 * et.mean() + allow:
        return
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    do = dout.double().numpy()
    ref_o, ref_l = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink, sink_layout=layout,
                                 softcap=cap)
    sk = sink.double().numpy()
    if layout == "sh":    # sk [S, Hq]; weights [Tq, S, Hq], gradients summed over rows
        w_gpu, w_ref = np.exp(sk[None] - l[:, None, :]), np.exp(sk[None] - ref_l[:, None, :])
        red = lambda x: x.sum(0)
    else:                 # sk [Tq, S, Hq]; one gradient per row
        w_gpu, w_ref = np.exp(sk - l[:, None, :]), np.exp(sk - ref_l[:, None, :])
        red = lambda x: x
    dd_gpu = (do * o).sum(-1)[:, None, :]
    term = red(w_gpu * np.abs(dd_gpu)) + 1e-30
    prop = red(w_ref * (np.abs(do) * np.abs(o - ref_o)).sum(-1)[:, None, :])
    # the weights themselves move with lse (<= 1e-3 absolute) and the sum with fp32
    slack = red(np.abs(w_gpu - w_ref) * np.abs(dd_gpu)) + 1e-5 * term
    log(f"    d sink: error {err.max():.3e} against the propagated output error {prop.max():.3e}")
    assert (err <= 1.01 * prop + slack).all(), "d sink error beyond the forward's output error"


def test_autograd_with_sink_and_cap(gpu_lib):
    p = W.random_problem(21, 250, 300, 4, 2, 128, n_types=4)
    dev = torch.device("cuda", 0)
    q, k, v = (x.to(dev) for x in W.make_qkv(p))
    dout = W.make_dout(p).to(dev)
    sink = make_sink(p, "sh", 2, 21).to(dev)
    qa, ka, va, sa = (x.clone().requires_grad_(True) for x in (q, k, v, sink))
    out, lse = gpu_lib.flex_flash_attn_func(qa, ka, va, p.q_ranges, p.k_ranges, p.mask_types, sink=sa, softcap=7.0)
    out.backward(dout)
    out2, lse2 = gpu_lib.flex_flash_attn_fwd(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink, softcap=7.0)
    dq, dk, dv, ds = gpu_lib.flex_flash_attn_bwd(dout, q, k, v, out2, lse2, p.q_ranges, p.k_ranges, p.mask_types,
                                                 sink=sink, softcap=7.0)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), out2) and torch.equal(lse, lse2)
    assert torch.equal(qa.grad, dq) and torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)
    assert torch.equal(sa.grad, ds)


def test_head_dim_32_sink_and_cap(gpu_lib):
    p = W.random_problem(1900, 300, 350, 4, 2, 32, n_types=4)
    q, k, v = W.make_qkv(p)
    q = q * 3
    sink = make_sink(p, "sh", 2, 19)
    out, lse = fwd(gpu_lib, p, q, k, v, sink, "sh", 6.0)
    ref = oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink, softcap=6.0)
    check_fwd(out, lse, *ref, "D 32 sink + cap")


@pytest.mark.parametrize("layout,d,f16", [("sh", 128, False), ("ssh", 64, False), ("sh", 32, True)])
def test_dsink_follows_its_definition(gpu_lib, layout, d, f16):
    # d sink = -sum_i exp(sink - lse_i) * rowsum(dout_i * out_i) (per row for "ssh"),
    # checked on seeded out / dout / lse / sink (the sum does not need out to be the
    # forward's), rows that see no key included; fp64 of the same 16-bit values.
    ffa = gpu_lib
    dt = torch.float16 if f16 else torch.bfloat16
    tq, tk, hq, hkv, ns = 300, 200, 4, 2, 3
    p = W.make_problem("dsink_def", tq, tk, hq, hkv, d,
                       [((0, 120), (0, 200), W.CAUSAL), ((180, 260), (40, 150), W.FULL)], seed=21)
    g = torch.Generator().manual_seed(40 + d)
    q, k, v = (torch.randn(*s_, generator=g).to(dt) for s_ in ((tq, hq, d), (tk, hkv, d), (tk, hkv, d)))
    out, dout = (torch.randn(tq, hq, d, generator=g).to(dt) for _ in range(2))
    lse = 2.0 + torch.rand(tq, hq, generator=g) * 3.0
    sink = torch.randn((ns, hq) if layout == "sh" else (tq, ns, hq), generator=g)
    dev = torch.device("cuda", 0)
    res = ffa.flex_flash_attn_bwd(dout.to(dev), q.to(dev), k.to(dev), v.to(dev), out.to(dev), lse.to(dev),
                                  p.q_ranges, p.k_ranges, p.mask_types, sink=sink.to(dev), sink_layout=layout)
    torch.cuda.synchronize()
    got = res[3].double().cpu().numpy()
    prod = dout.double() * out.double()
    dd, dd_abs = prod.sum(-1).numpy(), prod.abs().sum(-1).numpy()  # [Tq, Hq]
    sk, l = sink.double().numpy(), lse.double().numpy()
    w = np.exp(sk[None] - l[:, None, :]) if layout == "sh" else np.exp(sk - l[:, None, :])
    terms, scale = w * dd[:, None, :], w * dd_abs[:, None, :]
    want = -terms.sum(0) if layout == "sh" else -terms
    mag = scale.sum(0) if layout == "sh" else scale  # fp32 sums are good to a few ulp of this
    err = np.abs(got - want)
    log(f"  d sink definition {layout} D {d} fp16 {f16}: max error {err.max():.3e} (of sum |terms| "
        f"{(err / (mag + 1e-30)).max():.2e})")
    assert (err <= 2e-5 * mag + 1e-30).all()


@pytest.mark.parametrize("cap", [0.0, 6.0])
@pytest.mark.parametrize("f16", [False, True])
@pytest.mark.parametrize("d", [16, 32])
def test_small_head_dims_every_backward_instance(gpu_lib, d, f16, cap):
    # The D = 16 and 32 backward kernels live in an object of their own; together these
    # eight cases launch each of them once: dQ, dK/dV and total attention, for bf16 and
    # fp16, with and without the soft cap.  Gradients: the same-precision rule against
    # the fp64 oracle; total attention: 1e-3 relative.
    from tests.test_gpu_total import check_total

    dt = torch.float16 if f16 else torch.bfloat16
    seed = 3100 + 8 * (d == 32) + 4 * f16 + 2 * (cap > 0)
    rng = np.random.default_rng(seed)
    tq, tk = int(rng.integers(150, 400)), int(rng.integers(150, 400))
    p = W.random_problem(seed, tq, tk, 4, 2, d, n_types=4)
    q, k, v = W.make_qkv(p, dtype=dt)
    q = q * 3 if cap else q
    dout = W.make_dout(p, dtype=dt)
    what = f"D {d} {'fp16' if f16 else 'bf16'} cap {cap}"
    log(f"  {what}: Tq {tq} Tk {tk} slices {p.num_slices}")
    dev = torch.device("cuda", 0)
    qd, kd, vd, dd = q.to(dev), k.to(dev), v.to(dev), dout.to(dev)
    out, lse = gpu_lib.flex_flash_attn_fwd(qd, kd, vd, p.q_ranges, p.k_ranges, p.mask_types, softcap=cap)
    g = gpu_lib.flex_flash_attn_bwd(dd, qd, kd, vd, out, lse, p.q_ranges, p.k_ranges, p.mask_types, softcap=cap)
    tot = gpu_lib.flex_total_attention(qd, kd, lse, p.q_ranges, p.k_ranges, p.mask_types, softcap=cap)
    torch.cuda.synchronize()
    assert all(x.dtype == dt for x in g)
    ref = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types, softcap=cap)
    tb = torch_bf16_grads(p, q, k, v, dout, None, "sh", cap)
    for name, x, r, t in zip(("dq", "dk", "dv"), g, ref, tb):
        xn = x.double().cpu().numpy()
        assert not np.isnan(xn).any(), name
        err, et = np.abs(xn - r), np.abs(t - r)
        allow = 1e-3 * max(np.abs(r).max(), 1e-2)
        log(f"  {what} {name}: max {err.max():.3e} (same precision {et.max():.3e}) "
            f"mean {err.mean():.3e} (same precision {et.mean():.3e})")
        assert err.max() <= 2.0 * et.max() + allow, name
        assert err.mean() <= 2.0 * et.mean() + allow, name
    check_total(tot, oracle.total_attention(q, k, p.q_ranges, p.k_ranges, p.mask_types, softcap=cap), what)
