"""GPU parity of FlagAttention's total attention (``ffa_total_attention``: attention
probabilities summed over the query axis) and of the differentiable FlagAttention
adapter (``flash_attention`` on [B, H, M, D], forward and backward), against the fp64
oracle.

Total attention is built from fp32 scores of the exact bf16 inputs and the forward's fp32
lse, so it is held to 1e-3 relative (+1e-4 absolute) of the oracle; the adapter's out,
lse and gradients to the tolerances of test_gpu_parity / test_gpu_bwd.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.test_gpu_bwd import compare as compare_grads, torch_bf16_grads

pytestmark = pytest.mark.gpu


def check_total(got, ref, what):
    g = got.double().cpu().numpy()
    assert not np.isnan(g).any()
    err = np.abs(g - ref)
    bound = 1e-3 * np.abs(ref) + 1e-4
    print(f"  {what}: total max err {err.max():.3e} (max |ref| {np.abs(ref).max():.3e})", flush=True)
    assert (err <= bound).all(), f"{what}: total error {err.max()}"


@pytest.mark.parametrize("seed", range(6))
def test_total_attention_random_slices(gpu_lib, seed):
    rng = np.random.default_rng(2400 + seed)
    tq, tk = int(rng.integers(1, 500)), int(rng.integers(1, 500))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = [16, 32, 64, 128][seed % 4]
    p = W.random_problem(2400 + seed, tq, tk, hq, hkv, d, n_types=4)
    q, k, v = W.make_qkv(p)
    sink = torch.randn((2, hq), generator=torch.Generator().manual_seed(seed)) if seed % 2 else None
    cap = 5.0 if seed in (2, 5) else 0.0
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    sd = sink.to(dev) if sink is not None else None
    out, lse = gpu_lib.flex_flash_attn_fwd(qd, kd, vd, p.q_ranges, p.k_ranges, p.mask_types, sink=sd, softcap=cap)
    tot = gpu_lib.flex_total_attention(qd, kd, lse, p.q_ranges, p.k_ranges, p.mask_types, sink=sd, softcap=cap)
    torch.cuda.synchronize()
    assert tot.shape == (tk, hq)
    ref = oracle.total_attention(q, k, p.q_ranges, p.k_ranges, p.mask_types, sink=sink, softcap=cap)
    check_total(tot, ref, f"random {seed} (D {d}, sink {sink is not None}, cap {cap})")


def test_total_attention_packed_docs_full_size(gpu_lib):
    # the row-sum identity at full size: every row that sees a key gives exactly 1
    p = W.config(3)
    q, k, v = W.make_qkv(p)
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out, lse = gpu_lib.flex_flash_attn_fwd(qd, kd, vd, p.q_ranges, p.k_ranges, p.mask_types)
    tot = gpu_lib.flex_total_attention(qd, kd, lse, p.q_ranges, p.k_ranges, p.mask_types)
    torch.cuda.synchronize()
    sums = tot.double().sum(dim=0).cpu().numpy()
    np.testing.assert_allclose(sums, np.full(p.heads_q, float(p.total_q)), rtol=1e-4)


@pytest.mark.parametrize("causal", [True, False])
def test_flag_attention_total_and_log_normalizer(gpu_lib, causal):
    B, Hq, Hkv, M, N, D = 2, 8, 2, 300, 520, 64
    g = torch.Generator().manual_seed(7)
    q = torch.randn(B, Hq, M, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, N, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, D, generator=g).to(torch.bfloat16)
    dev = torch.device("cuda", 0)
    out, lse, tot, s, o = gpu_lib.flash_attention(q.to(dev), k.to(dev), v.to(dev), causal=causal,
                                                  return_log_normalizer=True, return_total_attention=True)
    torch.cuda.synchronize()
    assert s is None and o is None and tot.shape == (B, Hq, N) and lse.shape == (B, Hq, M)
    ty = W.CAUSAL if causal else W.FULL
    for b in range(B):
        qt, kt, vt = q[b].permute(1, 0, 2), k[b].permute(1, 0, 2), v[b].permute(1, 0, 2)
        ro, rl = oracle.attend(qt, kt, vt, [[0, M]], [[0, N]], [ty])
        assert np.abs(out[b].permute(1, 0, 2).double().cpu().numpy() - ro).max() <= 2e-2
        assert np.abs(lse[b].t().double().cpu().numpy() - rl).max() <= 1e-3
        rt = oracle.total_attention(qt, kt, [[0, M]], [[0, N]], [ty])
        check_total(tot[b].t(), rt, f"FlagAttention layout, batch {b}, causal {causal}")


@pytest.mark.parametrize("causal", [True, False])
def test_flag_attention_backward(gpu_lib, causal):
    B, Hq, Hkv, M, N, D = 2, 4, 2, 200, 330, 128
    g = torch.Generator().manual_seed(8)
    q = torch.randn(B, Hq, M, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, N, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, D, generator=g).to(torch.bfloat16)
    do = torch.randn(B, Hq, M, D, generator=g).to(torch.bfloat16)
    dev = torch.device("cuda", 0)
    qa, ka, va = (x.to(dev).requires_grad_(True) for x in (q, k, v))
    out = gpu_lib.flash_attention(qa, ka, va, causal=causal)
    out.backward(do.to(dev))
    torch.cuda.synchronize()
    ty = W.CAUSAL if causal else W.FULL
    for b in range(B):
        p = W.make_problem("flag", M, N, Hq, Hkv, D, [((0, M), (0, N), ty)])
        qt, kt, vt, dt = (x[b].permute(1, 0, 2).contiguous() for x in (q, k, v, do))
        refs = oracle.attend_backward(qt, kt, vt, dt, p.q_ranges, p.k_ranges, p.mask_types)
        grads = [x.grad[b].permute(1, 0, 2).cpu() for x in (qa, ka, va)]
        compare_grads(grads, refs, f"FlagAttention layout backward, batch {b}, causal {causal}",
                      torch_bf16_grads(p, qt, kt, vt, dt))
