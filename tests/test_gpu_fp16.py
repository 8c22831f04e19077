"""GPU parity with float16 inputs and outputs (FlagAttention's flash_attention example
runs in fp16) against the fp64 oracle, which reads the exact fp16 values.

Tolerances as for bfloat16 (test_gpu_parity: out max-abs <= 2e-2, mean-abs <= 2e-3, lse
<= 1e-3; test_gpu_bwd: the same-precision rule, here against PyTorch's fp16 autograd).
fp16 holds at most 65504, so the forward rescales a row exactly as soon as one of its
probabilities would pass 2^15 (bf16: 2^64); growing scores drive that path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.test_gpu_bwd import compare as compare_grads, torch_bf16_grads
from tests.test_gpu_parity import compare as compare_fwd

pytestmark = pytest.mark.gpu

F16 = torch.float16
DEV = torch.device("cuda", 0)


def fwd16(ffa, p, q, k, v, **kw):
    out, lse = ffa.flex_flash_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), p.q_ranges, p.k_ranges, p.mask_types, **kw)
    torch.cuda.synchronize()
    assert out.dtype == F16
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("seed", range(6))
def test_fp16_forward_random_slices(gpu_lib, seed):
    rng = np.random.default_rng(2500 + seed)
    tq, tk = int(rng.integers(1, 600)), int(rng.integers(1, 600))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = [32, 64, 128][seed % 3]
    p = W.random_problem(2500 + seed, tq, tk, hq, hkv, d, n_types=4)
    q, k, v = W.make_qkv(p, dtype=F16)
    out, lse = fwd16(gpu_lib, p, q, k, v, split_tiles=3 if seed == 5 else 0)
    compare_fwd(out, lse, *oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types), what=f"fp16 random {seed}")


@pytest.mark.parametrize("grow", [4.0, 12.0])
def test_fp16_growing_scores_take_the_exact_rescale(gpu_lib, grow):
    # one causal sequence whose keys grow along the axis: later tiles outgrow the first
    # tile's reference point by far more than 2^15, the fp16 bound
    T, H, D = 2048, 2, 128
    p = W.make_problem("grow", T, T, H, H, D, [((0, T), (0, T), W.CAUSAL)], seed=9)
    q, k, v = W.make_qkv(p, dtype=torch.float32)
    q = q.abs()
    k = (k.abs() * torch.linspace(0.1, grow, T)[:, None, None])
    q, k, v = q.to(F16), k.to(F16), v.to(F16)
    out, lse = fwd16(gpu_lib, p, q, k, v)
    rows = W.sample_rows(p, 160, seed=1)
    compare_fwd(out, lse, *oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, rows=rows), rows=rows,
                what=f"fp16 growing scores x{grow}")


def test_fp16_sink_and_softcap(gpu_lib):
    p = W.random_problem(2600, 300, 400, 4, 2, 128, n_types=4)
    q, k, v = W.make_qkv(p, dtype=F16)
    sink = torch.randn((2, 4), generator=torch.Generator().manual_seed(3))
    out, lse = fwd16(gpu_lib, p, q, k, v, sink=sink.to(DEV), softcap=6.0)
    compare_fwd(out, lse, *oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, sink=sink, softcap=6.0),
                what="fp16 sink + cap")


@pytest.mark.parametrize("seed", range(3))
def test_fp16_backward(gpu_lib, seed):
    rng = np.random.default_rng(2700 + seed)
    tq, tk = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = [32, 64, 128][seed]
    p = W.random_problem(2700 + seed, tq, tk, hq, hkv, d, n_types=4)
    q, k, v = W.make_qkv(p, dtype=F16)
    dout = W.make_dout(p, dtype=F16)
    qd, kd, vd, dd = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
    out, lse = gpu_lib.flex_flash_attn_fwd(qd, kd, vd, p.q_ranges, p.k_ranges, p.mask_types)
    dq, dk, dv = gpu_lib.flex_flash_attn_bwd(dd, qd, kd, vd, out, lse, p.q_ranges, p.k_ranges, p.mask_types)
    torch.cuda.synchronize()
    assert dq.dtype == F16
    refs = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types)
    compare_grads([x.cpu() for x in (dq, dk, dv)], refs, f"fp16 backward {seed}",
                  torch_bf16_grads(p, q, k, v, dout), stored=(p, q, k, v, dout, out.cpu(), None))


def test_flag_attention_fp16_example_shape(gpu_lib):
    # the FlagAttention user guide's example: B 2, Hq 16, Hkv 4, M 2048, N 4096, D 128,
    # fp16, causal (bottom-right), out.sum().backward(); forward rows sampled against the
    # oracle, gradients checked through the identity sum_j dv = sum_i dout (all rows see keys)
    B, Hq, Hkv, M, N, D = 2, 16, 4, 2048, 4096, 128
    g = torch.Generator().manual_seed(11)
    q = torch.randn(B, Hq, M, D, generator=g).to(F16)
    k = torch.randn(B, Hkv, N, D, generator=g).to(F16)
    v = torch.randn(B, Hkv, N, D, generator=g).to(F16)
    qa, ka, va = (x.to(DEV).requires_grad_(True) for x in (q, k, v))
    out = gpu_lib.flash_attention(qa, ka, va, causal=True)
    out.sum().backward()
    torch.cuda.synchronize()
    assert out.dtype == F16 and qa.grad.dtype == F16
    rows = np.sort(np.random.default_rng(3).choice(M, 24, replace=False))
    for b in range(B):
        ro, _ = oracle.attend(q[b].permute(1, 0, 2), k[b].permute(1, 0, 2), v[b].permute(1, 0, 2),
                              [[0, M]], [[0, N]], [W.CAUSAL], rows=rows)
        err = np.abs(out[b].permute(1, 0, 2).detach().double().cpu().numpy()[rows] - ro).max()
        assert err <= 2e-2, err
    # dout = 1 everywhere: sum over keys of dv per kv head = M * (Hq / Hkv) for every d
    sdv = va.grad.double().sum(dim=2).cpu().numpy()  # [B, Hkv, D]
    np.testing.assert_allclose(sdv, np.full_like(sdv, M * Hq // Hkv), rtol=2e-3)
    sdk = ka.grad.double().sum(dim=2).abs().max().item() / ka.grad.double().abs().sum(dim=2).max().item()
    assert sdk <= 1e-2
