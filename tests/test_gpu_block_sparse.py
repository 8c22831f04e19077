"""GPU parity on uniform block-sparse masks (many tiny FULL slices; the block sizes of
the MagiAttention experiment notes: 64/64, 128/128, small query blocks 8-32 against
64-key blocks, small key blocks 1-64 against 64-row blocks), forward and backward,
against the fp64 oracle.  Tolerances as in test_gpu_parity (forward) and
test_gpu_bwd (backward, FlagAttention's same-precision rule)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.test_gpu_bwd import compare as compare_grads, run_bwd, torch_bf16_grads
from tests.test_gpu_parity import compare as compare_fwd

pytestmark = pytest.mark.gpu

SHAPES = [(64, 64), (128, 128), (32, 64), (16, 64), (8, 64), (64, 32), (64, 16), (64, 8), (64, 1)]


@pytest.mark.parametrize("qb,kb", SHAPES)
def test_block_sparse_forward(gpu_lib, qb, kb):
    p = W.block_sparse_problem(1024, qb, kb, 0.25, 8, 2, 128, seed=qb * 1000 + kb)
    q, k, v = W.make_qkv(p)
    dev = torch.device("cuda", 0)
    out, lse = gpu_lib.flex_flash_attn_fwd(q.to(dev), k.to(dev), v.to(dev), p.q_ranges, p.k_ranges, p.mask_types)
    torch.cuda.synchronize()
    compare_fwd(out, lse, *oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types),
                what=f"block sparse q{qb} k{kb} ({p.num_slices} slices)")


@pytest.mark.parametrize("qb,kb", [(64, 64), (16, 64), (64, 16), (64, 1)])
def test_block_sparse_backward(gpu_lib, qb, kb):
    p = W.block_sparse_problem(512, qb, kb, 0.25, 4, 2, 64, seed=qb * 1000 + kb + 1)
    q, k, v = W.make_qkv(p)
    dout = W.make_dout(p)
    grads, out = run_bwd(gpu_lib, p, q, k, v, dout, return_out=True)
    refs = oracle.attend_backward(q, k, v, dout, p.q_ranges, p.k_ranges, p.mask_types)
    compare_grads(grads, refs, f"block sparse q{qb} k{kb}", torch_bf16_grads(p, q, k, v, dout),
                  stored=(p, q, k, v, dout, out, None))


@pytest.mark.parametrize("name", ["block_sparse", "block_sparse_k16", "block_sparse_q16"])
def test_block_sparse_full_size_sampled(gpu_lib, name):
    p = W.workload(name)
    q, k, v = W.make_qkv(p)
    dev = torch.device("cuda", 0)
    out, lse = gpu_lib.flex_flash_attn_fwd(q.to(dev), k.to(dev), v.to(dev), p.q_ranges, p.k_ranges, p.mask_types)
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(p.total_q, size=64, replace=False)
    rows = np.sort(np.concatenate([rows, [0, p.total_q - 1]]))
    compare_fwd(out, lse, *oracle.attend(q, k, v, p.q_ranges, p.k_ranges, p.mask_types, rows=rows), rows=rows,
                what=f"{name} full, sampled")
