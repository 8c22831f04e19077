"""ffa_fwd_noalloc (the forward for callers that cannot allocate device memory)
against ffa_fwd, through the C ABI.

The two entry points run the same kernels; only the home of the split-K
partials differs (the library's own device scratch against a caller
workspace), so on the same plan and inputs their out and lse must be bitwise
equal, and both within the oracle's tolerances.  Two calls in a row, the second
on a smaller problem, check that the scratch keeps no state a later call could
read.  A plan whose partials exceed the scratch is refused before any launch.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def both(ffa, p, split_tiles):
    dev = torch.device("cuda", 0)
    q, k, v = W.make_qkv(p)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, split_tiles=split_tiles)
    scale = p.head_dim ** -0.5
    res = []
    for fn in (ffa.run_fwd, ffa.run_fwd_noalloc):
        out = torch.full_like(qd, 7.0)
        lse = torch.full((p.total_q, p.heads_q), 7.0, dtype=torch.float32, device=dev)
        st = {"q": (0, qd.stride(0), qd.stride(1)), "k": (0, kd.stride(0), kd.stride(1)),
              "v": (0, vd.stride(0), vd.stride(1)), "out": (0, out.stride(0), out.stride(1)),
              "lse": (0, lse.stride(0), lse.stride(1))}
        log(f"  {p.name}: {fn.__name__} split_tiles={split_tiles}")
        fn(plan, qd, kd, vd, out, lse, st, 1, scale)
        torch.cuda.synchronize()
        res.append((out, lse))
    return plan, (q, k, v), res


def check(p, qkv, res, what):
    (o1, l1), (o2, l2) = res
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{what}: ffa_fwd_noalloc differs from ffa_fwd"
    ro, rl = oracle.attend(*qkv, p.q_ranges, p.k_ranges, p.mask_types)
    o = o2.double().cpu().numpy()
    l = l2.double().cpu().numpy()
    err = np.abs(o - ro)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(l), ~fin)
    lerr = np.abs(l[fin] - rl[fin]).max() if fin.any() else 0.0
    log(f"  {what}: out max {err.max():.2e} mean {err.mean():.2e} lse max {lerr:.2e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr <= 1e-3


def test_noalloc_matches_ffa_fwd_twice_second_smaller(gpu_lib):
    # a long causal head split into chunks of 4 key tiles, then a smaller mixed problem
    big = W.make_problem("noalloc_big", 2048, 2048, 8, 2, 128, [((0, 2048), (0, 2048), W.CAUSAL)], seed=21)
    plan, qkv, res = both(gpu_lib, big, 4)
    assert plan.info["num_split_items"] > 0 and plan.info["workspace_bytes"] > 0
    check(big, qkv, res, "first call (split)")
    small = W.make_problem("noalloc_small", 300, 500, 4, 1, 128,
                           [((0, 100), (0, 120), W.FULL), ((100, 300), (0, 500), W.CAUSAL)], seed=22)
    plan2, qkv2, res2 = both(gpu_lib, small, 2)
    assert plan2.info["num_split_items"] > 0
    assert plan2.info["workspace_bytes"] < plan.info["workspace_bytes"]
    check(small, qkv2, res2, "second call (smaller, split)")
    # and a plan without split rows: no scratch needed
    plan3, qkv3, res3 = both(gpu_lib, small, -1)
    assert plan3.info["workspace_bytes"] == 0
    check(small, qkv3, res3, "unsplit")


def test_noalloc_refuses_a_plan_beyond_the_scratch(gpu_lib):
    # 16384 causal rows of 8 heads in chunks of 4 key tiles: far more partials than 64 MiB
    T = 16384
    plan = gpu_lib.Plan([[0, T]], [[0, T]], [W.CAUSAL], T, T, 8, 8, 128, split_tiles=4)
    assert plan.info["workspace_bytes"] > 64 << 20
    fake = 1 << 20  # never dereferenced: the size check fails before anything else
    lib = gpu_lib.load_library()
    st = lib.ffa_fwd_noalloc(plan.handle, fake, 1, fake, 0, 1024, 128, fake, 0, 1024, 128, fake, 0, 1024, 128,
                             fake, 0, 1024, 128, fake, 0, 8, 1, 0.1, None, None)
    assert st == 7 and "scratch" in lib.ffa_last_error().decode()
