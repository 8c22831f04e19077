"""ffa_fwd (with the split-K combine) and ffa_bwd captured into one HIP graph.

The library never allocates, synchronises or clears memory inside its calls (its
kernels write every output element), so a caller can capture them.  The graph is
replayed three times with eager work in between that overwrites every output, and
each replay must reproduce the eager results bit for bit (the kernels use no
atomics, so they are deterministic).
"""
import math
import sys

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_graph_replay_matches_eager(gpu_lib):
    ffa = gpu_lib
    p = W.random_problem(4242, 700, 900, 8, 2, 128, n_types=4)
    dev = torch.device("cuda", 0)
    q, k, v = (x.to(dev) for x in W.make_qkv(p))
    dout = W.make_dout(p).to(dev)
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, split_tiles=3, backward=True)
    assert plan.info["num_combine"] > 0  # the combine kernel is part of the graph
    scale = 1.0 / math.sqrt(p.head_dim)
    ex = ffa.make_extras(dtype=q.dtype)

    def tensors():
        out = torch.empty_like(q)
        lse = torch.empty((p.total_q, p.heads_q), dtype=torch.float32, device=dev)
        return {"q": q, "k": k, "v": v, "out": out, "lse": lse, "dout": dout,
                "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v)}

    def strides(t):
        return {n: (0, x.stride(0), x.stride(1)) for n, x in t.items()}

    def step(t, st):
        ffa.run_fwd(plan, t["q"], t["k"], t["v"], t["out"], t["lse"], st, 1, scale, ex)
        ffa.run_bwd(plan, t, st, 1, scale, ex)

    s = torch.cuda.Stream()
    eager, graphed = tensors(), tensors()
    with torch.cuda.stream(s):
        step(eager, strides(eager))      # uploads the plan and sizes the workspaces on s
        step(graphed, strides(graphed))  # the same calls once more, eagerly
    s.synchronize()
    log("  eager reference done")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(graphed, strides(graphed))
    torch.cuda.synchronize()
    log("  captured")
    for rep in range(3):
        for n in ("out", "lse", "dq", "dk", "dv"):
            graphed[n].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in ("out", "lse", "dq", "dk", "dv"):
            assert torch.equal(graphed[n], eager[n]), f"replay {rep}: {n} differs from the eager call"
        log(f"  replay {rep} bitwise equal")
