"""CPU oracle for flexible-mask attention: forward, gradients and total attention (fp64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``flexible_mask_flash_amd``); both are fed by ``workloads``.

Every function here is pinned by ``tests/test_oracle_*.py`` against things
other than itself: brute force on tiny inputs, the pages' interval formula,
the pages' mask figures (``tests/golden/``), torch's fp64 scaled-dot-product
attention special cases, closed forms and the split/merge identity.
"""
from .fwd import (  # noqa: F401
    FULL,
    CAUSAL,
    INVCAUSAL,
    BICAUSAL,
    slice_row_interval,
    mask_rows,
    dense_mask,
    count_visible_pairs,
    attend,
    total_attention,
    capped_scores,
    sink_logits,
    merge_partials,
)
from .bwd import attend_backward  # noqa: F401,E402
