"""Plant plausible mistakes in a copy of the backward oracle and check that its pins catch each."""
import inspect
import types

import pytest

import oracle
import oracle.bwd as oracle_bwd
from tests import test_oracle_bwd_pins as pins

MUTATIONS = {
    "jacobian_term_dropped": ("ds = p * (dp - dd)", "ds = p * dp"),
    "dk_scale_dropped": ("dk[cols, g, :] += scale * (ds.T @ q[rb, h, :])", "dk[cols, g, :] += ds.T @ q[rb, h, :]"),
    "dv_squared_weights": ("dv[cols, g, :] += p.T @ do", "dv[cols, g, :] += (p * p).T @ do"),
    "dq_uses_v": ("dq[rb, h, :] = scale * (ds @ kg)", "dq[rb, h, :] = scale * (ds @ vg)"),
    "gqa_heads_not_summed": ("dk[cols, g, :] += scale", "dk[cols, g, :] = scale"),
}

PINS = [
    lambda: pins.test_backward_matches_finite_differences(0),
    lambda: pins.test_backward_matches_finite_differences(5),
    pins.test_full_slice_gradients_are_sdpa_gradients,
    pins.test_rect_causal_gradients_are_bottom_right_sdpa_gradients,
    lambda: pins.test_dv_sums_to_dout_of_visible_rows(0),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_backward_mutation(name, monkeypatch):
    old, new = MUTATIONS[name]
    src = inspect.getsource(oracle_bwd)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_bwd_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new).replace("from .fwd import", "from oracle.fwd import"), "oracle_bwd_mutant",
                 "exec"), mod.__dict__)
    monkeypatch.setattr(oracle, "attend_backward", mod.attend_backward)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught mutation {name}"
