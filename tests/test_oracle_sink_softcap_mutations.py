"""Plant plausible mistakes in the oracle's sink and softcap code (forward and
backward copies) and check that the pins of test_oracle_sink_softcap_pins catch each."""
import inspect
import types

import pytest

import oracle
import oracle.bwd as oracle_bwd
import oracle.fwd as oracle_fwd
from tests import test_oracle_sink_softcap_pins as pins

FWD = {
    "sink_left_out_of_denominator": ("den = p.sum(axis=1) + np.exp(sk - safe[:, None]).sum(axis=1)",
                                     "den = p.sum(axis=1)"),
    "sink_scaled_like_a_score": ("return np.broadcast_to(sk[None], (rows.shape[0],) + sk.shape)",
                                 "return np.broadcast_to(0.5 * sk[None], (rows.shape[0],) + sk.shape)"),
    "softcap_not_multiplied_back": ("return softcap * np.tanh(raw / softcap)", "return np.tanh(raw / softcap)"),
    "softcap_not_divided": ("return softcap * np.tanh(raw / softcap)", "return softcap * np.tanh(raw)"),
}
BWD = {
    "softcap_derivative_dropped": ("ds = ds * (1.0 - np.tanh(raw / softcap) ** 2)", "ds = ds"),
    "softcap_derivative_not_squared": ("ds = ds * (1.0 - np.tanh(raw / softcap) ** 2)",
                                       "ds = ds * (1.0 - np.tanh(raw / softcap))"),
    "dsink_sign_flipped": ("contrib = -ps * dd", "contrib = ps * dd"),
    "dsink_without_row_term": ("contrib = -ps * dd", "contrib = -ps"),
}

PINS = [
    lambda: pins.test_sink_is_a_zero_value_key(0, "sh"),
    lambda: pins.test_sink_is_a_zero_value_key(1, "ssh"),
    pins.test_row_without_keys_keeps_sink_normaliser,
    lambda: pins.test_softcap_and_sink_gradients_match_finite_differences(0),
    lambda: pins.test_softcap_and_sink_gradients_match_finite_differences(1),
    lambda: pins.test_softcap_gradients_without_sink_match_finite_differences(0),
    pins.test_large_softcap_is_no_softcap,
    pins.test_tiny_softcap_flattens_scores,
    pins.test_softcap_bounds_the_log_normaliser,
]


def mutant(module, old, new, name):
    src = inspect.getsource(module)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType(name)
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new).replace("from .fwd import", "from oracle.fwd import"), name, "exec"),
         mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(FWD) + sorted(BWD))
def test_pins_catch_sink_softcap_mutation(name, monkeypatch):
    if name in FWD:
        mod = mutant(oracle_fwd, *FWD[name], "oracle_fwd_mutant")
        monkeypatch.setattr(oracle, "attend", mod.attend)
    else:
        mod = mutant(oracle_bwd, *BWD[name], "oracle_bwd_mutant")
        monkeypatch.setattr(oracle, "attend_backward", mod.attend_backward)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught mutation {name}"
