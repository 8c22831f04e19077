"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each.

Each mutation edits the oracle's source text (an off-by-one, a wrong alignment,
a wrong GQA mapping, a dropped scale or term, a transposed operand, a lost
union), loads the edited copy as a fresh module, swaps it into the ``oracle``
package for the duration of the test, and runs the pins of
``test_oracle_pins.py``.  At least one pin must fail for every mutation.
"""
import importlib.util
import inspect
import types

import pytest

import oracle
import oracle.fwd as oracle_fwd
from tests import test_oracle_pins as pins

MUTATIONS = {
    "causal_off_by_one": ("end = ke - (qe - 1 - rows)", "end = ke - (qe - rows)"),
    "causal_top_left": ("end = ke - (qe - 1 - rows)", "end = ks + (rows - qs) + 1"),
    "gqa_interleaved": ("h = g * grp + hh\n                s = capped_scores(",
                        "h = hh * hkv + g\n                s = capped_scores("),
    "scale_dropped": ("s = capped_scores((q[rb, h, :] @ kg.T) * scale, softcap)",
                      "s = capped_scores((q[rb, h, :] @ kg.T), softcap)"),
    "v_replaced_by_k": ("o = (p @ vg)", "o = (p @ kg)"),
    "lse_drops_max": ("l = np.where(nonempty, safe + np.log(", "l = np.where(nonempty, 0.0 + np.log("),
    "union_lost": ("m |= vis", "m = vis"),
    "merge_weights_unshifted": ("w = np.exp(L - safe)", "w = np.exp(L - 2 * safe)"),
    "invcausal_from_the_end": ("start = ks + (rows - qs) if", "start = ks + (qe - 1 - rows) if"),
    "bicausal_loses_start": ("start = ks + (rows - qs) if t in (INVCAUSAL, BICAUSAL)",
                             "start = ks + (rows - qs) if t in (INVCAUSAL,)"),
    # the per-row interval of one slice (used by the visible-pair count)
    "row_interval_causal_off_by_one": ("b = ke - (qe - 1 - i) if mask_type in (CAUSAL, BICAUSAL) else ke",
                                       "b = ke - (qe - i) if mask_type in (CAUSAL, BICAUSAL) else ke"),
    "row_interval_full_is_causal": ("b = ke - (qe - 1 - i) if mask_type in (CAUSAL, BICAUSAL) else ke",
                                    "b = ke - (qe - 1 - i)"),
    # the union of a row's intervals in the visible-pair count
    "count_union_drops_overlap_merge": ("cur_b = max(cur_b, b)", "cur_b = b"),
    "count_union_double_counts": ("if a > cur_b:", "if True:"),
}

PINS = [
    lambda: pins.test_oracle_matches_brute_force(0),
    lambda: pins.test_oracle_matches_brute_force(3),
    lambda: pins.test_mask_equals_interval_formula(1),
    lambda: pins.test_mask_equals_interval_formula(4),
    pins.test_golden_full_then_causal_picture,
    pins.test_rect_causal_is_bottom_right,
    pins.test_gqa_is_mha_with_repeated_kv,
    lambda: pins.test_lse_is_logsumexp_of_masked_scores(0),
    lambda: pins.test_split_and_merge_reproduces_single_slice("causal"),
    pins.test_merge_with_empty_partial,
    pins.test_visible_pair_count_matches_mask_sum,
    lambda: pins.test_mask_equals_interval_formula(9),
    pins.test_square_inverse_causal_is_causal_on_reversed_sequences,
    pins.test_square_bicausal_sees_only_its_diagonal_key,
    pins.test_bicausal_band_splits_into_inverse_causal_and_causal,
    pins.test_visible_pair_counts_closed_forms,
]


def load_mutant(old, new):
    src = inspect.getsource(oracle_fwd)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    mod = load_mutant(*MUTATIONS[name])
    for attr in ("mask_rows", "dense_mask", "count_visible_pairs", "attend", "merge_partials",
                 "slice_row_interval"):
        monkeypatch.setattr(oracle, attr, getattr(mod, attr))
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1, f"no pin caught mutation {name}"


def test_unmutated_oracle_passes_the_same_pins():
    for pin in PINS:
        pin()
