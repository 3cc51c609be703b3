"""Planted mistakes in the oracle must be caught by the pins.

Each mutant replaces one piece of the oracle (on the CPU only) with a
plausible error: an off-by-one at a window edge, a sink that ignores
causality, a floored band width, a band indexed by the wrong head, a sign
flip in the band offset.  At least one pin in tests/test_oracle_pins.py must
then fail.
"""

import numpy as np
import pytest

import oracle.cowa_oracle as O
from tests import test_oracle_pins as P

_orig_visible = O.visible


def _mut_visible(kind):
    def vis(t, j, g, p):
        t = np.asarray(t, dtype=np.int64)
        j = np.asarray(j, dtype=np.int64)
        dist = t - j
        causal = dist >= 0
        if p.mode == O.MODE_CAUSAL:
            return causal
        L = O.resolved_band(p)
        lo, hi = p.window + g * L, p.window + (g + 1) * L
        sink = j < p.sink
        local = dist < p.window
        band = (dist >= lo) & (dist < hi)
        if kind == "band_inclusive":
            band = (dist >= lo) & (dist <= hi)
        elif kind == "local_inclusive":
            local = dist <= p.window
        elif kind == "sink_not_causal":
            return (causal & (local | band)) | sink
        elif kind == "band_sign":
            band = (-dist >= lo) & (-dist < hi)
        elif kind == "band_from_zero":
            band = (dist >= g * L) & (dist < (g + 1) * L)
        return causal & (sink | local | band)
    return vis


PINS = [
    P.test_golden_grid_16,
    P.test_golden_ragged_17,
    lambda: P._coverage_check_dense(1024, 16, 128, 4),
    lambda: P._coverage_check_dense(17, 2, 4, 4),
    P.test_pair_counts_tiny_bruteforce_and_closed_form,
    lambda: P.test_reduces_to_dense_causal("sink_plus_window_covers"),
    lambda: P.test_reduces_to_dense_causal("one_global_head"),
    P.test_band_only_closed_form,
]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("kind", ["band_inclusive", "local_inclusive", "sink_not_causal",
                                  "band_sign", "band_from_zero"])
def test_predicate_mutants_are_caught(kind, monkeypatch):
    monkeypatch.setattr(O, "visible", _mut_visible(kind))
    assert _some_pin_fails(), kind


def test_unmutated_passes_all_pins():
    assert not _some_pin_fails()


def test_floored_band_is_caught(monkeypatch):
    monkeypatch.setattr(O, "band_length",
                        lambda n, w, h: 0 if n <= w else (n - w) // h)
    assert _some_pin_fails()


def test_local_head_instead_of_global_is_caught(monkeypatch):
    orig = O.attention

    def attention_local_g(q, k, v, p, scale, **kw):
        p2 = O.Pattern(p.n_ctx, p.sink, p.window, p.band, p.h_kv_global, 0, p.mode)
        return orig(q, k, v, p2, scale, **kw)

    monkeypatch.setattr(O, "attention", attention_local_g)
    with pytest.raises(AssertionError):
        P.test_tensor_parallel_slice_equals_full_run()


# ---- error-bound helpers (pins in tests/test_oracle_sensitivity.py) ----

from tests import test_oracle_sensitivity as S  # noqa: E402

_orig_dsens = O._d_sensitivity
_orig_retained = O.retained_mask


def _sensitivity_pins_fail():
    for case in S.CASES:
        for pin in (S.test_d_sensitivity_closed_form_for_uniform_rows,
                    S.test_d_shift_bound_is_attained, S.test_d_shift_bound_holds_in_general):
            try:
                pin(case)
            except AssertionError:
                return True
    return False


@pytest.mark.parametrize("kind", ["double", "no_o_term", "no_abs_v"])
def test_d_sensitivity_mutants_are_caught(kind, monkeypatch):
    def mutant(P, v, o, do):
        if kind == "double":
            return 2.0 * _orig_dsens(P, v, o, do)
        if kind == "no_o_term":
            return (np.abs(do) * (P @ np.abs(v))).sum(axis=1)
        return (np.abs(do) * (np.abs(P @ v) + np.abs(o))).sum(axis=1)
    monkeypatch.setattr(O, "_d_sensitivity", mutant)
    assert _sensitivity_pins_fail(), kind


def test_retained_mask_prefix_or_is_caught(monkeypatch):
    def prefix_or(n_max, g, p):
        m = O.visible_mask(n_max, n_max, g, p)
        earlier = np.logical_or.accumulate(m, axis=0)
        return earlier & (np.arange(n_max)[None, :] <= np.arange(n_max)[:, None])
    monkeypatch.setattr(O, "retained_mask", prefix_or)
    with pytest.raises(AssertionError):
        for case in S.RET_PATTERNS:
            S.test_retained_mask_closed_form(case)


def test_unmutated_helpers_pass():
    assert not _sensitivity_pins_fail()
    for case in S.RET_PATTERNS:
        S.test_retained_mask_closed_form(case)
