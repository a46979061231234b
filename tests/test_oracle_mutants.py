"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant below is a plausible slip (a wrong level index, a decay range
off by one, swapped query/key roles, lambda read at the wrong level, a
dropped diagonal term, a wrong group mapping).  The mistake is planted in the
oracle module itself, on the CPU, and the pins of test_oracle_pins are run
against it; the test passes when some pin rejects the mutant.
"""
import os

import numpy as np
import pytest

from oracle import fenwick, loglin_ref

from . import test_oracle_pins as pins


def pin_results(golden_dir):
    """Run the pins as checks; return {name: passed}."""
    res = {}

    def run(name, fn):
        try:
            fn()
            res[name] = True
        except AssertionError:
            res[name] = False

    run("worked_T4", lambda: pins.test_worked_example_T4(golden_dir))
    run("closed_T1_T2", pins.test_closed_form_T1_T2)
    run("ssd", lambda: pins.test_reduces_to_ssd_when_lambda_constant(64))
    run("ssd_scaled", pins.test_reduces_to_scaled_ssd_when_lambda_level_free)
    run("prefix_sum", pins.test_reduces_to_causal_prefix_sum)
    run("recurrence", lambda: pins.test_dense_equals_fenwick_recurrence(33, 5))
    for lev in range(4):
        run(f"bucket_l{lev}",
            lambda lev=lev: pins.test_onehot_level_equals_bucket_brute_force(lev))
    return res


def _bitlen_minus_one(t, s):
    return np.maximum(fenwick.levels(t, s) - 1, 0)


def _absolute_position_level(t, s):
    # the partition the write-up rejects: level from the key's absolute position
    s = np.broadcast_to(np.asarray(s), np.broadcast_shapes(np.shape(t), np.shape(s)))
    return np.where(s == np.asarray(t), 0, fenwick.bit_length(s))


def _decay_includes_a_s(cum, t, s):
    prev = np.concatenate([[0.0], cum])
    return cum[t] - prev[s]


def _decay_excludes_a_t(cum, t, s):
    prev = np.concatenate([[0.0], cum])
    return prev[t] - prev[s]


def _decay_sign_flipped(cum, t, s):
    return cum[s] - cum[t]


def _swapped_roles(C_bg, B_bg, rows, ncols):
    return np.asarray(B_bg[rows], np.float64) @ np.asarray(C_bg[:ncols], np.float64).T


def _lambda_reversed(lam_rows, lev):
    return np.take_along_axis(lam_rows[:, ::-1], lev, axis=1)


def _no_diagonal(lam_rows, lev):
    w = np.take_along_axis(lam_rows, lev, axis=1)
    return np.where(lev == 0, 0.0, w)


def _group_modulo(h, nheads, ngroups):
    return h % ngroups


MUTANTS = {
    "level_off_by_one": ("_levels", _bitlen_minus_one),
    "level_absolute_position": ("_levels", _absolute_position_level),
    "decay_includes_a_s": ("_log_decay", _decay_includes_a_s),
    "decay_excludes_a_t": ("_log_decay", _decay_excludes_a_t),
    "decay_sign": ("_log_decay", _decay_sign_flipped),
    "query_key_swapped": ("_interaction", _swapped_roles),
    "lambda_levels_reversed": ("_level_weight", _lambda_reversed),
    "diagonal_dropped": ("_level_weight", _no_diagonal),
    "group_modulo": ("_group_of", _group_modulo),
}


def test_unmutated_oracle_passes_every_pin(golden_dir):
    res = pin_results(golden_dir)
    assert all(res.values()), res


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, golden_dir, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(loglin_ref, attr, fn)
    with np.errstate(over="ignore", invalid="ignore"):
        res = pin_results(golden_dir)
    failed = [k for k, ok in res.items() if not ok]
    assert failed, f"mutant {name} passed every pin"
