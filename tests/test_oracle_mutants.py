"""Plant one plausible mistake at a time in a step of the oracle (on the CPU)
and check that the independent pins catch it.

The pins used here exclude the materialised brute force, the fsum variant
and torch's SDPA: closed forms, invariants and the page's printed example
must be strong enough on their own.
"""

import numpy as np
import pytest

# a planted mistake may produce inf - inf or 0/0 on the way to failing a pin
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

from oracle import fp64 as O
from tests.oracle_pins import INDEPENDENT_PINS

MUTANTS = {
    "scores_transposed": ("_scores", lambda q, k, scale: scale * (k @ q.T) if q.shape[0] == k.shape[0]
                          else scale * (q @ k.T)[:, ::-1]),
    "scale_dropped": ("_scores", lambda q, k, scale: q @ k.T),
    "scale_squared": ("_scores", lambda q, k, scale: scale * scale * (q @ k.T)),
    "causal_strict": ("_visible", lambda rows, n, causal, kv: (
        (np.arange(n)[None, :] < rows[:, None]) if causal else np.ones((len(rows), n), bool))
        & (True if kv is None else kv[None, :])),
    "causal_local_rows": ("_visible", lambda rows, n, causal, kv: (
        (np.arange(n)[None, :] <= (rows - rows[0])[:, None]) if causal else np.ones((len(rows), n), bool))
        & (True if kv is None else kv[None, :])),
    "causal_upper": ("_visible", lambda rows, n, causal, kv: (
        (np.arange(n)[None, :] >= rows[:, None]) if causal else np.ones((len(rows), n), bool))
        & (True if kv is None else kv[None, :])),
    "key_mask_ignored": ("_visible", lambda rows, n, causal, kv: (
        (np.arange(n)[None, :] <= rows[:, None]) if causal else np.ones((len(rows), n), bool))),
    "no_max_shift": ("_row_max", lambda s: np.zeros(s.shape[0])),
    "exp_sign_flipped": ("_exp_shifted", lambda s, m: np.exp(m[:, None] - s)),
    "exp_base_two": ("_exp_shifted", lambda s, m: np.exp2(s - m[:, None])),
    "sum_drops_last_key": ("_row_sum", lambda e: e[:, :-1].sum(axis=1)),
    "values_reversed": ("_weighted_values", lambda e, v, vis: e @ v[::-1]),
    "hidden_values_multiplied": ("_weighted_values", lambda e, v, vis: e @ v),
    "not_normalised": ("_normalise", lambda ou, l: ou),
    "lse_without_max": ("_lse", lambda m, l: np.log(l)),
    "lse_base_two": ("_lse", lambda m, l: m + np.log2(l)),
    "lse_of_sum_only": ("_lse", lambda m, l: m),
    "key_mask_inverted": ("_visible", lambda rows, n, causal, kv: (
        (np.arange(n)[None, :] <= rows[:, None]) if causal else np.ones((len(rows), n), bool))
        & (True if kv is None else ~kv[None, :])),
    "empty_rows_nan": ("_empty_row_result", lambda o, lse, empty: (
        np.where(empty[:, None], np.nan, o), np.where(empty, np.nan, lse))),
    "empty_rows_lse_zero": ("_empty_row_result", lambda o, lse, empty: (
        np.where(empty[:, None], 0.0, o), np.where(empty, 0.0, lse))),
    "empty_rows_uniform": ("_empty_row_result", lambda o, lse, empty: (o, lse)),
    "block_mask_roles_swapped": ("_block_visible", lambda rows, n, bm: np.asarray(bm[0], dtype=bool)[
        (np.arange(n)[None, :] // bm[2]) % np.asarray(bm[0]).shape[0],
        (rows[:, None] // bm[1]) % np.asarray(bm[0]).shape[1]]),
    "block_sizes_swapped": ("_block_visible", lambda rows, n, bm: np.asarray(bm[0], dtype=bool)[
        (rows[:, None] // bm[2]) % np.asarray(bm[0]).shape[0], np.arange(n)[None, :] // bm[1]]),
    "block_mask_ignored": ("_block_visible", lambda rows, n, bm: np.ones((len(rows), n), dtype=bool)),
    "block_mask_local_rows": ("_block_visible", lambda rows, n, bm: np.asarray(bm[0], dtype=bool)[
        (rows - rows[0])[:, None] // bm[1], np.arange(n)[None, :] // bm[2]]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_independent_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in INDEPENDENT_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every independent pin"


def _p_ignoring_key_mask(q, k, scale, causal, rows, key_valid=None, block_mask=None):
    """Probabilities that forget the key-padding mask."""
    s = O._scores(q[rows], k, scale)
    s = np.where(O._visible(rows, k.shape[0], causal, None), s, -np.inf)
    e = np.exp(s - s.max(axis=1)[:, None])
    return e / e.sum(axis=1)[:, None]


def _p_ignoring_block_mask(q, k, scale, causal, rows, key_valid=None, block_mask=None):
    """Probabilities that forget the block mask."""
    s = O._scores(q[rows], k, scale)
    s = np.where(O._visible(rows, k.shape[0], causal, key_valid), s, -np.inf)
    empty = ~np.isfinite(s).any(axis=1)
    s[empty] = 0.0
    e = np.where(np.isfinite(s), np.exp(s - s.max(axis=1)[:, None]), 0.0)
    return np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, e.sum(axis=1))[:, None])


def _p_block_mask_transposed(q, k, scale, causal, rows, key_valid=None, block_mask=None):
    """Probabilities that read the block mask with query and key blocks swapped."""
    s = O._scores(q[rows], k, scale)
    vis = O._visible(rows, k.shape[0], causal, key_valid)
    if block_mask is not None:
        m, bq, bk = block_mask
        m = np.asarray(m, dtype=bool)
        vis &= m[(np.arange(k.shape[0])[None, :] // bk) % m.shape[0], (rows[:, None] // bq) % m.shape[1]]
    s = np.where(vis, s, -np.inf)
    empty = ~vis.any(axis=1)
    s[empty] = 0.0
    e = np.where(vis, np.exp(s - s.max(axis=1)[:, None]), 0.0)
    return e / np.where(empty, 1.0, e.sum(axis=1))[:, None]


def _p_empty_rows_uniform(q, k, scale, causal, rows, key_valid=None, block_mask=None):
    """Probabilities that spread a row with no visible key uniformly over
    every key instead of leaving it at 0."""
    s = O._scores(q[rows], k, scale)
    vis = O._visible(rows, k.shape[0], causal, key_valid)
    if block_mask is not None:
        vis &= O._block_visible(rows, k.shape[0], block_mask)
    s = np.where(vis, s, -np.inf)
    empty = ~vis.any(axis=1)
    s[empty] = 0.0
    e = np.exp(s - s.max(axis=1)[:, None])
    return e / e.sum(axis=1)[:, None]


# mistakes in the gradient steps (oracle.backward)
BACKWARD_MUTANTS = {
    "probabilities_ignore_key_mask": ("_probabilities", _p_ignoring_key_mask),
    "probabilities_empty_rows_uniform": ("_probabilities", _p_empty_rows_uniform),
    "probabilities_ignore_block_mask": ("_probabilities", _p_ignoring_block_mask),
    "probabilities_block_mask_transposed": ("_probabilities", _p_block_mask_transposed),
    "dv_not_transposed": ("_dv", lambda p, do: p @ do),
    "dp_uses_values_untransposed": ("_dp", lambda do, v: do @ v[::-1].T),
    "delta_sums_dp_only": ("_delta", lambda p, dp: dp.sum(axis=1)),
    "delta_dropped": ("_delta", lambda p, dp: np.zeros(p.shape[0])),
    "ds_sign_flipped": ("_ds", lambda p, dp, delta: p * (delta[:, None] - dp)),
    "ds_without_p": ("_ds", lambda p, dp, delta: dp - delta[:, None]),
    "dq_scale_dropped": ("_dq", lambda ds, k, scale: ds @ k),
    "dk_not_transposed": ("_dk", lambda ds, q, scale: scale * (ds @ q)),
    "dk_scale_squared": ("_dk", lambda ds, q, scale: scale * scale * (ds.T @ q)),
}


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_independent_pins_catch_backward_mutant(name, monkeypatch):
    from oracle import backward as OB
    attr, fn = BACKWARD_MUTANTS[name]
    monkeypatch.setattr(OB, attr, fn)
    caught = []
    for pin in INDEPENDENT_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every independent pin"


# mistakes in the steps only the sampled gradients use, caught by comparing
# them with the full backward oracle (itself pinned above)
from oracle.backward import _probability_columns as _ORIGINAL_COLUMNS  # noqa: E402

SAMPLED_MUTANTS = {
    "delta_from_output_dropped": ("_delta_from_output", lambda do, o: np.zeros(do.shape[0])),
    "delta_from_output_values": ("_delta_from_output", lambda do, o: do.sum(axis=1)),
    "columns_without_lse": ("_probability_columns", lambda q, kc, lse, scale, causal, cols, cols_valid=None, block_mask=None: (
        np.exp(scale * (q @ kc.T)))),
    "columns_causal_reversed": ("_probability_columns", lambda q, kc, lse, scale, causal, cols, cols_valid=None, block_mask=None: np.where(
        (cols[None, :] >= np.arange(q.shape[0])[:, None]) if causal else True,
        np.exp(scale * (q @ kc.T) - lse[:, None]), 0.0)),
    "columns_ignore_key_mask": ("_probability_columns", lambda q, kc, lse, scale, causal, cols, cols_valid=None, block_mask=None: (
        np.where((cols[None, :] <= np.arange(q.shape[0])[:, None]) if causal else True,
                 np.exp(scale * (q @ kc.T) - lse[:, None]), 0.0))),
    "columns_ignore_block_mask": ("_probability_columns",
                                  lambda q, kc, lse, scale, causal, cols, cols_valid=None, block_mask=None: (
                                      _ORIGINAL_COLUMNS(q, kc, lse, scale, causal, cols, cols_valid))),
    "columns_scale_dropped": ("_probability_columns", lambda q, kc, lse, scale, causal, cols, cols_valid=None, block_mask=None: np.where(
        (cols[None, :] <= np.arange(q.shape[0])[:, None]) if causal else True,
        np.exp(q @ kc.T - lse[:, None]), 0.0)),
}


@pytest.mark.parametrize("name", sorted(SAMPLED_MUTANTS))
def test_row_sampling_pin_catches_sampled_mutant(name, monkeypatch):
    from oracle import backward as OB
    from tests.oracle_pins import pin_backward_row_sampling
    attr, fn = SAMPLED_MUTANTS[name]
    monkeypatch.setattr(OB, attr, fn)
    with pytest.raises((AssertionError, ValueError, FloatingPointError, IndexError)):
        pin_backward_row_sampling()
