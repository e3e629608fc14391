"""Pins of the reference greedy selection and draft acceptance (host only)."""
import numpy as np

from greedy_ref import accepted_drafts, greedy_tokens


def test_greedy_tokens_ties_take_lowest_index():
    x = np.array([[0.5, 2.0, 2.0, -1.0], [-3.0, -3.0, -4.0, -3.5]])
    assert greedy_tokens(x).tolist() == [1, 0]


def test_acceptance_prefix_rule():
    g = np.array([[5, 6, 7, 8], [5, 6, 7, 8], [5, 6, 7, 8], [1, 2, 3, 4]], dtype=np.int32)
    t = np.array([[9, 5, 6, 7],   # every draft equals the greedy token before it
                  [9, 5, 0, 7],   # the second draft differs: one accepted (the third does not count)
                  [9, 0, 6, 7],   # the first draft differs: none accepted
                  [9, 1, 2, 0]], dtype=np.int32)
    assert accepted_drafts(t, g).tolist() == [3, 1, 0, 2]


def test_single_token_step_accepts_nothing():
    assert accepted_drafts(np.array([[3]], dtype=np.int32), np.array([[4]], dtype=np.int32)).tolist() == [0]
