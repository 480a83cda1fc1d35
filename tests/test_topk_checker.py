"""The GPU tests' TopK checker (gpu_util.check_topk) catches what it must, on
the CPU: a wrong id in a row with a clear gap, an invalid choice inside a
near-tie row, ids out of order or outside an H3 region; and it accepts the
other correct answer of an exact tie."""

import numpy as np
import pytest

import oracle
from gpu_util import check_topk


def _scores():
    rng = np.random.default_rng(11)
    E = rng.standard_normal((1, 2, 6, 10))
    E[0, 1, 3, :] = [0.5, 2.0, 1.0, 1.0, -1.0, 0.0, 0.2, 0.1, -0.3, 0.4]  # exact tie at the cut (R = 2)
    return E


def test_accepts_the_oracle_and_the_other_tie():
    E = _scores()
    idx, _, gap = oracle.select_topk(E, 2)
    assert check_topk(idx, E, 2, idx, gap) >= 1
    alt = idx.copy()
    assert list(alt[0, 1, 3]) == [1, 2]
    alt[0, 1, 3] = [1, 3]  # the other block of the tie: also a correct top-2
    check_topk(alt, E, 2, idx, gap)


def test_rejects_a_wrong_id_in_a_clear_row():
    E = _scores()
    idx, _, gap = oracle.select_topk(E, 2)
    bad = idx.copy()
    row = bad[0, 0, 0]
    worst = int(np.argmin(E[0, 0, 0]))
    bad[0, 0, 0] = np.sort([row[0], worst]) if worst != row[0] else np.sort([row[1], worst])
    with pytest.raises(AssertionError):
        check_topk(bad, E, 2, idx, gap)


def test_rejects_an_invalid_near_tie_choice():
    E = _scores()
    idx, _, gap = oracle.select_topk(E, 2)
    bad = idx.copy()
    bad[0, 1, 3] = [3, 4]  # keeps the tied block 3 but drops the clear winner 1
    with pytest.raises(AssertionError):
        check_topk(bad, E, 2, idx, gap)


def test_rejects_unsorted_and_out_of_region_ids():
    E = _scores()
    idx, _, gap = oracle.select_topk(E[..., 4:8], 2)
    idx = idx + 4
    check_topk(idx, E, 2, idx, gap, cols=(4, 8))
    with pytest.raises(AssertionError):
        check_topk(idx[..., ::-1], E, 2, idx, gap, cols=(4, 8))
    shifted = idx.copy()
    shifted[0, 0, 0, 0] = 3
    with pytest.raises(AssertionError):
        check_topk(shifted, E, 2, idx, gap, cols=(4, 8))
