"""The parity checker itself (CPU): what it accepts as a valid top-K selection
and what it rejects (routing equation of section 3: the chunks of rank < K)."""
import math

import numpy as np
import pytest

from tests.parity_util import TIE_BAND, Tally, check_selection


def _ref(scores, K):
    """Oracle-shaped record of one G = 1 row with the given group scores."""
    s = np.asarray(scores, dtype=np.float64)[None, :]
    order = np.lexsort((np.arange(s.shape[1]), -s[0]))
    sel = np.sort(order[:K])
    gap = float(s[0, order[K - 1]] - s[0, order[K]]) if s.shape[1] > K else math.inf
    return dict(sel=sel, gap=gap, s_hat=s)


def test_exact_selection_accepted():
    r = _ref([10.0, 5.0, 3.0, 1.0], 2)
    assert check_selection([0, 1], r, 2) == "exact"


def test_tie_alternative_accepted():
    # chunks 1 and 2 are within the band of each other: either may take the last slot
    r = _ref([10.0, 5.0 + 0.3 * TIE_BAND, 5.0, 1.0], 2)
    assert check_selection([0, 2], r, 2) == "tie"


def test_tie_alternative_dropping_the_top_chunk_rejected():
    # scores [10, 5.00005, 5], K = 2: {1, 2} is not a top-2 (chunk 0 is far above)
    r = _ref([10.0, 5.00005, 5.0], 2)
    with pytest.raises(AssertionError):
        check_selection([1, 2], r, 2)


def test_negative_or_out_of_range_ids_rejected():
    r = _ref([10.0, 5.00005, 5.0, 5.0], 2)
    with pytest.raises(AssertionError):
        check_selection([-1, 3], r, 2)          # -1 would index the last chunk
    with pytest.raises(AssertionError):
        check_selection([0, 4], r, 2)           # past |C_i|


def test_padding_order_and_length_rejected():
    r = _ref([3.0, 2.0], 4)                     # |C_i| = 2 < K: both chosen, then -1
    assert check_selection([0, 1, -1, -1], r, 4) == "exact"
    with pytest.raises(AssertionError):
        check_selection([0, 1, 0, -1], r, 4)    # padding slot not -1
    with pytest.raises(AssertionError):
        check_selection([1, 0, -1, -1], r, 4)   # not ascending
    with pytest.raises(AssertionError):
        check_selection([0, 1, -1], r, 4)       # wrong number of slots


def test_difference_outside_band_rejected():
    r = _ref([10.0, 5.0, 4.0, 1.0], 2)
    with pytest.raises(AssertionError):
        check_selection([0, 2], r, 2)


def test_tally_relative_error_per_head():
    # a head whose outputs are small is held to its own scale: an all-zero
    # output passes the absolute bar but not the relative one
    t = Tally()
    want = np.full((2, 8), 4e-3)
    want[0] = 0.5
    got = want.copy()
    got[1] = 0.0
    t.add(("case", 0, 0), got, want, "bf16", "test row")
    assert t.max_err <= 2e-2
    with pytest.raises(AssertionError):
        t.check_rel("bf16")
