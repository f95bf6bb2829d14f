"""Host grouping utility: contribution-sorted split (stable ascending order)."""

import numpy as np
import pytest

from grouped_quadratic_softmax_amd.grouping import groups_from_contribution


def test_sorted_split_and_tail_singletons():
    chi = np.array([[0.5, 0.1, 9.0, 0.3, 0.2, 4.0, 0.4, 0.6]])
    g = groups_from_contribution(chi, [3, 3], 2)
    # ascending order: 1(0.1) 4(0.2) 3(0.3) | 6(0.4) 0(0.5) 7(0.6) | 5(4.0) | 2(9.0)
    assert g.tolist() == [[1, 0, 3, 0, 0, 2, 1, 1]]


def test_ties_keep_index_order():
    chi = np.array([[1.0, 1.0, 1.0, 1.0]])
    assert groups_from_contribution(chi, [2], 2).tolist() == [[0, 0, 1, 2]]


def test_bad_budget():
    with pytest.raises(ValueError):
        groups_from_contribution(np.zeros((1, 4)), [2], 1)
