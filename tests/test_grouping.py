"""Host grouping utilities.

* ``groups_from_contribution``: contribution-sorted split with given sizes.
* ``group_dims`` / ``group_dims_budget``: the library's outlier-aware and
  fixed-budget grouping (OAL paper, App. B) through the C ABI, against the
  oracle's step-by-step version on the same inputs and bootstrap replicates.
  Both sides work in fp64 in the same order, so group maps, group counts,
  gap ratios and supports must agree exactly.
"""

import ctypes

import numpy as np
import pytest

import oracle as O
from grouped_quadratic_softmax_amd.grouping import (bootstrap_indices, group_dims, group_dims_budget,
                                                    groups_from_contribution)


def test_sorted_split_and_tail_singletons():
    chi = np.array([[0.5, 0.1, 9.0, 0.3, 0.2, 4.0, 0.4, 0.6]])
    g = groups_from_contribution(chi, [3, 3], 2)
    # ascending order: 1(0.1) 4(0.2) 3(0.3) | 6(0.4) 0(0.5) 7(0.6) | 5(4.0) | 2(9.0)
    assert g.tolist() == [[1, 0, 3, 0, 0, 2, 1, 1]]


def test_ties_keep_index_order():
    chi = np.array([[1.0, 1.0, 1.0, 1.0]])
    assert groups_from_contribution(chi, [2], 2).tolist() == [[0, 0, 1, 2]]


def test_sorted_split_matches_oracle_with_ties():
    """The library's contribution-sorted split and the oracle's (written from
    the pages separately) give identical maps, also with many exact ties."""
    rng = np.random.default_rng(21)
    bulk, tail = [11, 11, 10, 10, 10, 10], 2
    for chi in (rng.random((5, 64)), np.round(rng.random((5, 64)) * 4) / 4):
        assert np.array_equal(groups_from_contribution(chi, bulk, tail), O.groups_sorted_split(chi, bulk, tail))


def test_bad_budget():
    with pytest.raises(ValueError):
        groups_from_contribution(np.zeros((1, 4)), [2], 1)


def _synthetic_chi(rng, P, Hq, d, n_out=None, spread=0.3):
    """Per-prompt scores shaped like Eq. (2) on outlier inputs: a bulk near
    2/(pi sqrt(d)) with prompt-to-prompt spread, plus planted outlier
    dimensions whose size varies by prompt.  Head h carries h % 4 outliers
    (unless n_out is given) of strengths 1.4, 2.2 and 6 times the bulk, so
    that gaps range from unstable to clear."""
    base = 2 / np.pi / np.sqrt(d)
    chi = base * rng.lognormal(0.0, spread, size=(P, Hq, d))
    for h in range(Hq):
        n = h % 4 if n_out is None else n_out
        dims = rng.choice(d, size=n, replace=False)
        for i, r in enumerate(dims):
            chi[:, h, r] *= (1.4, 2.2, 6.0)[i % 3] * rng.lognormal(0.0, 0.6, size=P)
    return chi.astype(np.float32)


@pytest.mark.parametrize("alpha,gamma,g_min", [(0.25, 0.9, 2), (0.5, 0.5, 2), (0.25, 0.9, 4), (1.0, 0.0, 2)])
def test_bootstrap_grouping_matches_oracle(alpha, gamma, g_min):
    rng = np.random.default_rng(int(alpha * 100 + gamma * 10 + g_min))
    P, Hq, d = 12, 8, 64
    chi = _synthetic_chi(rng, P, Hq, d)
    boot = bootstrap_indices(P, 200, seed=5)
    gid, ng, rho, sup = group_dims(chi, alpha, gamma, g_min=g_min, boot=boot, details=True)
    for h in range(Hq):
        og, oG, orho, osup = O.group_dims_bootstrap(chi[:, h, :].tolist(), boot.tolist(), alpha, gamma,
                                                    g_min=g_min)
        assert gid[h].tolist() == og and ng[h] == oG, h
        cand = sorted(orho)
        assert np.isnan(np.delete(rho[h], cand)).all() and np.isnan(np.delete(sup[h], cand)).all()
        assert rho[h, cand].tolist() == [orho[k] for k in cand]
        assert sup[h, cand].tolist() == [osup[k] for k in cand]
        # a valid partition: ids 0..G-1, each used, contiguous in the sorted order
        assert sorted(set(gid[h].tolist())) == list(range(ng[h]))
        order = np.argsort(chi[:, h, :].astype(np.float64).mean(0), kind="stable")
        assert (np.diff(gid[h][order]) >= 0).all()
        assert ng[h] >= g_min


def test_bootstrap_grouping_edge_shapes():
    rng = np.random.default_rng(3)
    for P, d, B in ((1, 2, 1), (2, 16, 7), (40, 32, 50)):
        chi = _synthetic_chi(rng, P, 1, d, n_out=1)
        boot = bootstrap_indices(P, B, seed=P)
        for alpha in (0.01, 0.5, 1.0):
            gid, ng = group_dims(chi, alpha, 0.5, boot=boot)
            og, oG, _, _ = O.group_dims_bootstrap(chi[:, 0, :].tolist(), boot.tolist(), alpha, 0.5)
            assert gid[0].tolist() == og and ng[0] == oG


@pytest.mark.parametrize("G", [1, 2, 3, 5, 8, 64])
def test_budget_grouping_matches_oracle(G):
    rng = np.random.default_rng(G)
    chi = _synthetic_chi(rng, 1, 3, 64)[0]
    chi[1, 10:20] = chi[1, 5]  # equal scores: order by index
    gid = group_dims_budget(chi, G)
    for h in range(3):
        og, _ = O.group_dims_budget(chi[h].tolist(), G)
        assert gid[h].tolist() == og


def test_grouping_rejects_bad_arguments():
    from grouped_quadratic_softmax_amd import _lib as L
    lib = L.lib()
    chi = np.ones((2, 4), np.float32)
    boot = np.zeros((3, 2), np.int32)
    out = np.empty(4, np.int32)
    ok = L.OalGroupParams(0.5, 0.5, 1.5, 1e-12, 2)

    def call(d=4, P=2, c=chi, B=3, bt=boot, prm=ok):
        return lib.oal_group_dims(d, P, c.ctypes.data, B, bt.ctypes.data, ctypes.byref(prm), out.ctypes.data,
                                  None, None)

    assert call() == 2
    assert call(d=1) == L.OAL_ERR_INVALID_ARG
    assert call(B=0) == L.OAL_ERR_INVALID_ARG
    for bad in (L.OalGroupParams(0.0, 0.5, 1.5, 1e-12, 2), L.OalGroupParams(0.5, 1.5, 1.5, 1e-12, 2),
                L.OalGroupParams(0.5, 0.5, 1.5, 0.0, 2), L.OalGroupParams(0.5, 0.5, 1.5, 1e-12, 5),
                L.OalGroupParams(0.5, 0.5, float("nan"), 1e-12, 2)):
        assert call(prm=bad) == L.OAL_ERR_INVALID_ARG
    neg = chi.copy()
    neg[1, 2] = -1.0
    assert call(c=neg) == L.OAL_ERR_INVALID_ARG
    nan = chi.copy()
    nan[0, 0] = np.nan
    assert call(c=nan) == L.OAL_ERR_INVALID_ARG
    assert call(bt=np.full((3, 2), 2, np.int32)) == L.OAL_ERR_INVALID_ARG
    assert lib.oal_group_dims_budget(4, chi.ctypes.data, 0, 1e-12, out.ctypes.data) == L.OAL_ERR_INVALID_ARG
    assert lib.oal_group_dims_budget(4, chi.ctypes.data, 5, 1e-12, out.ctypes.data) == L.OAL_ERR_INVALID_ARG
    assert lib.oal_group_dims_budget(4, chi.ctypes.data, 2, 1e-12, out.ctypes.data) == 2


def test_bootstrap_indices_shape_and_range():
    b = bootstrap_indices(40, 1000, seed=1)
    assert b.shape == (1000, 40) and b.dtype == np.int32
    assert b.min() >= 0 and b.max() < 40
    assert (bootstrap_indices(40, 1000, seed=1) == b).all()
