"""Host-side grouping of head dimensions by contribution score.

The OAL paper (sec. 4.2 and App. B) groups the d_h dimensions of every query
head by sorting their contribution scores chi_r (Eq. (2)) in ascending order
with a stable sort and cutting the sorted order into contiguous runs: a large
low-contribution bulk and finer groups in the high-contribution tail.
"""

from __future__ import annotations

import numpy as np


def groups_from_contribution(chi, bulk_sizes, n_tail):
    """Contribution-sorted grouping with a fixed budget.

    chi: [Hq, d_h] scores.  For each head the dimensions are stably sorted by
    ascending chi; the last ``n_tail`` become singleton groups (ids after the
    bulk groups, in ascending chi order) and the remaining dimensions, in the
    same sorted order, are split into contiguous bulk groups of the given
    sizes (ids 0, 1, ...).  Returns int32 [Hq, d_h] group ids.
    """
    chi = np.asarray(chi, dtype=np.float64)
    Hq, d = chi.shape
    bulk_sizes = [int(x) for x in bulk_sizes]
    if sum(bulk_sizes) + n_tail != d or min(bulk_sizes + [1]) < 1 or n_tail < 0:
        raise ValueError("bulk sizes plus tail must partition the head dimensions")
    out = np.empty((Hq, d), dtype=np.int32)
    for h in range(Hq):
        order = np.argsort(chi[h], kind="stable")
        pos = 0
        for g, size in enumerate(bulk_sizes):
            out[h, order[pos:pos + size]] = g
            pos += size
        for i in range(n_tail):
            out[h, order[pos + i]] = len(bulk_sizes) + i
    return out


def bootstrap_indices(n_prompts: int, n_boot: int = 1000, seed: int = 0):
    """Prompt indices of ``n_boot`` bootstrap replicates, each ``n_prompts``
    draws with replacement from 0..n_prompts-1 (int32 [n_boot, n_prompts]),
    from numpy's seeded default generator."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, n_prompts, size=(n_boot, n_prompts)).astype(np.int32)


def group_dims(chi_per_prompt, alpha, gamma, tau=1.5, g_min=2, eps=1e-12, boot=None, n_boot=1000, seed=0,
               details=False):
    """Outlier-aware grouping of every query head (OAL paper, App. B), by the
    library's ``oal_group_dims``.

    chi_per_prompt: [P, Hq, d_h] per-prompt contribution scores (e.g.
    ``contrib(..., per_prompt=True)``); boot: int32 [B, P] bootstrap prompt
    indices shared by all heads (default: ``bootstrap_indices(P, n_boot,
    seed)``).  Returns int32 [Hq, d_h] group ids and int32 [Hq] group counts
    (and, with ``details``, fp64 [Hq, d_h] gap ratios and supports, NaN off
    the candidate cuts).  Group 0 is each head's low-contribution bulk.
    """
    import ctypes

    from . import _lib as L
    chi = np.ascontiguousarray(np.asarray(chi_per_prompt, dtype=np.float32))
    if chi.ndim != 3:
        raise ValueError("chi_per_prompt must be [P, Hq, d_h]")
    P, Hq, d = chi.shape
    boot = bootstrap_indices(P, n_boot, seed) if boot is None else np.ascontiguousarray(boot, dtype=np.int32)
    if boot.ndim != 2 or boot.shape[1] != P:
        raise ValueError("boot must be [B, P]")
    prm = L.OalGroupParams(float(alpha), float(gamma), float(tau), float(eps), int(g_min))
    gid = np.empty((Hq, d), np.int32)
    ng = np.empty(Hq, np.int32)
    rho = np.empty((Hq, d), np.float64)
    sup = np.empty((Hq, d), np.float64)
    for h in range(Hq):
        head = np.ascontiguousarray(chi[:, h, :])
        g = L.lib().oal_group_dims(d, P, head.ctypes.data, boot.shape[0], boot.ctypes.data, ctypes.byref(prm),
                                   gid[h].ctypes.data, rho[h].ctypes.data, sup[h].ctypes.data)
        if g < 1:
            L.check(g, "oal_group_dims")
        ng[h] = g
    return (gid, ng, rho, sup) if details else (gid, ng)


def group_dims_budget(chi, n_groups, eps=1e-12):
    """Fixed-budget grouping of every head (OAL paper, App. B, group-budget
    diagnostic), by the library's ``oal_group_dims_budget``: chi [Hq, d_h]
    -> int32 [Hq, d_h] group ids in 0..n_groups-1."""
    from . import _lib as L
    chi = np.ascontiguousarray(np.asarray(chi, dtype=np.float32))
    Hq, d = chi.shape
    gid = np.empty((Hq, d), np.int32)
    for h in range(Hq):
        row = np.ascontiguousarray(chi[h])
        g = L.lib().oal_group_dims_budget(d, row.ctypes.data, int(n_groups), float(eps), gid[h].ctypes.data)
        if g < 1:
            L.check(g, "oal_group_dims_budget")
    return gid
