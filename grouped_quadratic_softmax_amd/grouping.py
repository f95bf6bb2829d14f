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
