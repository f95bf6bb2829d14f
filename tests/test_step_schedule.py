"""GPU check of the benchmark's step schedule against the fp64 oracle.

The step enqueues chi on a second stream right after the chunk scan, then the
readout and one decode step per sequence on the main stream, and joins the
streams at the end of the step (steps may overlap the previous step's side
work).  Several steps run back to back; every output of the last one must
match the oracle: chi, the prefill outputs, and the decoded token (whose
state is the scan's final state plus that token).
"""

import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import TOL, log, oracle_coeffs, rel_err, require_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu


def test_two_stream_step_matches_oracle():
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=2, n_q_heads=4, n_kv_heads=2, seq_len=301)
    N = wl.seq_len - 1
    qa, ka, va = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    q, k, v = (t[:, :, :N].contiguous() for t in (qa, ka, va))
    qn, kn, vn = (t[:, :, N].contiguous() for t in (qa, ka, va))
    a, b, c = oal.coeffs_from_factor(wl.coeff["eps"], wl.coeff["L"])
    co = oal.Coeffs(wl.group_of_dim, a, b, c)

    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    pre = oal.PrefillPlan(q, k, v, co)
    dec = oal.DecodePlan(qn, kn, vn, co, pre.state_out)
    with torch.cuda.stream(side):
        chi_plan = oal.ContribPlan(q, k)
    for _ in range(5):
        pre.states()
        chi_plan.run()
        pre.outputs()
        dec.run()
        main.wait_stream(side)
    torch.cuda.synchronize()

    ao, bo, co_ = O.coeffs_from_factor(wl.coeff["eps"], wl.coeff["L"])
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, ao, bo, co_)
    got = np.concatenate([to_np(pre.y), to_np(dec.y)[:, :, None]], axis=2)
    err = rel_err(got, ref)
    _, chi_ref = O.chi_separable(wl.q[:, :, :N], wl.k[:, :, :N])
    chi_err = np.abs(to_np(chi_plan.chi) / chi_ref - 1).max()
    log(f"[step] two-stream schedule: max rel err {err:.3e}, chi {chi_err:.3e}")
    assert err <= TOL["bf16"]
    assert chi_err <= 1e-4
