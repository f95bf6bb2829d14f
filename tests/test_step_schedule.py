"""GPU check of the benchmark's step schedule against the fp64 oracle.

The step (``StepPlan``) runs the prefill (one oal_fwd call) and the decode
step on the main stream; a second stream runs chi from the start of the step, and
the main stream waits for it at the end of the step.  Several steps run back
to back; every output of the last one must match the oracle: chi, the
prefill outputs, and the decoded token (whose state is the scan's final state
plus that token).
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

    plan = oal.StepPlan(q, k, v, qn, kn, vn, co)
    for _ in range(5):
        plan.run()
    torch.cuda.synchronize()
    pre, dec, chi_plan = plan.prefill, plan.decode, plan.chi

    ao, bo, co_ = O.coeffs_from_factor(wl.coeff["eps"], wl.coeff["L"])
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, ao, bo, co_)
    got = np.concatenate([to_np(pre.y), to_np(dec.y)[:, :, None]], axis=2)
    err = rel_err(got, ref)
    _, chi_ref = O.chi_separable(wl.q[:, :, :N], wl.k[:, :, :N])
    chi_err = np.abs(to_np(chi_plan.chi) / chi_ref - 1).max()
    log(f"[step] two-stream schedule: max rel err {err:.3e}, chi {chi_err:.3e}")
    assert err <= TOL["bf16"]
    assert chi_err <= 1e-4


def test_two_stream_step_full_size_sampled():
    """The same schedule at the timed workload's shape (B=4, Hq=14, Hkv=2,
    N=2048 prompt tokens + 1 decoded, d_h=d_v=64, G=4), where chi runs
    beside a scan long enough for the two to overlap: the decoded token,
    sampled prefill rows and chi against the oracle after several
    back-to-back steps."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    from helpers import sample_rows
    wl = S.make(2, seq_len=2048 + 1)
    N = wl.seq_len - 1
    qa, ka, va = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    q, k, v = (t[:, :, :N].contiguous() for t in (qa, ka, va))
    qn, kn, vn = (t[:, :, N].contiguous() for t in (qa, ka, va))
    a, b, c = oal.coeffs_from_factor(wl.coeff["eps"], wl.coeff["L"])
    co = oal.Coeffs(wl.group_of_dim, a, b, c)
    plan = oal.StepPlan(q, k, v, qn, kn, vn, co)
    for _ in range(4):
        plan.run()
    torch.cuda.synchronize()

    rows = np.append(sample_rows(N, 64, 24, seed=11), N)
    ao, bo, co_ = O.coeffs_from_factor(wl.coeff["eps"], wl.coeff["L"])
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, ao, bo, co_, rows=rows)
    got = np.concatenate([to_np(plan.prefill.y)[:, :, rows[:-1]], to_np(plan.decode.y)[:, :, None]], axis=2)
    err = rel_err(got, ref)
    dec_err = rel_err(got[:, :, -1:], ref[:, :, -1:])
    _, chi_ref = O.chi_separable(wl.q[:, :, :N], wl.k[:, :, :N])
    chi_err = np.abs(to_np(plan.chi.chi) / chi_ref - 1).max()
    log(f"[step] full-size two-stream schedule: rows {err:.3e}, decoded {dec_err:.3e}, chi {chi_err:.3e}")
    assert err <= TOL["bf16"]
    assert dec_err <= TOL["bf16"]
    assert chi_err <= 1e-4


def test_two_stream_step_based_full_size_sampled():
    """The timed step at its full size: the Based Taylor workload (B=8,
    H=16, N=8192 prompt tokens + 1 decoded, d_h=16, d_v=64, bf16), where the
    prefill is the one-pass path.  After back-to-back steps: the decoded
    token of every sequence, sampled prefill rows (all of them at every
    chunk edge of one sequence and head) and chi against the oracle."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    from helpers import sample_rows
    wl = S.make(3, seq_len=8192 + 1)
    N = wl.seq_len - 1
    qa, ka, va = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    q, k, v = (t[:, :, :N].contiguous() for t in (qa, ka, va))
    qn, kn, vn = (t[:, :, N].contiguous() for t in (qa, ka, va))
    co = oal.Coeffs(wl.group_of_dim, wl.coeff["a"], wl.coeff["b"], wl.coeff["c"])
    plan = oal.StepPlan(q, k, v, qn, kn, vn, co)
    for _ in range(3):
        plan.run()
    torch.cuda.synchronize()

    rows = np.append(sample_rows(N, 64, 24, seed=13), N)
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, wl.coeff["a"], wl.coeff["b"], wl.coeff["c"],
                             rows=rows)
    got = np.concatenate([to_np(plan.prefill.y)[:, :, rows[:-1]], to_np(plan.decode.y)[:, :, None]], axis=2)
    err = rel_err(got, ref)
    dec_err = rel_err(got[:, :, -1:], ref[:, :, -1:])
    edges = np.unique(np.concatenate([np.arange(0, N, 64), np.arange(63, N, 64)]))
    ref_e = O.attention_direct(wl.q[:1, :1], wl.k[:1, :1], wl.v[:1, :1], wl.group_of_dim[:1], wl.coeff["a"][:1],
                               wl.coeff["b"][:1], wl.coeff["c"][:1], rows=edges)
    edge_err = rel_err(to_np(plan.prefill.y)[:1, :1, edges], ref_e)
    _, chi_ref = O.chi_separable(wl.q[:, :, :N], wl.k[:, :, :N])
    chi_err = np.abs(to_np(plan.chi.chi) / chi_ref - 1).max()
    log(f"[step] Based full-size step: rows {err:.3e}, chunk edges {edge_err:.3e}, decoded {dec_err:.3e}, "
        f"chi {chi_err:.3e}")
    assert err <= TOL["bf16"]
    assert edge_err <= TOL["bf16"]
    assert dec_err <= TOL["bf16"]
    assert chi_err <= 1e-4
