"""GPU parity of oal_fwd (chunked causal prefill) against the fp64 oracle.

Small cases compare every output row; the full-size workloads run exactly as
the benchmark launches them and compare a seeded sample of rows (every chunk
boundary where affordable, the last row, random rows).
"""

import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import (TOL, diag_form_mask, gpu_coeffs, gpu_prep, log, oracle_coeffs, oracle_prep, rel_err,
                     require_gpu, sample_rows, to_dev, to_np, with_l2_premap)

pytestmark = pytest.mark.gpu


def _run_case(wl, groups=None, rows=None, tol=None):
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    groups = wl.group_of_dim if groups is None else groups
    log(f"[fwd] {wl.name} B={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} N={wl.seq_len} d={wl.d_h} "
        f"G={wl.n_groups} {wl.dtype} rows={'all' if rows is None else len(rows)}")
    q, k, v = to_dev(wl.q, wl.dtype), to_dev(wl.k, wl.dtype), to_dev(wl.v, wl.dtype)
    y = to_np(oal.fwd(q, k, v, gpu_coeffs(wl, groups), gpu_prep(wl)))
    a, b, c = oracle_coeffs(wl)
    ref = O.attention_direct(wl.q, wl.k, wl.v, groups, a, b, c, oracle_prep(wl), rows=rows)
    got = y if rows is None else y[:, :, rows]
    err = rel_err(got, ref)
    log(f"[fwd]   max rel err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= (tol or TOL[wl.dtype]), err
    return y


def test_c1_fp32_full():
    _run_case(S.make(1))


def test_c1_fp32_ragged():
    _run_case(S.make(1, seq_len=200))


def test_c2_gqa_bf16_small():
    _run_case(S.make(2, batch=2, seq_len=300))


def test_c2_gqa_fp32_small():
    _run_case(S.make(2, batch=1, seq_len=130, dtype="f32"))


def test_c3_taylor_d16_small():
    _run_case(S.make(3, batch=2, n_q_heads=4, n_kv_heads=4, seq_len=333))


def test_c3_taylor_d16_fp32():
    _run_case(S.make(3, batch=1, n_q_heads=2, n_kv_heads=2, seq_len=200, dtype="f32"))


def test_c4_rebased_elementwise_premap():
    # the default ReBased reading: one singleton group per dimension, c = d I
    wl = S.make(4, batch=2, n_q_heads=2, n_kv_heads=2, seq_len=150)
    assert wl.n_groups == 64
    _run_case(wl)


def _diag_workload(d, dtype, seed, Hq=4, Hkv=2, N=200, B=2):
    """Singleton groups (a permutation per head), diagonal c > 0 and b, with a
    large enough that every kernel value is >= 0.05:
    c x^2 + b x >= -b^2 / (4 c)."""
    wl = S.make(2, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, seq_len=N, dtype=dtype)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, 64)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = S.bf16_round(q), S.bf16_round(k), S.bf16_round(v)
    groups = np.stack([rng.permutation(d) for _ in range(Hq)]).astype(np.int32)
    cd = rng.uniform(0.5, 2.0, (Hq, d))
    b = rng.uniform(-1.0, 1.0, (Hq, d))
    c = np.stack([np.diag(x) for x in cd])
    # per-dimension terms in x = q k / sqrt(d): b/sqrt(d) x + c/d x^2
    a = 0.05 + ((b / np.sqrt(d)) ** 2 / (4 * cd / d)).sum(axis=1)
    wl.q, wl.k, wl.v, wl.d_h, wl.n_groups = q, k, v, d, d
    wl.group_of_dim = groups
    wl.coeff = {"kind": "abc", "a": a, "b": b, "c": c}
    return wl


@pytest.mark.parametrize("d", [16, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dimensionwise_form(d, dtype):
    _run_case(_diag_workload(d, dtype, seed=d))


@pytest.mark.parametrize("N", [31, 32, 33, 129, 200, 300, 1000])
def test_dimensionwise_form_own_keys(N):
    """d_h = 64, bf16, a KV head per query head: the one-wave build (32-token
    chunks).  N = 33: two segments in three launches; 129 and 200: one group
    of four chained segments (129: the fourth empty); 300: two chained groups
    whose second holds one segment and three empty ones; 1000: two full
    groups with a ragged last chunk."""
    _run_case(_diag_workload(64, "bf16", seed=640 + N, Hq=3, Hkv=3, N=N))


def test_dimensionwise_chained_back_to_back():
    """Two calls of the same shape with different inputs, the second reusing
    the first's workspace: the hand-over between the chained groups of
    segments must carry the second call's totals, not the first's."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    ws = None
    for seed in (21, 22):
        wl = _diag_workload(64, "bf16", seed=seed, N=1000, Hq=3, Hkv=3)
        co = gpu_coeffs(wl, wl.group_of_dim)
        q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
        if ws is None:
            nbytes = oal.fwd_workspace_bytes_for(q, k, v, co)
            assert nbytes > 0  # two chained groups publish a total
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        y = oal.fwd(q, k, v, co, workspace=ws)
        a, b, c = oracle_coeffs(wl)
        assert rel_err(to_np(y), O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c)) <= TOL["bf16"]


def test_dimensionwise_own_keys_premap_segments():
    """The ReBased pre-map on the one-wave build over several segments."""
    _run_case(S.make(4, batch=2, n_q_heads=3, n_kv_heads=3, seq_len=777))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dimensionwise_one_segment_matches(dtype):
    """Without room for segment sums the one-pass path walks each sequence in
    one segment; outputs and state still match the oracle."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = _diag_workload(32, dtype, seed=11, N=700)
    co = gpu_coeffs(wl, wl.group_of_dim)
    q, k, v = to_dev(wl.q, dtype), to_dev(wl.k, dtype), to_dev(wl.v, dtype)
    a, b, c = oracle_coeffs(wl)
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c)
    y_seg, s_seg = oal.fwd(q, k, v, co, return_state=True)
    y_one, s_one = oal.fwd(q, k, v, co, return_state=True,
                           workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    for y in (y_seg, y_one):
        assert rel_err(to_np(y), ref) <= TOL[dtype]
    touched = diag_form_mask(32, 64)
    ref_s = np.stack([[O.abi_state_from_matrix(O.state_from_prefix(wl.k[bi, kh], wl.v[bi, kh]))
                       for kh in range(wl.n_kv_heads)] for bi in range(wl.batch)])
    scale = np.abs(ref_s).max()
    for s_ in (s_seg, s_one):
        assert np.abs(to_np(s_)[..., touched] - ref_s[..., touched]).max() <= 1e-2 * scale


@pytest.mark.parametrize("dtype,heads,N,n1", [("bf16", (4, 2), 170, 90), ("f32", (4, 2), 170, 90),
                                              ("bf16", (3, 3), 170, 90), ("bf16", (3, 3), 1000, 600)])
def test_dimensionwise_state_and_continuation(dtype, heads, N, n1):
    """Final state and continuation from it; (3, 3) at N = 1000 runs both
    halves as two chained groups of segments (the initial state enters the
    first segment's sum)."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = _diag_workload(64, dtype, seed=7, N=N, Hq=heads[0], Hkv=heads[1])
    co = gpu_coeffs(wl, wl.group_of_dim)
    assert co.diagonal
    q, k, v = to_dev(wl.q, dtype), to_dev(wl.k, dtype), to_dev(wl.v, dtype)
    sf = oal.state_floats(64, 64)
    sentinel = 7.0
    s1 = torch.full((wl.batch, wl.n_kv_heads, sf), sentinel, device="cuda")
    y1, _ = oal.fwd(q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), co,
                    return_state=True, state_out=s1)
    s2 = torch.full_like(s1, sentinel)
    y2, _ = oal.fwd(q[:, :, n1:].contiguous(), k[:, :, n1:].contiguous(), v[:, :, n1:].contiguous(), co,
                    state_in=s1, return_state=True, state_out=s2)
    a, b, c = oracle_coeffs(wl)
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c)
    assert rel_err(np.concatenate([to_np(y1), to_np(y2)], axis=2), ref) <= TOL[dtype]
    # state: the form's entries against the oracle's raw moments (bf16
    # features: unit roundoff 2^-9 per feature value; fp32: 2^-24), the rest
    # of state_out untouched
    touched = diag_form_mask(64, 64)
    u = 2.0 ** -9 if dtype == "bf16" else 2.0 ** -24
    N = wl.seq_len
    for bi in range(wl.batch):
        for kh in range(wl.n_kv_heads):
            ref_s = O.abi_state_from_matrix(O.state_from_prefix(wl.k[bi, kh], wl.v[bi, kh]))
            absum = O.abi_state_from_matrix(O.state_from_prefix(np.abs(wl.k[bi, kh]), np.abs(wl.v[bi, kh])))
            bound = (3 * u + N * 2.0 ** -24) * absum + 2.0 ** -24 * absum.max()
            got = to_np(s2)[bi, kh]
            assert (np.abs(got - ref_s)[touched] <= bound[touched]).all(), (bi, kh)
            assert (got[~touched] == sentinel).all()


def test_dimensionwise_form_rejects_two_stage_calls():
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    wl = _diag_workload(16, "bf16", seed=3, N=64)
    q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    plan = oal.PrefillPlan(q, k, v, gpu_coeffs(wl, wl.group_of_dim))
    with pytest.raises(oal.OalError) as info:
        plan.outputs()
    assert info.value.status == -2  # OAL_ERR_UNSUPPORTED
    plan.run()  # one oal_fwd call


def test_taylorshift_premap_gqa_bf16():
    """The unit-l2-norm pre-map with per-dimension gamma and beta on the
    chunk path (grouped-query heads, d_h = 64, four groups)."""
    _run_case(with_l2_premap(S.make(2, batch=2, seq_len=150), seed=51))


def test_taylorshift_premap_fp32():
    _run_case(with_l2_premap(S.make(2, batch=1, seq_len=130, dtype="f32"), seed=52))


def test_taylorshift_based_d16():
    """The TaylorShift baseline itself ([OAL] App. F.1): unit vectors, s = tau
    qhat.khat with a temperature per head, kernel 1 + s + s^2/2 (the Based
    coefficients), here at d_h = 16 (the pre-map takes the CTA build)."""
    wl = S.make(3, batch=2, n_q_heads=4, n_kv_heads=4, seq_len=333)
    _run_case(with_l2_premap(wl, seed=53, tau=[0.5, 1.0, 1.7, 3.0]))


def test_taylorshift_premap_dimensionwise():
    """The unit-l2-norm pre-map on the dimension-wise form: heads with their
    own keys (the one-launch kernel, two chained groups) and grouped-query
    heads (the small-space kernel)."""
    _run_case(with_l2_premap(S.make(4, batch=2, n_q_heads=3, n_kv_heads=3, seq_len=777), seed=54))
    _run_case(with_l2_premap(S.make(4, batch=1, n_q_heads=4, n_kv_heads=2, seq_len=150), seed=55))


def test_c4_rebased_squared_dot_premap():
    _run_case(S.make(4, batch=2, n_q_heads=2, n_kv_heads=2, seq_len=150, rebased_reading="d"))


def test_c4_rebased_squared_dot_premap_many_heads():
    # pre-map in the scan's eight-compute-wave layout: 16 (sequence, KV head)
    # pairs at d_h = 64 need more than 256 CTAs with four K-blocks per CTA
    wl = S.make(4, batch=2, n_q_heads=8, n_kv_heads=8, seq_len=140, rebased_reading="d")
    assert ((70 + 1 + 3) // 4) * wl.batch * wl.n_kv_heads > 256
    _run_case(wl)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 129])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_edge_lengths(N, dtype):
    _run_case(S.make(2, batch=2, n_q_heads=4, n_kv_heads=2, seq_len=N, dtype=dtype))


def _d32_workload(dtype="bf16"):
    # d_h = 32 variant of the outlier workload (seeded, same recipe)
    rng = np.random.default_rng(1032)
    B, Hq, Hkv, N, d, dv, G = 2, 4, 2, 150, 32, 64, 3
    q = rng.standard_normal((B, Hq, N, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, dv)).astype(np.float32)
    q[..., [5, 20]] *= 6
    k[..., [5, 20]] *= 6
    if dtype == "bf16":
        q, k, v = S.bf16_round(q), S.bf16_round(k), S.bf16_round(v)
    groups = np.tile(np.array([2 if r in (5, 20) else r % 2 for r in range(d)], np.int32), (Hq, 1))
    Ls = np.stack([np.tril(rng.uniform(0.2, 1.0, size=(G + 1, G + 1))) for _ in range(Hq)])
    return S.Workload("d32", B, Hq, Hkv, N, d, dv, dtype, q, k, v, G, groups,
                      {"kind": "factor", "eps": 1e-3, "L": Ls})


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_d32(dtype):
    _run_case(_d32_workload(dtype))


# Relative accuracy of the library's fp32 chi (non-negative terms, blocked
# fp32 sums) against the oracle's fp64 value.
CHI_RTOL = 2e-5


def _c5_groups(wl, q, k):
    """Group map of the contribution-sorted workload, taken from the oracle:
    chi by the oracle's separable form of Eq. (2), split by the oracle's
    stable sort.  The HIP path's chi, split by the library's host helper,
    must give the same map bit for bit; where two dimensions' scores sit
    closer than the fp32 accuracy of chi across a group boundary, either
    order is a correct split, and the library's map must then be a valid
    split of the oracle's scores within that accuracy (same group sizes,
    every higher group's scores >= every lower group's, up to CHI_RTOL)."""
    import grouped_quadratic_softmax_amd as oal
    bulk, tail = wl.group_budget["bulk_sizes"], wl.group_budget["n_tail"]
    _, chi_o = O.chi_separable(wl.q, wl.k)
    g_o = O.groups_sorted_split(chi_o, bulk, tail).astype(np.int32)
    chi_g = oal.contrib(q, k).cpu().numpy().astype(np.float64)
    chi_err = float(np.abs(chi_g / chi_o - 1.0).max())
    assert chi_err <= CHI_RTOL, chi_err
    g_g = oal.groups_from_contribution(chi_g, bulk, tail)
    cuts = np.cumsum(list(bulk) + [1] * tail)[:-1]
    srt = np.sort(chi_o, axis=1)
    gap = float(((srt[:, cuts] - srt[:, cuts - 1]) / srt[:, cuts]).min())
    log(f"[fwd]   chi max rel err {chi_err:.2e}; smallest relative gap at a group boundary {gap:.2e}")
    if gap > 2 * CHI_RTOL:
        assert np.array_equal(g_g, g_o)
    else:
        G = len(bulk) + tail
        for h in range(chi_o.shape[0]):
            assert np.array_equal(np.bincount(g_g[h], minlength=G), np.bincount(g_o[h], minlength=G))
            for g in range(G - 1):
                lo, hi = chi_o[h][g_g[h] == g].max(), chi_o[h][g_g[h] == g + 1].min()
                assert lo <= hi * (1 + 2 * CHI_RTOL), (h, g)
    return g_o


def test_c5_eight_groups_small():
    require_gpu()
    wl = S.make(5, n_q_heads=4, n_kv_heads=4, seq_len=260)
    groups = _c5_groups(wl, to_dev(wl.q, wl.dtype), to_dev(wl.k, wl.dtype))
    assert groups.max() == 7
    _run_case(wl, groups=groups)


@pytest.mark.parametrize("hq,hkv,dtype", [(14, 2, "bf16"), (12, 2, "bf16"), (10, 2, "bf16"), (8, 2, "bf16"),
                                          (6, 2, "bf16"), (4, 2, "bf16"), (4, 2, "f32"), (14, 2, "f32")])
def test_eight_groups_grouped_query_heads(hq, hkv, dtype):
    """Eight contribution-derived groups with several query heads per KV head:
    the readout builds with eight, four and two head slots, the ones that run
    shortest of registers, with every slot live (8, 4 and 2 query heads per
    KV head) and with dead slots (7, 6, 5 and 3)."""
    require_gpu()
    wl = S.make(5, batch=2, n_q_heads=hq, n_kv_heads=hkv, seq_len=200, dtype=dtype)
    groups = _c5_groups(wl, to_dev(wl.q, wl.dtype), to_dev(wl.k, wl.dtype))
    assert groups.max() == 7
    _run_case(wl, groups=groups)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_many_kv_heads_eight_wave_scan(dtype):
    # 16 (sequence, KV head) pairs at d_h = 64: the scan grid with four
    # K-blocks per CTA would need 18 x 16 = 288 CTAs, more than the compute
    # units, so the library takes eight K-blocks per CTA; outputs and the
    # final state must match as in the four-K-block layout
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=2, n_q_heads=16, n_kv_heads=8, seq_len=170, dtype=dtype)
    assert ((70 + 1 + 3) // 4) * wl.batch * wl.n_kv_heads > 256
    co = gpu_coeffs(wl, wl.group_of_dim)
    q, k, v = to_dev(wl.q, dtype), to_dev(wl.k, dtype), to_dev(wl.v, dtype)
    y, st = oal.fwd(q, k, v, co, return_state=True)
    a, b, c = oracle_coeffs(wl)
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c)
    err = rel_err(to_np(y), ref)
    log(f"[fwd] eight-wave scan {dtype}: max rel err {err:.3e}")
    assert err <= TOL[dtype]
    # final state: the same derived bound as the continuation test
    u = 2.0 ** -11 if dtype == "bf16" else 2.0 ** -24
    for bi in range(wl.batch):
        for kh in range(wl.n_kv_heads):
            ref_s = O.abi_state_from_matrix(O.state_from_prefix(wl.k[bi, kh], wl.v[bi, kh]))
            absum = O.abi_state_from_matrix(O.state_from_prefix(np.abs(wl.k[bi, kh]), np.abs(wl.v[bi, kh])))
            bound = (2 * u + wl.seq_len * 2.0 ** -24) * absum + 2.0 ** -24 * absum.max()
            assert (np.abs(to_np(st)[bi, kh] - ref_s) <= bound).all(), (bi, kh)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_state_out_and_continuation(dtype):
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=2, n_q_heads=4, n_kv_heads=2, seq_len=190, dtype=dtype)
    co = gpu_coeffs(wl, wl.group_of_dim)
    q, k, v = to_dev(wl.q, dtype), to_dev(wl.k, dtype), to_dev(wl.v, dtype)
    n1 = 100
    y_full, s_full = oal.fwd(q, k, v, co, return_state=True)
    y1, s1 = oal.fwd(q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), co,
                     return_state=True)
    y2, s2 = oal.fwd(q[:, :, n1:].contiguous(), k[:, :, n1:].contiguous(), v[:, :, n1:].contiguous(), co,
                     state_in=s1, return_state=True)
    y_cat = np.concatenate([to_np(y1), to_np(y2)], axis=2)
    a, b, c = oracle_coeffs(wl)
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c)
    assert rel_err(y_cat, ref) <= TOL[dtype]
    assert rel_err(to_np(y_full), ref) <= TOL[dtype]
    # final state against the oracle's raw Eq. (5) moments.  Error bound of
    # the update arithmetic: every feature product k_r k_t is rounded once
    # (fp16 for bf16 inputs, unit roundoff u = 2^-11; fp32 for fp32 inputs,
    # u = 2^-24) and the sums accumulate in fp32, so per entry
    #   |got - ref| <= (2u + N 2^-24) * sum_j |phi_f(k_j)| |u_jl|
    # where the right-hand sum is the oracle's own state of |K| and |V|; a
    # floor of 2^-24 of its maximum covers fp16 values that underflow.
    D = O.feature_count(wl.d_h)
    u = 2.0 ** -11 if dtype == "bf16" else 2.0 ** -24
    N = wl.seq_len
    for bi in range(wl.batch):
        for kh in range(wl.n_kv_heads):
            ref_s = O.abi_state_from_matrix(O.state_from_prefix(wl.k[bi, kh], wl.v[bi, kh]))
            absum = O.abi_state_from_matrix(O.state_from_prefix(np.abs(wl.k[bi, kh]), np.abs(wl.v[bi, kh])))
            bound = (2 * u + N * 2.0 ** -24) * absum + 2.0 ** -24 * absum.max()
            for got in (to_np(s_full)[bi, kh], to_np(s2)[bi, kh]):
                assert (np.abs(got - ref_s) <= bound).all(), (bi, kh)
    assert to_np(s_full).shape[-1] == D * 65


@pytest.mark.parametrize("dtype,heads", [("bf16", (4, 2)), ("f32", (4, 2)), ("bf16", (4, 4)), ("f32", (4, 4))])
def test_d16_workspace_sizes_stages_and_state(dtype, heads):
    """d_h = 16 full space: oal_fwd with its default workspace and with a
    minimal one (refused by the chunk path, fewer segments on a one-pass
    path) and the two-stage calls all match the oracle; the final state
    matches Eq. (5) and carries a continuation across a ragged split.  With
    four query heads on two KV heads the bf16 prefill is the one-pass CTA
    build; with a KV head per query head it is the one-wave-per-segment
    build, here over eight segments of three chunks."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(3, batch=2, n_q_heads=heads[0], n_kv_heads=heads[1], seq_len=1500, dtype=dtype)
    co = gpu_coeffs(wl, wl.group_of_dim)
    q, k, v = to_dev(wl.q, dtype), to_dev(wl.k, dtype), to_dev(wl.v, dtype)
    a, b, c = oracle_coeffs(wl)
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c)
    y_seg, s_seg = oal.fwd(q, k, v, co, return_state=True)
    tiny = torch.empty(1, dtype=torch.uint8, device="cuda")
    try:
        y_one, s_one = oal.fwd(q, k, v, co, return_state=True, workspace=tiny)
    except oal.OalError as e:
        assert e.status == -3  # OAL_ERR_WORKSPACE
        y_one, s_one = y_seg, s_seg
    plan = oal.PrefillPlan(q, k, v, co)
    plan.states()
    plan.outputs()
    torch.cuda.synchronize()
    for name, y in (("segments", y_seg), ("one segment", y_one), ("two stages", plan.y)):
        err = rel_err(to_np(y), ref)
        log(f"[fwd]   small path {name}: max rel err {err:.3e}")
        assert err <= TOL[dtype], name
    n1 = 700
    y1, s1 = oal.fwd(q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous(), co,
                     return_state=True)
    y2, s2 = oal.fwd(q[:, :, n1:].contiguous(), k[:, :, n1:].contiguous(), v[:, :, n1:].contiguous(), co,
                     state_in=s1, return_state=True)
    assert rel_err(np.concatenate([to_np(y1), to_np(y2)], axis=2), ref) <= TOL[dtype]
    # state bound as in the chunk path's test, with bf16 feature values
    # (u = 2^-9) in place of fp16 ones
    u = 2.0 ** -9 if dtype == "bf16" else 2.0 ** -24
    N = wl.seq_len
    for bi in range(wl.batch):
        for kh in range(wl.n_kv_heads):
            ref_s = O.abi_state_from_matrix(O.state_from_prefix(wl.k[bi, kh], wl.v[bi, kh]))
            absum = O.abi_state_from_matrix(O.state_from_prefix(np.abs(wl.k[bi, kh]), np.abs(wl.v[bi, kh])))
            bound = (2 * u + N * 2.0 ** -24) * absum + 2.0 ** -24 * absum.max()
            for got in (s_seg, s_one, s2, plan.state_out):
                assert (np.abs(to_np(got)[bi, kh] - ref_s) <= bound).all(), (bi, kh)


@pytest.mark.parametrize("G,N", [(16, 777), (16, 64), (12, 130), (9, 1500)])
def test_d16_dimension_aware_general_c(G, N):
    """The dimension-aware kernel with a general symmetric C ([Slides]
    "Relax sharing ...", Eq. (3): b_r and C_rt per dimension), here G = 16 =
    d_h singleton groups in a random order, and 9-12 uneven groups: more
    than eight groups take the within-chunk scores in the packed feature
    space (the one-wave build, heads with their own keys).  C = M[1:, 1:] of
    a PSD M = L L^T ([OAL] Eq. (7)), so every weight is positive."""
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    rng = np.random.default_rng(1600 + G + N)
    wl = S.make(3, batch=2, n_q_heads=3, n_kv_heads=3, seq_len=N)
    groups = np.stack([rng.permutation(np.arange(16) % G) for _ in range(3)]).astype(np.int32)
    a, b, c = O.coeffs_from_factor(1e-3, rng.standard_normal((3, G + 1, G + 1)) * 0.5)
    co = oal.Coeffs(groups, a.astype(np.float32), b.astype(np.float32), c.astype(np.float32))
    q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    y, st = oal.fwd(q, k, v, co, return_state=True)
    ref = O.attention_direct(wl.q, wl.k, wl.v, groups, a, b, c)
    err = rel_err(to_np(y), ref)
    log(f"[fwd]   d16 dimension-aware G={G} N={N}: max rel err {err:.3e}")
    assert err <= TOL["bf16"]
    u = 2.0 ** -9
    for bi in range(wl.batch):
        for kh in range(wl.n_kv_heads):
            ref_s = O.abi_state_from_matrix(O.state_from_prefix(wl.k[bi, kh], wl.v[bi, kh]))
            absum = O.abi_state_from_matrix(O.state_from_prefix(np.abs(wl.k[bi, kh]), np.abs(wl.v[bi, kh])))
            bound = (2 * u + N * 2.0 ** -24) * absum + 2.0 ** -24 * absum.max()
            assert (np.abs(to_np(st)[bi, kh] - ref_s) <= bound).all(), (bi, kh)


def test_d16_chained_back_to_back():
    """d_h = 16, a KV head per query head, two chained groups of segments:
    two calls with different inputs on one workspace, each against the
    oracle (the second must not take the first call's hand-over)."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    ws = None
    for seed in (31, 32):
        wl = S.make(3, batch=2, n_q_heads=3, n_kv_heads=3, seq_len=1500, seed=seed)
        co = gpu_coeffs(wl, wl.group_of_dim)
        q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
        if ws is None:
            nbytes = oal.fwd_workspace_bytes_for(q, k, v, co)
            assert nbytes > 0
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        y = oal.fwd(q, k, v, co, workspace=ws)
        a, b, c = oracle_coeffs(wl)
        assert rel_err(to_np(y), O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c)) <= TOL["bf16"]


@pytest.mark.parametrize("G,N", [(2, 777), (3, 130), (5, 64), (8, 1000)])
def test_d16_heads_with_own_keys_grouped(G, N):
    """The one-wave-per-segment build at d_h = 16 (as many query heads as KV
    heads) with several groups of uneven size: every row against the
    oracle, and the final state against Eq. (5)."""
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    rng = np.random.default_rng(160 + G)
    wl = S.make(3, batch=2, n_q_heads=3, n_kv_heads=3, seq_len=N)
    groups = np.stack([rng.permutation(np.arange(16) % G) for _ in range(3)]).astype(np.int32)
    a, b, c = O.coeffs_from_factor(1e-3, rng.standard_normal((3, G + 1, G + 1)) * 0.5)
    co = oal.Coeffs(groups, a.astype(np.float32), b.astype(np.float32), c.astype(np.float32))
    q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    y, st = oal.fwd(q, k, v, co, return_state=True)
    ref = O.attention_direct(wl.q, wl.k, wl.v, groups, a, b, c)
    err = rel_err(to_np(y), ref)
    log(f"[fwd]   d16 own-keys G={G} N={N}: max rel err {err:.3e}")
    assert err <= TOL["bf16"]
    u = 2.0 ** -9
    for bi in range(wl.batch):
        for kh in range(wl.n_kv_heads):
            ref_s = O.abi_state_from_matrix(O.state_from_prefix(wl.k[bi, kh], wl.v[bi, kh]))
            absum = O.abi_state_from_matrix(O.state_from_prefix(np.abs(wl.k[bi, kh]), np.abs(wl.v[bi, kh])))
            bound = (2 * u + N * 2.0 ** -24) * absum + 2.0 ** -24 * absum.max()
            assert (np.abs(to_np(st)[bi, kh] - ref_s) <= bound).all(), (bi, kh)


def test_zero_length_passes_state_through():
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=2, n_q_heads=4, n_kv_heads=2, seq_len=70)
    co = gpu_coeffs(wl, wl.group_of_dim)
    q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    _, s = oal.fwd(q, k, v, co, return_state=True)
    e = lambda t: t[:, :, :0].contiguous()
    _, s0 = oal.fwd(e(q), e(k), e(v), co, state_in=s, return_state=True)
    assert torch.equal(s0, s)
    _, z = oal.fwd(e(q), e(k), e(v), co, return_state=True)
    assert float(z.abs().max()) == 0.0


# ------------------------------------------------------------- full sizes

def test_c2_full_size_sampled():
    wl = S.make(2)
    _run_case(wl, rows=sample_rows(wl.seq_len, 64, 64, seed=2))


def test_c3_full_size_sampled():
    """Based workload at full size: a seeded sample of rows over every
    (sequence, head), plus the first and last row of every 64-token chunk of
    one (sequence, head)."""
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(3)
    q, k, v = to_dev(wl.q, wl.dtype), to_dev(wl.k, wl.dtype), to_dev(wl.v, wl.dtype)
    y = to_np(oal.fwd(q, k, v, gpu_coeffs(wl, wl.group_of_dim)))
    a, b, c = oracle_coeffs(wl)
    rows = sample_rows(wl.seq_len, 512, 48, seed=3)
    err = rel_err(y[:, :, rows], O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c, rows=rows))
    bi, h = 5, 11
    edge = sample_rows(wl.seq_len, 64, 0, seed=0)
    sl = lambda x: x[bi:bi + 1, h:h + 1]
    err_e = rel_err(y[bi, h, edge], O.attention_direct(sl(wl.q), sl(wl.k), sl(wl.v), wl.group_of_dim[h:h + 1],
                                                       a[h:h + 1], b[h:h + 1], c[h:h + 1], rows=edge)[0, 0])
    log(f"[fwd] c3 full size: sampled rows {err:.3e}, every chunk edge of (b={bi}, h={h}) {err_e:.3e}")
    assert np.isfinite(y).all()
    assert max(err, err_e) <= TOL["bf16"]


def test_c4_full_size_sampled():
    # ReBased elementwise workload at full size (dimension-wise form, one
    # fused launch as the benchmark runs it)
    wl = S.make(4)
    _run_case(wl, rows=sample_rows(wl.seq_len, 512, 16, seed=4))


def test_c5_full_size_sampled():
    """Long-context workload at full size with the oracle's group map: random
    rows over every head, plus the first and last row of every 64-token chunk
    of one head."""
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(5)
    q, k, v = to_dev(wl.q, wl.dtype), to_dev(wl.k, wl.dtype), to_dev(wl.v, wl.dtype)
    groups = _c5_groups(wl, q, k)
    y = to_np(oal.fwd(q, k, v, gpu_coeffs(wl, groups)))
    a, b, c = oracle_coeffs(wl)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, wl.seq_len, 40), [0, 63, 64, 4095, 4096, wl.seq_len - 1]]))
    err = rel_err(y[:, :, rows], O.attention_direct(wl.q, wl.k, wl.v, groups, a, b, c, rows=rows))
    h = 9
    edge = sample_rows(wl.seq_len, 64, 0, seed=0)
    sl = lambda x: x[:, h:h + 1]
    err_e = rel_err(y[0, h, edge], O.attention_direct(sl(wl.q), sl(wl.k), sl(wl.v), groups[h:h + 1], a[h:h + 1],
                                                      b[h:h + 1], c[h:h + 1], rows=edge)[0, 0])
    log(f"[fwd] c5 full size: sampled rows {err:.3e}, every chunk edge of head {h} {err_e:.3e}")
    assert np.isfinite(y).all()
    assert max(err, err_e) <= TOL["bf16"]


def test_stages_compose_to_fwd_bitwise():
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=2, n_q_heads=14, n_kv_heads=2, seq_len=250)
    co = gpu_coeffs(wl, wl.group_of_dim)
    q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    y, st = oal.fwd(q, k, v, co, return_state=True)
    plan = oal.PrefillPlan(q, k, v, co)
    plan.states()
    plan.outputs()
    torch.cuda.synchronize()
    assert torch.equal(plan.y, y) and torch.equal(plan.state_out, st)


def test_stages_compose_with_initial_state():
    """The two stages given an initial state: the first chunk of the outputs
    stage must read it (it is not re-read, only whether it exists), so that
    states() + outputs() equals one fwd call bit for bit and continues a
    split sequence as the oracle's direct Eq. (6) does."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=2, n_q_heads=4, n_kv_heads=2, seq_len=230)
    co = gpu_coeffs(wl, wl.group_of_dim)
    q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    n1 = 90
    head = [t[:, :, :n1].contiguous() for t in (q, k, v)]
    tail = [t[:, :, n1:].contiguous() for t in (q, k, v)]
    y1, s1 = oal.fwd(*head, co, return_state=True)
    y2, s2 = oal.fwd(*tail, co, state_in=s1, return_state=True)
    plan = oal.PrefillPlan(*tail, co, state_in=s1)
    plan.states()
    plan.outputs()
    torch.cuda.synchronize()
    assert torch.equal(plan.y, y2) and torch.equal(plan.state_out, s2)
    a, b, c = oracle_coeffs(wl)
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c)
    got = np.concatenate([to_np(y1), to_np(plan.y)], axis=2)
    assert rel_err(got, ref) <= TOL["bf16"]
