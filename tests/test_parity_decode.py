"""GPU parity of oal_decode_step against the fp64 oracle."""

import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import (TOL, diag_form_mask, gpu_coeffs, gpu_prep, log, oracle_coeffs, oracle_prep, rel_err,
                     require_gpu, to_dev, to_np, with_l2_premap)

pytestmark = pytest.mark.gpu


def _oracle_states(wl, lengths):
    """Packed fp64 states of each (sequence, KV head) over its seeded prefix."""
    prep = oracle_prep(wl)
    st = np.zeros((wl.batch, wl.n_kv_heads, O.feature_count(wl.d_h), wl.d_v + 1))
    for s in range(wl.batch):
        n = int(lengths[s])
        for kh in range(wl.n_kv_heads):
            pk = None if prep is None else (prep["gamma_k"][kh], prep["beta_k"][kh])
            st[s, kh] = O.state_from_prefix(wl.k[s, kh, :n], wl.v[s, kh, :n], pk,
                                            1e-5 if prep is None else prep["ln_eps"])
    return st


def _decode_case(wl, lengths, groups=None, tol=None):
    """Prefix of length lengths[s] builds the state; token lengths[s] is decoded."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    groups = wl.group_of_dim if groups is None else groups
    log(f"[decode] {wl.name} S={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} d={wl.d_h} G={wl.n_groups} "
        f"{wl.dtype}")
    st64 = _oracle_states(wl, lengths)
    idx = np.asarray(lengths)
    sel = lambda x: np.stack([x[s, :, idx[s]] for s in range(wl.batch)])
    qn, kn, vn = sel(wl.q), sel(wl.k), sel(wl.v)
    a, b, c = oracle_coeffs(wl)
    st32 = st64.astype(np.float32).astype(np.float64)  # the library state is float32
    y_ref, st_ref = O.decode_step(st32, qn, kn, vn, groups, a, b, c, wl.n_q_heads, oracle_prep(wl))
    state = torch.from_numpy(O.abi_state_from_matrix(st32).astype(np.float32)).cuda().contiguous()
    co = gpu_coeffs(wl, groups)
    state0 = to_np(state)
    y = oal.decode_step(to_dev(qn, wl.dtype), to_dev(kn, wl.dtype), to_dev(vn, wl.dtype), co, state,
                        gpu_prep(wl))
    err = rel_err(to_np(y), y_ref)
    log(f"[decode]   max rel err {err:.3e} (dimension-wise form: {co.diagonal})")
    assert err <= (tol or TOL[wl.dtype])
    got_state = to_np(state)
    ref_state = O.abi_state_from_matrix(st_ref)
    scale = np.abs(ref_state).max(axis=-1, keepdims=True)
    close = np.abs(got_state - ref_state) <= 1e-6 * scale + 1e-30
    if co.diagonal:
        # only the constant, linear and squared entries are updated; the
        # other entries of the state are left as they were
        touched = diag_form_mask(wl.d_h, wl.d_v)
        assert close[..., touched].all()
        assert (got_state[..., ~touched] == state0[..., ~touched]).all()
    else:
        assert close.all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_gqa_small(dtype):
    wl = S.make(2, batch=6, n_q_heads=4, n_kv_heads=2, seq_len=48, dtype=dtype)
    lengths = np.random.default_rng(0).integers(1, 47, size=6)
    _decode_case(wl, lengths)


def test_decode_gqa_seven_heads():
    wl = S.make(2, batch=3, seq_len=30)
    _decode_case(wl, np.array([0, 7, 29]))


def test_decode_d16_taylor():
    wl = S.make(3, batch=4, n_q_heads=3, n_kv_heads=3, seq_len=40)
    _decode_case(wl, np.array([0, 1, 20, 39]))


@pytest.mark.parametrize("reading", ["d", "e"])
def test_decode_rebased_premap(reading):
    wl = S.make(4, batch=3, n_q_heads=2, n_kv_heads=2, seq_len=25, rebased_reading=reading)
    _decode_case(wl, np.array([3, 10, 24]))


def test_decode_taylorshift_premap():
    wl = with_l2_premap(S.make(2, batch=3, n_q_heads=4, n_kv_heads=2, seq_len=25), seed=56)
    _decode_case(wl, np.array([3, 10, 24]))


def test_decode_dimension_aware_general_c():
    """d_h = 16, one group per dimension with a general symmetric C."""
    rng = np.random.default_rng(1616)
    wl = S.make(3, batch=3, n_q_heads=2, n_kv_heads=2, seq_len=30)
    groups = np.stack([rng.permutation(16) for _ in range(2)]).astype(np.int32)
    a, b, c = O.coeffs_from_factor(1e-3, rng.standard_normal((2, 17, 17)) * 0.5)
    wl.coeff = {"kind": "abc", "a": a, "b": b, "c": c}
    wl.n_groups = 16
    _decode_case(wl, np.array([0, 11, 29]), groups=groups)


def test_decode_eight_groups():
    wl = S.make(5, n_q_heads=4, n_kv_heads=4, seq_len=33, batch=3)
    groups = np.stack([np.arange(64) % 8 for _ in range(4)]).astype(np.int32)
    _decode_case(wl, np.array([5, 17, 32]), groups=groups)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_then_decode_matches_longer_prefill(dtype):
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=2, n_q_heads=4, n_kv_heads=2, seq_len=131, dtype=dtype)
    co = gpu_coeffs(wl, wl.group_of_dim)
    q, k, v = to_dev(wl.q, dtype), to_dev(wl.k, dtype), to_dev(wl.v, dtype)
    n = 130
    _, st = oal.fwd(q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous(), co,
                    return_state=True)
    yd = oal.decode_step(q[:, :, n].contiguous(), k[:, :, n].contiguous(), v[:, :, n].contiguous(), co, st)
    a, b, c = oracle_coeffs(wl)
    ref = O.attention_direct(wl.q, wl.k, wl.v, wl.group_of_dim, a, b, c, rows=np.array([n]))[:, :, 0]
    assert rel_err(to_np(yd), ref) <= TOL[dtype]


def test_c5_decode_full_batch():
    """256 sequences x 16 heads, fp32 states: the benchmark's decode launch.

    States of 16 seeded prefixes (lengths in [1, 512]) are built by the oracle
    and tiled over the 256 sequences; each sequence decodes its own token."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    n_seq, H, d = 256, 16, 64
    base = S.make(5, n_q_heads=H, n_kv_heads=H, seq_len=513, batch=16)
    lengths = S.decode_prefix_lengths(16)
    groups = np.stack([(np.arange(d) * 8) // d for _ in range(H)]).astype(np.int32)
    st16 = _oracle_states(base, lengths).astype(np.float32).astype(np.float64)
    tile = np.arange(n_seq) % 16
    st = st16[tile]
    rng = np.random.default_rng(1205)
    qn = S.bf16_round(rng.standard_normal((n_seq, H, d)).astype(np.float32))
    kn = S.bf16_round(rng.standard_normal((n_seq, H, d)).astype(np.float32))
    vn = S.bf16_round(rng.standard_normal((n_seq, H, 64)).astype(np.float32))
    a, b, c = oracle_coeffs(base)
    log("[decode] c5 full batch 256 x 16")
    y_ref, _ = O.decode_step(st, qn, kn, vn, groups, a, b, c, H)
    state = torch.from_numpy(O.abi_state_from_matrix(st).astype(np.float32)).cuda().contiguous()
    y = oal.decode_step(to_dev(qn, "bf16"), to_dev(kn, "bf16"), to_dev(vn, "bf16"),
                        gpu_coeffs(base, groups), state)
    err = rel_err(to_np(y), y_ref)
    log(f"[decode]   max rel err {err:.3e}")
    assert err <= TOL["bf16"]
