"""Prefill of sequences of different lengths in the padded layout
(oal_fwd_varlen) against the oracle on each sequence's own prefix: outputs
below each length, untouched rows above it, the final states (continuing
from an initial state where given), and empty sequences.  Prompts of
different lengths are [OAL] sec. 3.1, Eq. (2)'s N_p."""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import (TOL, diag_form_mask, gpu_coeffs, gpu_prep, log, oracle_coeffs, oracle_prep, rel_err,
                     require_gpu, to_dev, to_np)

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _varlen_case(wl, lens, groups=None, with_state_in=False, diagonal_state=False):
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    groups = wl.group_of_dim if groups is None else groups
    lens = np.asarray(lens, np.int32)
    B, Hq, N, d = wl.q.shape
    Hkv = wl.n_kv_heads
    log(f"[varlen] {wl.name} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {wl.dtype} lens={lens.tolist()}")
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q, k, v = to_dev(wl.q, wl.dtype), to_dev(wl.k, wl.dtype), to_dev(wl.v, wl.dtype)
    co = gpu_coeffs(wl, groups)
    a, b, c = oracle_coeffs(wl)
    sf = oal.state_floats(d, 64)
    # an initial state: the oracle's state of a random prefix of P tokens
    P = 37
    rng = np.random.default_rng(70 + N)
    kp = rng.standard_normal((B, Hkv, P, d)) * np.std(wl.k)
    vp = rng.standard_normal((B, Hkv, P, 64))
    if wl.dtype == "bf16":
        kp, vp = S.bf16_round(kp), S.bf16_round(vp)
    sin = None
    if with_state_in:
        kp_m = kp
        if wl.premap is not None:
            p = oracle_prep(wl)
            kp_m = np.stack([[O.premap(kp[bi, kh], p["gamma_k"][kh], p["beta_k"][kh], p["ln_eps"],
                                       p.get("kind", "layernorm")) for kh in range(Hkv)] for bi in range(B)])
        s0 = np.stack([[O.abi_state_from_matrix(O.state_from_prefix(kp_m[bi, kh], vp[bi, kh]))
                        for kh in range(Hkv)] for bi in range(B)])
        sin = torch.from_numpy(s0.astype(np.float32)).cuda()
    y = torch.full((B, Hq, N, 64), SENTINEL, dtype=dt, device="cuda")
    st = torch.full((B, Hkv, sf), SENTINEL, dtype=torch.float32, device="cuda")
    oal.fwd(q, k, v, co, gpu_prep(wl), state_in=sin, y=y, state_out=st, seq_lens=torch.from_numpy(lens).cuda())
    y, st = to_np(y), to_np(st)
    touched = diag_form_mask(d, 64) if diagonal_state else np.ones(sf, bool)
    u = 2.0 ** -9 if wl.dtype == "bf16" else 2.0 ** -24
    for bi, n in enumerate(lens):
        n = int(min(max(n, 0), N))
        assert (y[bi, :, n:] == SENTINEL).all(), (bi, "rows past the length were written")
        sl = slice(bi, bi + 1)
        Pn = P if with_state_in else 0
        qs = np.concatenate([np.zeros((1, Hq, Pn, d)), wl.q[sl, :, :n]], axis=2)
        ks = np.concatenate([kp[sl][:, :, :Pn], wl.k[sl, :, :n]], axis=2)
        vs = np.concatenate([vp[sl][:, :, :Pn], wl.v[sl, :, :n]], axis=2)
        if n > 0:
            ref = O.attention_direct(qs, ks, vs, groups, a, b, c, oracle_prep(wl), rows=np.arange(Pn, Pn + n))
            err = rel_err(y[sl, :, :n], ref)
            log(f"[varlen]   b={bi} n={n}: max rel err {err:.3e}")
            assert err <= TOL[wl.dtype], (bi, n, err)
        p = oracle_prep(wl)
        for kh in range(Hkv):
            kk = ks[0, kh]
            if p is not None:
                kk = O.premap(kk, p["gamma_k"][kh], p["beta_k"][kh], p["ln_eps"], p.get("kind", "layernorm"))
            ref_s = O.abi_state_from_matrix(O.state_from_prefix(kk, vs[0, kh]))
            absum = O.abi_state_from_matrix(O.state_from_prefix(np.abs(kk), np.abs(vs[0, kh])))
            bound = (2 * u + (Pn + n) * 2.0 ** -24) * absum + 2.0 ** -24 * max(absum.max(), 1.0)
            got = st[bi, kh]
            assert (np.abs(got - ref_s)[touched] <= bound[touched]).all(), (bi, kh, n)
            assert (got[~touched] == SENTINEL).all()


def test_varlen_d16_own_keys():
    """d_h = 16 bf16, a KV head per query head: the one-launch chained build
    (two groups of segments), lengths from full to empty."""
    _varlen_case(S.make(3, batch=4, n_q_heads=3, n_kv_heads=3, seq_len=1500), [1500, 777, 0, 65])


def test_varlen_d16_own_keys_with_initial_state():
    _varlen_case(S.make(3, batch=3, n_q_heads=3, n_kv_heads=3, seq_len=1000), [900, 0, 401], with_state_in=True)


def test_varlen_d16_grouped_query_heads():
    """d_h = 16 with grouped-query heads: the chunk path."""
    _varlen_case(S.make(3, batch=3, n_q_heads=4, n_kv_heads=2, seq_len=300), [300, 129, 1])


def test_varlen_chunk_path_gqa():
    """d_h = 64, four groups, seven query heads per KV head: the chunk path
    (chunks past a sequence's end skipped by the readout)."""
    _varlen_case(S.make(2, batch=3, seq_len=300), [300, 64, 0], with_state_in=True)


def test_varlen_chunk_path_fp32():
    _varlen_case(S.make(2, batch=2, seq_len=130, dtype="f32"), [130, 50])


def test_varlen_dimensionwise_premap():
    """The ReBased dimension-wise form with its pre-map, heads with their own
    keys: the one-launch kernel."""
    _varlen_case(S.make(4, batch=3, n_q_heads=3, n_kv_heads=3, seq_len=777), [777, 300, 31],
                 diagonal_state=True)


def test_varlen_rejects_grouped_dimensionwise_and_null_lengths():
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(4, batch=2, n_q_heads=4, n_kv_heads=2, seq_len=64)
    q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    lens = torch.tensor([64, 10], dtype=torch.int32, device="cuda")
    with pytest.raises(oal.OalError) as info:
        oal.fwd(q, k, v, gpu_coeffs(wl, wl.group_of_dim), gpu_prep(wl), seq_lens=lens)
    assert info.value.status == -2  # OAL_ERR_UNSUPPORTED
