"""Backward pass (oal_bwd) against the oracle's fp64 gradients
(oracle.attention_backward, pinned by finite differences of the forward
definition): dq, dk, dv and the coefficient gradients da, db, dc that the
output-matching calibration ([OAL] App. B, Eq. (20)) and the joint adaptation
of the coefficients ([OAL] App. F.2) take.

Both sides see the same inputs (bf16 inputs are bf16-exact values), so the
error is the library's fp32 arithmetic alone, and every element is held to
the recursive-summation bound
    |got - ref| <= n u cond M,   n = 2 N + 300,  u = 2^-24,
with M the element's absolute-value majorant (the same sums over |terms|:
|kappa| -> kappa_abs = |a| + sum |b_g| |s|_g + sum |c_gh| |s|_g |s|_h with
|s| the group scores of |q|, |k|; dkappa_ij -> |g_i| . |u_j| with
g_i = [dy_i, -(dy_i . y_i)] / den_i and u_j = [v_j, 1]) and cond =
max_i sum_j kappa_abs_ij / den_i the conditioning of the denominators, all in
fp64 from the oracle's forward quantities.  The coefficient gradients need
this form: they cancel by construction (y is unchanged when (a, b, c) are
scaled together, so a da + b . db + c . dc = 0) and are typically 1e-4 ..
1e-3 of their majorants.  The same bound checks that scaling identity on
the library's own outputs.  On top of it every gradient tensor meets the
fp32 parity bar of the forward pass, max |err| <= 2e-3 max |ref| (the
measured errors are below 1e-5 of max |ref|, also at the full 8192-token
size; a dropped term or a wrong sign moves a result by O(1) of itself),
except where a closed form makes the reference zero (N = 1: y = v).
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import log, require_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24
REL_BAR = 2e-3  # the fp32 parity bar


def _draw(rng, shape, dtype, std=1.0):
    x = rng.standard_normal(shape) * std
    return (S.bf16_round(x) if dtype == "bf16" else x.astype(np.float32)).astype(np.float64)


def _coeffs(rng, H, G):
    """a, b, c from a PSD factor ([OAL] Eq. (7): every weight positive) with
    a small antisymmetric part added to c (it leaves the kernel unchanged;
    every ordered entry is still its own parameter)."""
    a, b, c = O.coeffs_from_factor(1e-3, rng.standard_normal((H, G + 1, G + 1)) * 0.5)
    e = 0.05 * rng.standard_normal(c.shape)
    c = c + (e - np.swapaxes(e, 1, 2))
    return (a.astype(np.float32).astype(np.float64), b.astype(np.float32).astype(np.float64),
            c.astype(np.float32).astype(np.float64))


def _majorants(q, k, v, dy, groups, a, b, c):
    """fp64 absolute-value majorants of every gradient (dq, dk, dv in their
    shapes; da [H], db [H, G], dc [H, G, G] summed over the batch) and the
    conditioning of the denominators."""
    B, H, N, d = q.shape
    G = b.shape[1]
    Mq, Mk, Mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    Ma, Mb, Mc = np.zeros(H), np.zeros((H, G)), np.zeros((H, G, G))
    cond = 1.0
    causal = np.tril(np.ones((N, N)))
    for bi in range(B):
        for h in range(H):
            qa, ka = np.abs(q[bi, h]), np.abs(k[bi, h])
            gd = np.asarray(groups[h])
            s = O.group_scores(q[bi, h], k[bi, h], gd, G)
            sa = O.group_scores(qa, ka, gd, G)
            w = O.kappa_from_scores(s, a[h], b[h], c[h]) * causal
            kabs = O.kappa_from_scores(sa, abs(a[h]), np.abs(b[h]), np.abs(c[h])) * causal
            den = w.sum(axis=1)
            cond = max(cond, float((kabs.sum(axis=1) / den).max()))
            y = (w @ v[bi, h]) / den[:, None]
            ga = np.concatenate([np.abs(dy[bi, h]), np.abs((dy[bi, h] * y).sum(1))[:, None]], 1) / den[:, None]
            ua = np.concatenate([np.abs(v[bi, h]), np.ones((N, 1))], 1)
            A = (ga @ ua.T) * causal
            Mv[bi, h] = kabs.T @ (np.abs(dy[bi, h]) / den[:, None])
            cs = np.abs(c[h] + c[h].T)
            for g in range(G):
                Bg = abs(b[h][g]) + sum(cs[g, hh] * sa[hh] for hh in range(G))  # |d kappa / d s_g|
                ABg = A * Bg
                for r in np.nonzero(gd == g)[0]:
                    Mq[bi, h][:, r] = ABg @ ka[:, r] / np.sqrt(d)
                    Mk[bi, h][:, r] = ABg.T @ qa[:, r] / np.sqrt(d)
            Ma[h] += A.sum()
            for g in range(G):
                Asg = A * sa[g]
                Mb[h, g] += Asg.sum()
                for hh in range(G):
                    Mc[h, g, hh] += (Asg * sa[hh]).sum()
    return (Mq, Mk, Mv, Ma, Mb, Mc), cond


def _run_gpu(q, k, v, dy, groups, a, b, c, dtype):
    import grouped_quadratic_softmax_amd as oal
    co = oal.Coeffs(groups, a.astype(np.float32), b.astype(np.float32), c.astype(np.float32))
    out = oal.bwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to_dev(dy, dtype), co)
    return [to_np(t) for t in out]


NAMES = ("dq", "dk", "dv", "da", "db", "dc")


def _check(got, ref, maj, N, tag, coef=None, names=NAMES):
    Ms, cond = maj
    tau = (2 * N + 300) * U32 * cond
    for name, x, r, M in zip(names, got, ref, Ms):
        ratio = float((np.abs(x - r) / np.maximum(M, 1e-300)).max())
        rel = float(np.abs(x - r).max() / max(np.abs(r).max(), 1e-300))
        log(f"[bwd]   {tag} {name}: max |err| / majorant {ratio:.3e} (bound {tau:.3e}), "
            f"max |err| / max |ref| {rel:.3e}")
        assert ratio <= tau, (name, ratio, tau)
        if N > 1:
            assert rel <= REL_BAR, (name, rel)
    if coef is not None:  # scaling identity on the library's own outputs
        a, b, c = coef
        da, db, dc = got[3], got[4], got[5]
        Ma, Mb, Mc = Ms[3], Ms[4], Ms[5]
        lhs = a * da + (b * db).sum(1) + (c * dc).sum((1, 2))
        bound = tau * (np.abs(a) * Ma + (np.abs(b) * Mb).sum(1) + (np.abs(c) * Mc).sum((1, 2)))
        log(f"[bwd]   {tag} a.da + b.db + c.dc: max {float(np.abs(lhs).max()):.3e} (bound {float(bound.min()):.3e})")
        assert (np.abs(lhs) <= bound).all()


CASES = [  # (B, H, N, G, dtype)
    (2, 3, 200, 1, "bf16"),
    (1, 2, 130, 4, "f32"),
    (2, 2, 65, 16, "bf16"),
    (1, 3, 64, 3, "f32"),
    (1, 2, 300, 16, "f32"),
    (3, 2, 1, 4, "bf16"),
    (1, 1, 127, 9, "bf16"),
]


@pytest.mark.parametrize("B,H,N,G,dtype", CASES)
def test_bwd_matches_oracle(B, H, N, G, dtype):
    """Several 64-token chunks with a ragged tail, single chunks, N = 1 (y = v:
    only dv is nonzero), G = 1 .. 16 uneven groups in random orders, both
    activation types."""
    require_gpu()
    rng = np.random.default_rng(2000 + 7 * N + G)
    log(f"[bwd] B={B} H={H} N={N} G={G} {dtype}")
    q, k = _draw(rng, (B, H, N, 16), dtype), _draw(rng, (B, H, N, 16), dtype)
    v, dy = _draw(rng, (B, H, N, 64), dtype), _draw(rng, (B, H, N, 64), dtype)
    groups = np.stack([rng.permutation(np.arange(16) % G) for _ in range(H)]).astype(np.int32)
    a, b, c = _coeffs(rng, H, G)
    got = _run_gpu(q, k, v, dy, groups, a, b, c, dtype)
    ref = O.attention_backward(q, k, v, dy, groups, a, b, c)
    _check(got, ref, _majorants(q, k, v, dy, groups, a, b, c), N, f"G={G} N={N} {dtype}", coef=(a, b, c))


def test_bwd_based_workload():
    """The Based Taylor workload's recipe (d_h = 16 projections of std 0.25,
    one group, a = 1, b = 1, c = 1/2) at a small size."""
    require_gpu()
    wl = S.make(3, batch=2, n_q_heads=3, n_kv_heads=3, seq_len=256)
    rng = np.random.default_rng(2101)
    dy = _draw(rng, wl.v.shape, "bf16")
    q, k, v = (x.astype(np.float64) for x in (wl.q, wl.k, wl.v))
    a = np.asarray(wl.coeff["a"], np.float64)
    b = np.asarray(wl.coeff["b"], np.float64)
    c = np.asarray(wl.coeff["c"], np.float64)
    got = _run_gpu(q, k, v, dy, wl.group_of_dim, a, b, c, "bf16")
    ref = O.attention_backward(q, k, v, dy, wl.group_of_dim, a, b, c)
    _check(got, ref, _majorants(q, k, v, dy, wl.group_of_dim, a, b, c), 256, "based N=256", coef=(a, b, c))


def test_bwd_full_size_sampled_heads():
    """The Based workload at its full size (8 sequences x 16 heads x 8192
    tokens) in one call: dq, dk, dv of two (sequence, head) slices against
    the oracle on that slice alone (sequences and heads are independent), and
    the coefficient gradients of those slices through one-sequence,
    one-head calls, all to the bound above."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(3)
    B, H, N = wl.batch, wl.n_q_heads, wl.seq_len
    rng = np.random.default_rng(2102)
    dy = S.bf16_round(rng.standard_normal(wl.v.shape).astype(np.float32))
    a = np.asarray(wl.coeff["a"], np.float64)
    b = np.asarray(wl.coeff["b"], np.float64)
    c = np.asarray(wl.coeff["c"], np.float64)
    log(f"[bwd] full size B={B} H={H} N={N}")
    co = oal.Coeffs(wl.group_of_dim, a.astype(np.float32), b.astype(np.float32), c.astype(np.float32))
    outs = oal.bwd(to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16"), to_dev(dy, "bf16"), co)
    torch.cuda.synchronize()
    for t in outs:
        assert torch.isfinite(t).all()
    for bi, h in ((0, 0), (B - 1, H - 1)):
        sl = (slice(bi, bi + 1), slice(h, h + 1))
        q1, k1, v1, dy1 = (x[sl].astype(np.float64) for x in (wl.q, wl.k, wl.v, dy))
        hs = slice(h, h + 1)
        g1, a1, b1, c1 = wl.group_of_dim[hs], a[hs], b[hs], c[hs]
        ref = O.attention_backward(q1, k1, v1, dy1, g1, a1, b1, c1)
        maj = _majorants(q1, k1, v1, dy1, g1, a1, b1, c1)
        got = [to_np(t[sl]) for t in outs[:3]]
        _check(got, ref[:3], maj, N, f"full size b={bi} h={h}", names=NAMES[:3])
        co1 = oal.Coeffs(g1, a1.astype(np.float32), b1.astype(np.float32), c1.astype(np.float32))
        got1 = oal.bwd(to_dev(q1, "bf16"), to_dev(k1, "bf16"), to_dev(v1, "bf16"), to_dev(dy1, "bf16"), co1)
        got1 = [to_np(t) for t in got1[3:]]
        _check(got1, ref[3:], ((maj[0][3:]), maj[1]), N, f"full size b={bi} h={h}", names=NAMES[3:])


def test_bwd_empty_inputs():
    """No tokens or no sequences: nothing to differentiate, so the coefficient
    gradients are zero and the (empty) activation gradients untouched."""
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    rng = np.random.default_rng(2103)
    a, b, c = _coeffs(rng, 2, 4)
    groups = np.stack([np.arange(16) % 4] * 2).astype(np.int32)
    co = oal.Coeffs(groups, a.astype(np.float32), b.astype(np.float32), c.astype(np.float32))
    for B, N in ((2, 0), (0, 5)):
        z16 = torch.zeros((B, 2, N, 16), dtype=torch.bfloat16, device="cuda")
        z64 = torch.zeros((B, 2, N, 64), dtype=torch.bfloat16, device="cuda")
        dq, dk, dv, da, db, dc = oal.bwd(z16, z16.clone(), z64, z64.clone(), co)
        torch.cuda.synchronize()
        assert dq.numel() == 0 and dk.numel() == 0 and dv.numel() == 0
        for t in (da, db, dc):
            assert (to_np(t) == 0).all()


def test_bwd_bad_group_id_gives_nan():
    """A group id outside [0, G) cannot be seen on the host: every output of
    that head is NaN, the other heads are unaffected."""
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    rng = np.random.default_rng(2104)
    B, H, N, G = 1, 2, 70, 4
    q, k = _draw(rng, (B, H, N, 16), "bf16"), _draw(rng, (B, H, N, 16), "bf16")
    v, dy = _draw(rng, (B, H, N, 64), "bf16"), _draw(rng, (B, H, N, 64), "bf16")
    groups = np.stack([np.arange(16) % G] * H).astype(np.int32)
    groups[1, 5] = G  # out of range
    a, b, c = _coeffs(rng, H, G)
    import torch
    co = oal.Coeffs(np.stack([np.arange(16) % G] * H), a.astype(np.float32), b.astype(np.float32),
                    c.astype(np.float32))
    co.group_of_dim = torch.from_numpy(groups).cuda()  # planted after the host-side check
    dq, dk, dv, da, db, dc = (to_np(t) for t in oal.bwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                                         to_dev(dy, "bf16"), co))
    for t in (dq, dk, dv):
        assert np.isnan(t[:, 1]).all() and np.isfinite(t[:, 0]).all()
    assert np.isnan(da[1]) and np.isnan(db[1]).all() and np.isnan(dc[1]).all()
    assert np.isfinite(da[0]) and np.isfinite(db[0]).all() and np.isfinite(dc[0]).all()


def test_bwd_deterministic():
    """Two calls on the same inputs give identical bits."""
    require_gpu()
    rng = np.random.default_rng(2105)
    B, H, N, G = 2, 2, 150, 6
    q, k = _draw(rng, (B, H, N, 16), "bf16"), _draw(rng, (B, H, N, 16), "bf16")
    v, dy = _draw(rng, (B, H, N, 64), "bf16"), _draw(rng, (B, H, N, 64), "bf16")
    groups = np.stack([rng.permutation(np.arange(16) % G) for _ in range(H)]).astype(np.int32)
    a, b, c = _coeffs(rng, H, G)
    one = _run_gpu(q, k, v, dy, groups, a, b, c, "bf16")
    two = _run_gpu(q, k, v, dy, groups, a, b, c, "bf16")
    for x, y in zip(one, two):
        assert np.array_equal(x, y)
