"""Bit-exact checks of group-index, head-map and causal-mask handling on GPU.

1. With small-integer inputs and dyadic coefficients every partial sum of the
   fp32 path is exactly representable, so the GPU output must equal the fp64
   oracle rounded to float32, bit for bit.
2. One-hot values v_j = e_(j mod 64) expose exactly which keys enter each row:
   y_i[l] must be exactly zero when no key j <= i has j mod 64 == l.
3. A group id outside [0, G) poisons only its own query head (NaN).
4. Two runs give bitwise identical outputs (no atomics on the output path).
"""

import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import log, require_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu


def _dyadic_case(seed, B=2, Hq=4, Hkv=2, N=160, d=64, G=4):
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, size=(B, Hq, N, d)) * (rng.random((B, Hq, N, d)) < 0.35)
    k = rng.integers(-1, 2, size=(B, Hkv, N, d)) * (rng.random((B, Hkv, N, d)) < 0.35)
    v = rng.integers(-2, 3, size=(B, Hkv, N, 64))
    groups = np.stack([rng.permutation(np.arange(d) % G) for _ in range(Hq)]).astype(np.int32)
    # M = L L^T + eps with dyadic L: a, b, c are dyadic and the kernel is >= eps
    Ls = np.stack([np.tril(rng.integers(1, 5, size=(G + 1, G + 1)) / 4.0) for _ in range(Hq)])
    a, b, c = O.coeffs_from_factor(1.0 / 16, Ls)
    return (q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), groups, a, b, c)


def test_fp32_path_is_bit_exact_on_dyadic_inputs():
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    for seed in (0, 1):
        q, k, v, groups, a, b, c = _dyadic_case(seed)
        y_ref, num, den = O.attention_direct(q, k, v, groups, a, b, c, return_parts=True)
        # premise: numerator and denominator are exact in float32
        assert np.array_equal(num.astype(np.float32).astype(np.float64), num)
        assert np.array_equal(den.astype(np.float32).astype(np.float64), den)
        y = oal.fwd(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"),
                    oal.Coeffs(groups, a.astype(np.float32), b.astype(np.float32), c.astype(np.float32)))
        got = y.cpu().numpy()
        want = y_ref.astype(np.float32)
        log(f"[exact] seed {seed}: mismatches {int((got != want).sum())} of {got.size}")
        assert np.array_equal(got, want)


def _sparse_dyadic_case(seed, d, dtype, diagonal, B=2, Hq=4, Hkv=2, N=160, G=4, heads=None):
    """Inputs on which every operand of every path is exact in bf16 (8
    significant bits), so the kernels' (num, den) are exact whatever the
    operand format (fp32, fp16 or bf16) and the accumulation order.

    Every token of q and k has exactly two nonzero dimensions, each +-1, and
    v is in {-1, 0, 1}: a state entry is an integer of magnitude <= N, every
    group score s_g is in {0, +-1, +-2} / sqrt(d_h), and with a = 2, b in
    {+-1/2} and c from {0, 1, 2} every kernel value is a multiple of 1/64
    below 4 (at most 8 significant bits) and >= 1 (positive denominators).  At d_h = 32, sqrt(d_h) is irrational, so b = 0 there (the
    quadratic term carries 1/d_h, which is dyadic).  The dimension-wise form
    (singleton groups, diagonal c) uses c_rr in {1, 2}.
    """
    rng = np.random.default_rng(seed)
    if heads is not None:
        Hq, Hkv = heads

    def two_hot(shape):
        x = np.zeros(shape + (d,), np.float32)
        for idx in np.ndindex(*shape):
            dims = rng.choice(d, size=2, replace=False)
            x[idx + (dims,)] = rng.choice([-1.0, 1.0], size=2)
        return x

    q, k = two_hot((B, Hq, N)), two_hot((B, Hkv, N))
    v = rng.integers(-1, 2, size=(B, Hkv, N, 64)).astype(np.float32)
    if diagonal:
        G = d
        groups = np.stack([rng.permutation(d) for _ in range(Hq)]).astype(np.int32)
        c = np.stack([np.diag(rng.integers(1, 3, size=d).astype(np.float64)) for _ in range(Hq)])
    else:
        groups = np.stack([rng.permutation(np.arange(d) % G) for _ in range(Hq)]).astype(np.int32)
        w = (rng.random((Hq, G)) < 0.5).astype(np.float64)
        c = np.eye(G)[None] + w[:, :, None] * w[:, None, :]  # I + w w^T: PSD, entries in {0, 1, 2}
    b = rng.choice([-0.5, 0.5], size=(Hq, G))
    if d == 32:
        b[:] = 0.0
    a = np.full(Hq, 2.0)
    return q, k, v, groups, a, b, c


def _ulp(x, dtype):
    """Spacing of the output format at |x| (float32 or bfloat16)."""
    x = np.abs(np.asarray(x, np.float32))
    e = np.floor(np.log2(np.maximum(x, np.float32(2.0 ** -126))))
    return np.ldexp(1.0, (e - (23 if dtype == "f32" else 7)).astype(np.int32))


@pytest.mark.parametrize("d,dtype,diagonal,heads", [(16, "bf16", False, None), (16, "bf16", False, (3, 3)),
                                                    (16, "f32", False, None), (32, "bf16", False, None),
                                                    (32, "f32", False, None), (64, "bf16", False, None),
                                                    (16, "bf16", True, None), (64, "bf16", True, None),
                                                    (64, "bf16", True, (3, 3)),
                                                    (32, "f32", True, None)])
def test_exact_on_sparse_dyadic_inputs(d, dtype, diagonal, heads):
    """Every build (fp32, the bf16-input chunk kernels, the one-pass kernels
    and the dimension-wise form) on inputs where all operands are exact: the
    output equals the oracle's y rounded once to the output format; the only
    freedom left is the rounding of the final division (one unit in the last
    place).  A wrong group id, head map or mask changes y by far more."""
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    q, k, v, groups, a, b, c = _sparse_dyadic_case(100 + d, d, dtype, diagonal, heads=heads)
    y_ref, num, den = O.attention_direct(q, k, v, groups, a, b, c, return_parts=True)
    # premises: numerator and denominator are exact in float32, den >= 1
    assert np.array_equal(num.astype(np.float32).astype(np.float64), num)
    assert np.array_equal(den.astype(np.float32).astype(np.float64), den)
    assert den.min() >= 1.0
    co = oal.Coeffs(groups, a.astype(np.float32), b.astype(np.float32), c.astype(np.float32))
    assert co.diagonal == diagonal
    y = oal.fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), co)
    got = to_np(y)
    want = y_ref.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        want = S.bf16_round(want.astype(np.float32)).astype(np.float64)
    diff = np.abs(got - want)
    exact = int((diff == 0).sum())
    log(f"[exact] d={d} {dtype} diagonal={diagonal} heads={heads}: exact {exact} of {got.size}, max diff in ulps "
        f"{float((diff / _ulp(want, dtype)).max()):.2f}")
    assert (diff <= _ulp(want, dtype)).all()
    # rows whose output is exactly representable (e.g. y_1 = v_1) must be exact
    assert np.array_equal(got[:, :, 0], want[:, :, 0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_mask_with_one_hot_values(dtype):
    require_gpu()
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=1, n_q_heads=2, n_kv_heads=1, seq_len=200, dtype=dtype)
    N = wl.seq_len
    v = np.zeros((1, 1, N, 64), np.float32)
    v[0, 0, np.arange(N), np.arange(N) % 64] = 1.0
    from helpers import gpu_coeffs
    y = to_np(oal.fwd(to_dev(wl.q, dtype), to_dev(wl.k, dtype), to_dev(v, dtype),
                      gpu_coeffs(wl, wl.group_of_dim)))
    i = np.arange(N)[:, None]
    l = np.arange(64)[None, :]
    present = l <= i  # some j <= i with j % 64 == l  <=>  l <= i
    for h in range(2):
        # keys that never entered a row contribute exactly nothing
        assert np.all(y[0, h][~present] == 0.0)
        # first chunk: only the intra-chunk path, whose weights are >= eps > 0
        first = y[0, h][:64]
        assert np.all(first[present[:64]] > 0.0)


def test_bad_group_id_poisons_only_its_head():
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=1, n_q_heads=4, n_kv_heads=2, seq_len=70)
    from helpers import gpu_coeffs
    co = gpu_coeffs(wl, wl.group_of_dim)
    bad = co.group_of_dim.clone()
    bad[2, 5] = 9  # outside [0, 4); bypasses the host check on purpose
    co.group_of_dim = bad
    q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    y = oal.fwd(q, k, v, co).float().cpu()
    assert torch.isnan(y[0, 2]).all()
    assert torch.isfinite(y[0, [0, 1, 3]]).all()


def test_runs_are_bitwise_deterministic():
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    wl = S.make(2, batch=2, n_q_heads=14, n_kv_heads=2, seq_len=300)
    from helpers import gpu_coeffs
    co = gpu_coeffs(wl, wl.group_of_dim)
    q, k, v = to_dev(wl.q, "bf16"), to_dev(wl.k, "bf16"), to_dev(wl.v, "bf16")
    y1, s1 = oal.fwd(q, k, v, co, return_state=True)
    y2, s2 = oal.fwd(q, k, v, co, return_state=True)
    assert torch.equal(y1, y2) and torch.equal(s1, s2)
    c1 = oal.contrib(q, k)
    c2 = oal.contrib(q, k)
    assert torch.equal(c1, c2)
