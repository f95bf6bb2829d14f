"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

None of these re-types the oracle's own formula: each compares it with a
printed value, a closed-form special case, an independent exact computation
(rational arithmetic) or an invariant that a plausible mistake (dropped term,
wrong sign, wrong index, transposed operand, wrong head map) would break.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


# ---------------------------------------------------------------- counts

def test_state_entry_count_matches_pages(golden):
    g = golden("state_counts.json")
    d, dv = 64, 64
    D = O.feature_count(d)
    assert D * (dv + 1) == g["state_entries_d64_dv64"]
    # the oracle's own feature maps have exactly D entries
    rng = np.random.default_rng(0)
    assert O.phi_k_packed(_rand(rng, d)).shape[-1] == D
    assert O.state_from_prefix(_rand(rng, 3, d), _rand(rng, 3, dv)).shape == (D, dv + 1)
    # d_h = 16 workload: (1 + 16 + 136) features
    assert O.feature_count(16) == 153
    # ordered-pair count of App. D
    assert (1 + d + d * d) * (dv + 1) == 1 + d + d * d + (1 + d + d * d) * dv


def test_factor_parameter_count(golden):
    """The factor map (eps, L) -> (a, b, c) of the positive group-aware kernel
    has the printed number of free parameters: at a generic lower-triangular
    L with positive diagonal, the Jacobian of the independent outputs (a, b
    and the upper triangle of the symmetric c) with respect to the
    lower-triangular entries of L is square, of size (G+1)(G+2)/2, and of full
    rank (M = L L^T is a local bijection there).  A map that dropped an entry
    of L, or wrote an asymmetric c, fails the rank or the symmetry check."""
    rng = np.random.default_rng(39)
    for G, n in golden("state_counts.json")["params"]:
        tri = [(i, j) for i in range(G + 1) for j in range(i + 1)]
        assert len(tri) == n
        L0 = np.zeros((G + 1, G + 1))
        for (i, j) in tri:
            L0[i, j] = rng.uniform(0.5, 1.5) if i == j else rng.uniform(-0.5, 0.5)

        def outputs(Lm):
            a, b, c = O.coeffs_from_factor(0.0, Lm)
            assert np.array_equal(c, c.T)
            iu = np.triu_indices(G)
            return np.concatenate([[a], b, c[iu]])

        assert outputs(L0).size == n
        h = 1e-6
        J = np.zeros((n, n))
        for col, (i, j) in enumerate(tri):
            Lp, Lm = L0.copy(), L0.copy()
            Lp[i, j] += h
            Lm[i, j] -= h
            J[:, col] = (outputs(Lp) - outputs(Lm)) / (2 * h)
        assert np.linalg.matrix_rank(J, tol=1e-6) == n


# ---------------------------------------------------------------- closed forms

def test_taylor_special_case_single_group():
    """One group with a=1, b=1, c=1/2 is the second-order Taylor polynomial of s."""
    rng = np.random.default_rng(1)
    d = 64
    for _ in range(20):
        q, k = _rand(rng, d), _rand(rng, d)
        s = float(np.dot(q, k)) / math.sqrt(d)
        want = 1.0 + s + 0.5 * s * s
        got = O.kappa(q, k, np.zeros(d, int), 1.0, [1.0], [[0.5]])
        assert got == pytest.approx(want, rel=1e-14, abs=1e-14)


def test_taylor_with_uniform_coefficients_over_any_partition():
    """Equal b_g and c_gh over any partition reduce to the global polynomial
    (OAL App. D, positive global reference: s is the sum of the s_g)."""
    rng = np.random.default_rng(2)
    d = 16
    for G in (2, 3, 5, 16):
        gmap = rng.integers(0, G, size=d)
        gmap[:G] = np.arange(G)  # every group non-empty
        rng.shuffle(gmap)
        b = np.full(G, 1.0)
        c = np.full((G, G), 0.5)
        q, k = _rand(rng, d), _rand(rng, d)
        s = float(np.dot(q, k)) / math.sqrt(d)
        assert O.kappa(q, k, gmap, 1.0, b, c) == pytest.approx(1 + s + 0.5 * s * s, rel=1e-13)


def test_based_parabola_floor(golden):
    pts = golden("taylor_parabola.json")["points"]
    d = 16
    for t, want in pts:
        # q = 2 e_0 and k = (t * 2) e_0 give s = 4t / sqrt(16) = t exactly
        q = np.zeros(d); q[0] = 2.0
        k = np.zeros(d); k[0] = 2.0 * t
        assert O.kappa(q, k, np.zeros(d, int), 1.0, [1.0], [[0.5]]) == want
    rng = np.random.default_rng(3)
    vals = [O.kappa(_rand(rng, d), _rand(rng, d), np.zeros(d, int), 1.0, [1.0], [[0.5]]) for _ in range(200)]
    assert min(vals) >= 0.5


def test_grouped_kernel_hand_example(golden):
    g = golden("grouped_kernel_example.json")
    got = O.kappa(np.array(g["q"]), np.array(g["k"]), np.array(g["group_of_dim"]), g["a"], g["b"], g["c"])
    want = g["kappa_rational_part"] + g["kappa_coefficient_of_inv_sqrt2"] / math.sqrt(2.0)
    assert got == pytest.approx(want, rel=1e-15)


def test_asymmetric_group_pair_terms_enter_with_both_orders():
    """c_gh and c_hg are both summed: an off-diagonal-only c gives 2 c s_1 s_2."""
    d = 2
    q, k = np.array([1.0, 1.0]), np.array([2.0, 3.0])
    s1, s2 = 2.0 / math.sqrt(2), 3.0 / math.sqrt(2)
    c = [[0.0, 0.25], [0.25, 0.0]]
    got = O.kappa(q, k, np.array([0, 1]), 0.0, [0.0, 0.0], c)
    assert got == pytest.approx(2 * 0.25 * s1 * s2, rel=1e-15)
    # a linear-only kernel picks the right group for each b
    got = O.kappa(q, k, np.array([0, 1]), 0.0, [1.0, -2.0], [[0, 0], [0, 0]])
    assert got == pytest.approx(s1 - 2 * s2, rel=1e-15)


# ---------------------------------------------------------------- positivity

def test_eq7_positivity_and_denominator_floor():
    rng = np.random.default_rng(4)
    d, G, eps = 8, 3, 1e-3
    gmap = np.array([0, 1, 2, 2, 1, 0, 2, 2])
    for trial in range(5):
        L = np.tril(rng.uniform(-1, 1, size=(G + 1, G + 1)))
        a, b, c = O.coeffs_from_factor(eps, L)
        for _ in range(50):
            assert O.kappa(_rand(rng, d, std=3), _rand(rng, d, std=3), gmap, a, b, c) >= eps * (1 - 1e-12)
    # den_i >= (i+1) eps along a sequence
    B, H, N, dv = 1, 1, 40, 3
    Q, K, V = _rand(rng, B, H, N, d, std=2), _rand(rng, B, H, N, d, std=2), _rand(rng, B, H, N, dv)
    _, _, den = O.attention_direct(Q, K, V, [gmap], [a], [b], [c], return_parts=True)
    assert np.all(den[0, 0] >= (np.arange(N) + 1) * eps * (1 - 1e-12))


def test_psd_c_alone_does_not_give_nonnegative_kernel():
    """The positivity needs the full M = [[a, b/2], [b/2, c]] PSD, not c alone."""
    d = 4
    q = np.array([1.0, 0, 0, 0]); k = np.array([-1.0, 0, 0, 0])  # s = -1/2
    val = O.kappa(q, k, np.zeros(d, int), 0.1, [1.0], [[1.0]])
    assert val == pytest.approx(-0.15, rel=1e-14)


def test_global_embedding_is_psd_and_matches():
    """OAL App. D: M_00 = m00, M_0g = m01, M_gh = m11 embeds a PSD global
    quadratic into any partition, stays PSD and gives the same kernel."""
    rng = np.random.default_rng(5)
    d, G = 12, 4
    gmap = np.array([0, 1, 2, 3] * 3)
    for _ in range(5):
        Lg = np.tril(rng.uniform(-1, 1, size=(2, 2)))
        Mg = Lg @ Lg.T
        M = np.empty((G + 1, G + 1))
        M[0, 0] = Mg[0, 0]
        M[0, 1:] = M[1:, 0] = Mg[0, 1]
        M[1:, 1:] = Mg[1, 1]
        assert np.linalg.eigvalsh(M).min() >= -1e-12
        eps = 0.01
        a, b, c = eps + M[0, 0], 2 * M[0, 1:], M[1:, 1:]
        q, k = _rand(rng, d), _rand(rng, d)
        s = float(np.dot(q, k)) / math.sqrt(d)
        want = eps + Mg[0, 0] + 2 * Mg[0, 1] * s + Mg[1, 1] * s * s
        assert O.kappa(q, k, gmap, a, b, c) == pytest.approx(want, rel=1e-12)


# ---------------------------------------------------------------- worked example

def test_mercer_counterexample(golden):
    g = golden("mercer_counterexample.json")
    eps = 0.25
    a, b, c = O.coeffs_from_factor(eps, np.array(g["L_factor"]))
    assert np.allclose(np.array(g["L_factor"]) @ np.array(g["L_factor"]).T, g["M"])
    assert (a, b[0], c[0][0]) == (eps + 1.0, -2.0, 1.0)
    xs = g["inputs"]
    gram = np.array([[O.kappa(np.array([x]), np.array([z]), np.zeros(1, int), a, b, c) for z in xs] for x in xs])
    want = eps * np.array(g["gram_eps_coefficient"]) + np.array(g["gram_constant"])
    assert np.array_equal(gram, want)
    ev = sorted(np.linalg.eigvalsh(gram))
    want_ev = sorted(ec * eps + cst for ec, cst in g["eigenvalues_as_eps_coeff_and_constant"])
    assert np.allclose(ev, want_ev, rtol=0, atol=1e-14)
    # derived causal output at position 2
    v = np.array([[3.0, -1.0], [0.5, 2.0]])
    Q = np.array([0.0, -1.0]).reshape(1, 1, 2, 1)
    K = np.array([1.0, -1.0]).reshape(1, 1, 2, 1)
    y = O.attention_direct(Q, K, v.reshape(1, 1, 2, 2), [np.zeros(1, int)], [a], [b], [c])
    want_y2 = ((eps + 4) * v[0] + eps * v[1]) / (2 * eps + 4)
    assert np.allclose(y[0, 0, 1], want_y2, rtol=1e-15, atol=0)


def test_coeffs_from_factor_hand_example():
    # L = [[1, 0], [0.5, 2]] -> M = [[1, 0.5], [0.5, 4.25]]
    a, b, c = O.coeffs_from_factor(0.125, np.array([[1.0, 0.0], [0.5, 2.0]]))
    assert a == 1.125 and b[0] == 1.0 and c[0][0] == 4.25


# ---------------------------------------------------------------- exact brute force

def _fraction_attention(Q, K, V, gmap, a, b, c, sqrt_d):
    """Definition in exact rational arithmetic; sqrt(d) must be an integer."""
    N, d = len(Q), len(Q[0])
    G = len(b)
    out = []
    for i in range(N):
        num = [Fraction(0)] * len(V[0])
        den = Fraction(0)
        for j in range(i + 1):
            s = [Fraction(0)] * G
            for r in range(d):
                s[gmap[r]] += Fraction(Q[i][r]) * Fraction(K[j][r]) / sqrt_d
            kap = Fraction(a) + sum(Fraction(b[g]) * s[g] for g in range(G))
            kap += sum(Fraction(c[g][h]) * s[g] * s[h] for g in range(G) for h in range(G))
            den += kap
            num = [num[l] + kap * Fraction(V[j][l]) for l in range(len(V[0]))]
        out.append([x / den for x in num])
    return out


def test_direct_form_matches_exact_rational_bruteforce():
    rng = np.random.default_rng(6)
    d, dv, N, G = 4, 3, 6, 2
    gmap = [1, 0, 1, 0]
    Q = np.round(_rand(rng, N, d) * 8) / 8
    K = np.round(_rand(rng, N, d) * 8) / 8
    V = np.round(_rand(rng, N, dv) * 8) / 8
    a, b, c = 0.75, [0.5, -0.25], [[0.5, 0.125], [0.125, 0.375]]
    want = np.array(_fraction_attention(Q.tolist(), K.tolist(), V.tolist(), gmap, a, b, c, 2), dtype=float)
    got = O.attention_direct(Q[None, None], K[None, None], V[None, None], [gmap], [a], [b], [c])[0, 0]
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- forms agree

def _small_case(rng, B=2, Hq=4, Hkv=2, N=11, d=4, dv=3, G=3):
    Q, K, V = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, dv)
    groups = np.stack([rng.permutation(np.arange(d) % G) for _ in range(Hq)])
    Ls = [np.tril(rng.uniform(0.1, 1.0, size=(G + 1, G + 1))) for _ in range(Hq)]
    abc = [O.coeffs_from_factor(1e-3, L) for L in Ls]
    a = np.array([x[0] for x in abc]); b = np.array([x[1] for x in abc]); c = np.array([x[2] for x in abc])
    return Q, K, V, groups, a, b, c


def test_direct_equals_packed_and_ordered_recurrences():
    rng = np.random.default_rng(7)
    Q, K, V, groups, a, b, c = _small_case(rng)
    yd = O.attention_direct(Q, K, V, groups, a, b, c)
    yp = O.attention_recurrent_packed(Q, K, V, groups, a, b, c)
    yo = O.attention_recurrent_ordered(Q, K, V, groups, a, b, c)
    assert np.allclose(yp, yd, rtol=1e-11, atol=1e-12)
    assert np.allclose(yo, yd, rtol=1e-11, atol=1e-12)


def test_row_subset_is_exact():
    rng = np.random.default_rng(8)
    Q, K, V, groups, a, b, c = _small_case(rng, N=17)
    rows = np.array([0, 5, 16])
    assert np.allclose(O.attention_direct(Q, K, V, groups, a, b, c, rows=rows),
                       O.attention_direct(Q, K, V, groups, a, b, c)[:, :, rows], rtol=1e-14, atol=1e-15)


def test_gqa_head_map_is_consecutive_blocks():
    rng = np.random.default_rng(9)
    Q, K, V, groups, a, b, c = _small_case(rng, Hq=6, Hkv=2)
    y = O.attention_direct(Q, K, V, groups, a, b, c)
    for h in range(6):
        kh = h // 3
        yh = O.attention_direct(Q[:, h:h + 1], K[:, kh:kh + 1], V[:, kh:kh + 1], groups[h:h + 1],
                                a[h:h + 1], b[h:h + 1], c[h:h + 1])
        assert np.allclose(yh[:, 0], y[:, h], rtol=1e-14, atol=1e-15)


def test_invariants():
    rng = np.random.default_rng(10)
    Q, K, V, groups, a, b, c = _small_case(rng, B=1, Hq=2, Hkv=1)
    y = O.attention_direct(Q, K, V, groups, a, b, c)
    # first position returns its own value
    assert np.allclose(y[:, :, 0], V[:, [0, 0], 0], rtol=1e-14)
    # constant values are reproduced everywhere
    Vc = np.broadcast_to(np.array([1.5, -2.0, 0.25]), V.shape).copy()
    assert np.allclose(O.attention_direct(Q, K, Vc, groups, a, b, c), 1.5 * 0 + Vc[:, [0, 0]], rtol=1e-13)
    # positive rescaling of (a, b, c)
    assert np.allclose(O.attention_direct(Q, K, V, groups, 3 * a, 3 * b, 3 * c), y, rtol=1e-12)
    # joint permutation of the dimensions and the group map
    perm = rng.permutation(Q.shape[-1])
    yp = O.attention_direct(Q[..., perm], K[..., perm], V, groups[:, perm], a, b, c)
    assert np.allclose(yp, y, rtol=1e-12)
    # identical query heads give identical outputs
    Q2 = Q.copy(); Q2[:, 1] = Q2[:, 0]
    g2 = groups.copy(); g2[1] = g2[0]
    y2 = O.attention_direct(Q2, K, V, g2, a[[0, 0]], b[[0, 0]], c[[0, 0]])
    assert np.array_equal(y2[:, 0], y2[:, 1])


def test_decode_step_matches_direct_last_row_and_state():
    rng = np.random.default_rng(11)
    d, dv, G, Hq, Hkv, n = 4, 3, 2, 4, 2, 9
    Q, K, V, groups, a, b, c = _small_case(rng, B=1, Hq=Hq, Hkv=Hkv, N=n + 1, d=d, dv=dv, G=G)
    state = np.stack([O.state_from_prefix(K[0, kh, :n], V[0, kh, :n]) for kh in range(Hkv)])[None]
    y, st = O.decode_step(state, Q[:, :, n], K[:, :, n], V[:, :, n], groups, a, b, c, Hq)
    yd = O.attention_direct(Q, K, V, groups, a, b, c, rows=np.array([n]))
    assert np.allclose(y, yd[:, :, 0], rtol=1e-12)
    full = np.stack([O.state_from_prefix(K[0, kh], V[0, kh]) for kh in range(Hkv)])[None]
    assert np.allclose(st, full, rtol=1e-13)
    # the packed state holds raw moments: entry for pair (r, t) is sum k_r k_t v
    D = O.feature_count(d)
    pairs = O.packed_pairs(d)
    f = 1 + d + pairs.index((1, 3))
    assert np.isclose(full[0, 0, f, 0], np.sum(K[0, 0, :, 1] * K[0, 0, :, 3] * V[0, 0, :, 0]))
    assert full.shape[2] == D


def test_state_resume_equals_full_run():
    rng = np.random.default_rng(12)
    Q, K, V, groups, a, b, c = _small_case(rng, B=1, N=14)
    y_full, S_full = O.attention_recurrent_packed(Q, K, V, groups, a, b, c, return_state=True)
    y1, S1 = O.attention_recurrent_packed(Q[:, :, :6], K[:, :, :6], V[:, :, :6], groups, a, b, c, return_state=True)
    y2, S2 = O.attention_recurrent_packed(Q[:, :, 6:], K[:, :, 6:], V[:, :, 6:], groups, a, b, c,
                                          state_in=S1, return_state=True)
    assert np.allclose(np.concatenate([y1, y2], axis=2), y_full, rtol=1e-12)
    assert np.allclose(S2, S_full, rtol=1e-13)


def test_abi_state_layout_roundtrip():
    rng = np.random.default_rng(13)
    S = _rand(rng, 2, 3, 15, 5)
    flat = O.abi_state_from_matrix(S)
    assert flat.shape == (2, 3, 15 * 4 + 15)
    assert np.array_equal(flat[..., :4], S[..., 0, :4])  # first H row
    assert np.array_equal(flat[..., 60:], S[..., :, 4])  # z column at the end
    assert np.array_equal(O.matrix_from_abi_state(flat, 15, 4), S)


# ---------------------------------------------------------------- ReBased readings

def test_premap_affine_golden(golden):
    """gamma and beta of the ReBased pre-map, against hand-worked values:
    gamma scales the normalised value, beta is added after the scaling, and
    the LayerNorm epsilon is added to the biased variance inside the root."""
    g = golden("premap_affine.json")
    for case in g["cases"]:
        got = O.premap(np.array(case["x"], float), np.array(case["gamma"], float), np.array(case["beta"], float),
                       case["eps"])
        assert np.allclose(got, case["want"], rtol=1e-15, atol=1e-15), (case, got)
    # over a batch of rows the map acts row by row
    rows = np.array([g["cases"][0]["x"], g["cases"][0]["x"]], float)
    got = O.premap(rows, np.array(g["cases"][0]["gamma"]), np.array(g["cases"][0]["beta"]), 2.0)
    assert np.array_equal(got, np.array([g["cases"][0]["want"]] * 2))


def test_rebased_premap_and_feature_readings():
    rng = np.random.default_rng(14)
    d = 16
    x = _rand(rng, 5, d, std=3)
    z = O.premap(x, np.ones(d), np.zeros(d), 1e-5)
    assert np.allclose(z.mean(-1), 0, atol=1e-12)
    var = x.var(-1)
    assert np.allclose((z ** 2).mean(-1), var / (var + 1e-5), rtol=1e-12)
    gq, bq = 1 + 0.3 * _rand(rng, d), 0.3 * _rand(rng, d)
    gk, bk = 1 + 0.3 * _rand(rng, d), 0.3 * _rand(rng, d)
    q, k = _rand(rng, d), _rand(rng, d)
    qt, kt = O.premap(q, gq, bq), O.premap(k, gk, bk)
    # elementwise-square reading: d singleton groups, c = d I, a = b = 0
    val = O.kappa(qt, kt, np.arange(d), 0.0, np.zeros(d), d * np.eye(d))
    assert val == pytest.approx(float(np.dot(qt ** 2, kt ** 2)), rel=1e-12)
    # squared-dot-product reading: one group, c = d
    val = O.kappa(qt, kt, np.zeros(d, int), 0.0, [0.0], [[float(d)]])
    assert val == pytest.approx(float(np.dot(qt, kt)) ** 2, rel=1e-12)


def test_premap_l2_golden(golden):
    """The TaylorShift-style pre-map (unit l2 norm, then gamma and beta),
    against hand-worked values: no centring, the sum (not the mean) of
    squares, epsilon inside the root."""
    g = golden("premap_l2.json")
    for case in g["cases"]:
        got = O.premap(np.array(case["x"], float), np.array(case["gamma"], float), np.array(case["beta"], float),
                       case["eps"], kind="l2")
        assert np.allclose(got, case["want"], rtol=1e-15, atol=1e-15), (case, got)


def test_premap_l2_unit_norm_and_scale_invariance():
    rng = np.random.default_rng(41)
    d = 16
    x = _rand(rng, 7, d, std=3)
    z = O.premap(x, np.ones(d), np.zeros(d), 0.0, kind="l2")
    assert np.allclose(np.linalg.norm(z, axis=-1), 1.0, rtol=1e-14)
    assert np.allclose(O.premap(4.5 * x, np.ones(d), np.zeros(d), 0.0, kind="l2"), z, rtol=1e-14)
    # the direction is kept (z is a positive multiple of x)
    assert np.allclose(z * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-13)


def test_taylorshift_through_the_grouped_kernel():
    """[OAL] App. F.1, the TaylorShift baseline: kappa = 1 + s + s^2 / 2 with
    s = tau * qhat . khat over unit vectors, causal and normalised.  The
    oracle's path (l2 pre-map with gamma_q = tau sqrt(d), gamma_k = 1, beta =
    0, then one group with a = 1, b = 1, c = 1/2) must equal that formula
    written out here with numpy's norm."""
    rng = np.random.default_rng(42)
    B, H, N, d, dv = 2, 3, 9, 8, 5
    Q, K, V = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d), _rand(rng, B, H, N, dv)
    tau = np.array([0.7, 1.0, 2.3])
    p = {"gamma_q": np.repeat((tau * math.sqrt(d))[:, None], d, 1), "beta_q": np.zeros((H, d)),
         "gamma_k": np.ones((H, d)), "beta_k": np.zeros((H, d)), "ln_eps": 0.0, "kind": "l2"}
    got = O.attention_direct(Q, K, V, np.zeros((H, d), int), np.ones(H), np.ones((H, 1)), np.full((H, 1, 1), 0.5),
                             premap_params=p)
    want = np.zeros_like(got)
    for bi in range(B):
        for h in range(H):
            qh = Q[bi, h] / np.linalg.norm(Q[bi, h], axis=-1, keepdims=True)
            kh = K[bi, h] / np.linalg.norm(K[bi, h], axis=-1, keepdims=True)
            s = tau[h] * qh @ kh.T
            w = np.tril(1 + s + 0.5 * s ** 2)
            want[bi, h] = (w @ V[bi, h]) / w.sum(1, keepdims=True)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- backward

def test_attention_backward_against_finite_differences():
    """The oracle's analytic gradients of sum(dY * y) against central finite
    differences of the forward definition (attention_direct) in fp64, on a
    tiny grouped-query case with uneven groups: every element of Q, K, V and
    of a, b, c."""
    rng = np.random.default_rng(61)
    B, Hq, Hkv, N, d, dv, G = 1, 2, 1, 5, 4, 3, 2
    Q, K, V = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, dv)
    dY = _rand(rng, B, Hq, N, dv)
    groups = np.array([[0, 1, 1, 0], [1, 0, 0, 1]])
    a, b, c = O.coeffs_from_factor(0.1, rng.standard_normal((Hq, G + 1, G + 1)) * 0.7)
    c = c + 0.05 * rng.standard_normal(c.shape)  # not symmetric: every ordered entry is its own parameter

    def loss(Q_, K_, V_, a_, b_, c_):
        return float((dY * O.attention_direct(Q_, K_, V_, groups, a_, b_, c_)).sum())

    got = O.attention_backward(Q, K, V, dY, groups, a, b, c)
    args = [Q, K, V, a, b, c]
    h = 1e-6
    for which, g in enumerate(got):
        x = args[which]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            up = [np.array(t, dtype=np.float64, copy=True) for t in args]
            dn = [np.array(t, dtype=np.float64, copy=True) for t in args]
            up[which][idx] += h
            dn[which][idx] -= h
            fd[idx] = (loss(*up) - loss(*dn)) / (2 * h)
        scale = max(np.abs(fd).max(), 1e-3)
        assert np.abs(g - fd).max() <= 1e-6 * scale, (which, np.abs(g - fd).max(), scale)


def test_attention_backward_closed_form_single_key():
    """N = 1: y = v (any kernel), so dV = dY and every other gradient is 0."""
    rng = np.random.default_rng(62)
    Q, K, V, dY = _rand(rng, 1, 1, 1, 4), _rand(rng, 1, 1, 1, 4), _rand(rng, 1, 1, 1, 3), _rand(rng, 1, 1, 1, 3)
    a, b, c = O.coeffs_from_factor(0.1, rng.standard_normal((1, 3, 3)))
    dQ, dK, dV, da, db, dc = O.attention_backward(Q, K, V, dY, np.array([[0, 0, 1, 1]]), a, b, c)
    assert np.allclose(dV, dY, rtol=1e-14)
    for g in (dQ, dK, da, db, dc):
        assert np.abs(g).max() <= 1e-14


# ---------------------------------------------------------------- contribution score

def test_chi_bruteforce_equals_separable_varlen_gqa():
    rng = np.random.default_rng(15)
    P, Hq, Hkv, N, d = 3, 4, 2, 9, 5
    Q, K = _rand(rng, P, Hq, N, d), _rand(rng, P, Hkv, N, d)
    lens = np.array([9, 4, 1])
    pb, mb = O.chi_bruteforce(Q, K, lens)
    ps, ms = O.chi_separable(Q, K, lens)
    assert np.allclose(pb, ps, rtol=1e-12) and np.allclose(mb, ms, rtol=1e-12)
    # equal-weight average over prompts, not over pairs
    assert np.allclose(mb, pb.mean(0))


def test_chi_closed_forms():
    P, Hq, Hkv, N, d = 2, 2, 1, 7, 4
    ones = np.ones((P, Hq, N, d))
    _, m = O.chi_bruteforce(ones, np.ones((P, Hkv, N, d)))
    assert np.allclose(m, 1 / math.sqrt(d), rtol=1e-14)
    rng = np.random.default_rng(16)
    Q, K = _rand(rng, P, Hq, N, d), _rand(rng, P, Hkv, N, d)
    _, m0 = O.chi_bruteforce(Q, K)
    Q2, K2 = Q.copy(), K.copy()
    Q2[..., 2] *= -3.0
    K2[..., 2] *= 0.5
    _, m1 = O.chi_bruteforce(Q2, K2)
    assert np.allclose(m1[:, 2], 1.5 * m0[:, 2], rtol=1e-13)
    assert np.allclose(m1[:, [0, 1, 3]], m0[:, [0, 1, 3]], rtol=1e-14)


def test_chi_gaussian_expectation():
    rng = np.random.default_rng(17)
    P, H, N, d = 4, 2, 400, 16
    _, m = O.chi_separable(_rand(rng, P, H, N, d), _rand(rng, P, H, N, d))
    assert abs(m.mean() - (2 / math.pi) / math.sqrt(d)) < 0.03 * (2 / math.pi) / math.sqrt(d)


# ---------------------------------------------------------------- grouping
# Hand-worked cases of the outlier-aware grouping ([OAL] App. B; the
# bootstrap separation R_k^(b) of the deck's backup slide on bootstrap
# support).  Expected partitions, gap ratios and supports are derived in the
# comments, not by the oracle's own arithmetic.

def test_grouping_stable_outliers_become_tail_groups():
    # means: dims 0..5 ~ 1, dim 6 = 10, dim 7 = 30; alpha = 0.25 -> m = 2,
    # candidate cuts k = 6, 7.  rho_6 = 10 / 1, rho_7 = 30 / 10 = 3.  In every
    # replicate min(dims 6, 7) / max(dims 0..5) >= 9 / 1.1 and dim 7 / max(dims
    # 0..6) >= 89/3 / (31/3) > 2.8, so S_6 = S_7 = 1: both cuts are natural.
    chi_pp = [[1, 1, 1, 1, 1, 1, 10, 30], [1.1, 0.9, 1, 1, 1, 1, 11, 29], [0.9, 1.1, 1, 1, 1, 1, 9, 31]]
    boot = [[0, 1, 2], [0, 0, 1], [2, 2, 2], [1, 2, 0]]
    gid, G, rho, sup = O.group_dims_bootstrap(chi_pp, boot, alpha=0.25, gamma=0.9)
    assert gid == [0, 0, 0, 0, 0, 0, 1, 2] and G == 3
    assert sorted(rho) == [6, 7]
    assert rho[6] == pytest.approx(10.0, rel=1e-12) and rho[7] == pytest.approx(3.0, rel=1e-12)
    assert sup == {6: 1.0, 7: 1.0}


def test_grouping_unstable_gap_is_not_a_natural_cut():
    # dim 3 is large only in prompt 0: mean 28.1875 against dim 2 = 4, so
    # rho_3 = 7.046875 >= tau, but the replicates that miss prompt 0 see
    # 4.25 / 4 < 1.5: S_3 = 2/4 < gamma.  The cut k = 2 (dims {0,1} | {2,3})
    # has rho_2 = 4 / 2 = 2 and R_2 = 4 / 2 in every replicate: natural.
    chi_pp = [[1, 2, 4, 100], [1, 2, 4, 4.25], [1, 2, 4, 4.25], [1, 2, 4, 4.25]]
    boot = [[0, 0, 1, 2], [1, 2, 3, 1], [1, 1, 2, 3], [0, 1, 2, 3]]
    gid, G, rho, sup = O.group_dims_bootstrap(chi_pp, boot, alpha=0.5, gamma=0.9)
    assert gid == [0, 0, 1, 1] and G == 2
    assert rho == {2: 2.0, 3: 28.1875 / 4}
    assert sup == {2: 1.0, 3: 0.5}
    # with three groups required, the remaining candidate is added
    gid3, G3, _, _ = O.group_dims_bootstrap(chi_pp, boot, alpha=0.5, gamma=0.9, g_min=3)
    assert gid3 == [0, 0, 1, 2] and G3 == 3


def test_grouping_flat_profile_falls_back_to_first_candidate():
    # all scores equal: rho = 1 < tau and R = 1 < tau everywhere, so no natural
    # cut; every candidate ties on (S, rho) = (0, 1) and the first candidate
    # cut, k = d - ceil(alpha d) = 3, is taken: G_min = 2 groups.
    chi_pp = [[1.0] * 6, [1.0] * 6]
    gid, G, rho, sup = O.group_dims_bootstrap(chi_pp, [[0, 1], [1, 1]], alpha=0.5, gamma=0.5)
    assert gid == [0, 0, 0, 1, 1, 1] and G == 2
    assert rho == {3: 1.0, 4: 1.0, 5: 1.0} and sup == {3: 0.0, 4: 0.0, 5: 0.0}


def test_grouping_fallback_prefers_support_over_gap():
    # means [1, 2.05, 4.65]: rho_1 = 2.05, rho_2 = 4.65 / 2.05.  Replicates:
    # p0 alone [1, 3, 3.3]: R_1 = 3, R_2 = 1.1; p1 alone [1, 1.1, 6]: R_1 =
    # 1.1, R_2 = 6 / 1.1; the mean: R_1 = 2.05, R_2 = 2.27.  With replicates
    # (p0 p0), (p1 p1), (p0 p1), (p0 p0): S_1 = 3/4, S_2 = 2/4, both below
    # gamma = 0.9.  The fallback takes k = 1 (higher S) although rho_1 < rho_2.
    chi_pp = [[1, 3, 3.3], [1, 1.1, 6]]
    boot = [[0, 0], [1, 1], [0, 1], [0, 0]]
    gid, G, rho, sup = O.group_dims_bootstrap(chi_pp, boot, alpha=1.0, gamma=0.9)
    assert sup == {1: 0.75, 2: 0.5}
    assert rho[1] < rho[2]
    assert gid == [0, 1, 1] and G == 2


def test_grouping_budget_rule():
    # sorted values 1, 2, 3, 4, 30 (dims 0, 1, 2, 4, 3): gaps rho_1..4 = 2,
    # 1.5, 4/3, 7.5; the two largest are k = 4 and k = 1.
    gid, rho = O.group_dims_budget([1, 2, 3, 30, 4], 3)
    assert gid == [0, 1, 1, 2, 1]
    assert rho == pytest.approx({1: 2.0, 2: 1.5, 3: 4 / 3, 4: 7.5})
    assert O.group_dims_budget([1, 2, 3, 30, 4], 1)[0] == [0] * 5
    # a group per dimension: the group id is the rank
    assert O.group_dims_budget([1, 2, 3, 30, 4], 5)[0] == [0, 1, 2, 4, 3]
    # equal scores keep index order: sorted dims 1, 3, 0, 2; one gap of 5
    assert O.group_dims_budget([5, 1, 5, 1], 2)[0] == [1, 0, 1, 0]


# ---------------------------------------------------------------- contribution-sorted split

def test_groups_sorted_split_golden(golden):
    g = golden("sorted_split.json")
    got = O.groups_sorted_split([g["chi"]], g["bulk_sizes"], g["n_tail"])
    assert got.tolist() == [g["want"]]


def test_groups_sorted_split_properties():
    """Every dimension gets exactly one group; bulk groups have the requested
    sizes; every dimension of a higher group has a score >= every dimension
    of a lower group (contiguous runs of the ascending order); the top n_tail
    scores are singletons; and a permutation of the scores permutes the map
    (no dependence on position except through ties)."""
    rng = np.random.default_rng(77)
    bulk, tail = [11, 11, 10, 10, 10, 10], 2
    chi = rng.random((3, 64))
    gid = O.groups_sorted_split(chi, bulk, tail)
    for h in range(3):
        sizes = np.bincount(gid[h], minlength=8)
        assert sizes.tolist() == bulk + [1, 1]
        for g in range(7):
            assert chi[h][gid[h] == g].max() <= chi[h][gid[h] == g + 1].min()
        top = np.argsort(chi[h])[-2:]
        assert gid[h][top].tolist() == [6, 7]
        perm = rng.permutation(64)
        gp = O.groups_sorted_split(chi[h:h + 1, perm], bulk, tail)[0]
        assert np.array_equal(gp, gid[h][perm])
    with pytest.raises(ValueError):
        O.groups_sorted_split(chi, [10], 2)


# ---------------------------------------------------------------- calibration

def test_softmax_attention_bruteforce_and_closed_forms():
    """The calibration target against pure-Python loops of its definition on
    a tiny grouped-query case, and closed forms: one key gives y = v; equal
    keys give the prefix mean of the values."""
    rng = np.random.default_rng(71)
    B, Hq, Hkv, N, d, dv = 1, 2, 1, 5, 3, 2
    Q, K, V = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, dv)
    got = O.softmax_attention(Q, K, V)
    for h in range(Hq):
        for i in range(N):
            w = [math.exp(sum(Q[0, h, i, r] * K[0, 0, j, r] for r in range(d)) / math.sqrt(d)) for j in range(i + 1)]
            for col in range(dv):
                ref = sum(w[j] * V[0, 0, j, col] for j in range(i + 1)) / sum(w)
                assert abs(got[0, h, i, col] - ref) <= 1e-13 * max(1.0, abs(ref))
    one = O.softmax_attention(Q[:, :, :1], K[:, :, :1], V[:, :, :1])
    assert np.allclose(one[0, 0, 0], V[0, 0, 0], rtol=1e-15)
    Ke = np.repeat(K[:, :, :1], N, axis=2)
    eq = O.softmax_attention(Q, Ke, V)
    for i in range(N):
        assert np.allclose(eq[0, 1, i], V[0, 0, : i + 1].mean(axis=0), rtol=1e-13)


def test_factor_grad_finite_differences():
    """dJ/dL for J = w_a a + w_b . b + sum w_c * c (non-symmetric weights),
    (a, b, c) = coeffs_from_factor(eps, L), against central differences in
    every lower-triangular entry of L."""
    rng = np.random.default_rng(72)
    G = 3
    L = np.tril(rng.standard_normal((G + 1, G + 1)))
    wa, wb, wc = rng.standard_normal(), rng.standard_normal(G), rng.standard_normal((G, G))

    def J(L_):
        a, b, c = O.coeffs_from_factor(0.01, L_)
        return wa * a + (wb * b).sum() + (wc * c).sum()

    g = O.factor_grad(L, wa, wb, wc)
    h = 1e-6
    for i in range(G + 1):
        for j in range(G + 1):
            if j > i:
                assert g[i, j] == 0.0
                continue
            up, dn = L.copy(), L.copy()
            up[i, j] += h
            dn[i, j] -= h
            fd = (J(up) - J(dn)) / (2 * h)
            assert abs(g[i, j] - fd) <= 1e-7 * max(1.0, abs(fd)), (i, j)


def test_adam_clip_step_closed_forms():
    """First Adam step: the bias-corrected moments are g and g^2, so each
    coordinate moves by -lr g / (|g| + eps).  A gradient of norm 100 with the
    clip at 10 enters the moments scaled by 10 / (100 + 1e-6); a second step
    follows the moment recursions written out by hand."""
    g = np.array([3.0, -0.5, 1e-3])
    th, m, v = O.adam_clip_step(np.zeros(3), g, np.zeros(3), np.zeros(3), 1, 0.02, 10.0)
    assert np.allclose(th, -0.02 * g / (np.abs(g) + 1e-8), rtol=1e-14)
    big = np.array([60.0, -80.0, 0.0])
    th, m, v = O.adam_clip_step(np.zeros(3), big, np.zeros(3), np.zeros(3), 1, 0.02, 10.0)
    gc = big * (10.0 / (100.0 + 1e-6))
    assert np.allclose(m, 0.1 * gc, rtol=1e-14) and np.allclose(v, 0.001 * gc * gc, rtol=1e-14)
    g2 = np.array([1.0, 2.0, -1.0])
    th2, m2, v2 = O.adam_clip_step(th, g2, m, v, 2, 0.02, 10.0)
    mm = 0.9 * 0.1 * gc + 0.1 * g2
    vv = 0.999 * 0.001 * gc * gc + 0.001 * g2 * g2
    step = (mm / (1 - 0.9 ** 2)) / (np.sqrt(vv / (1 - 0.999 ** 2)) + 1e-8)
    assert np.allclose(th2, th - 0.02 * step, rtol=1e-13)


def _calib_case(rng, T=2, V=1, H=2, N=12, d=4, dv=3, G=2):
    tr = tuple(_rand(rng, T, H, N, x) for x in (d, d, dv))
    va = tuple(_rand(rng, V, H, N, x) for x in (d, d, dv))
    groups = np.array([np.arange(d) % G, (np.arange(d) + 1) % G])[:H]
    return tr, va, groups


def test_calibrate_fixed_point_of_its_own_kernel():
    """Targets made by the OAL kernel itself at factors L_true: the loss and
    every gradient are zero there, so Adam does not move (0 / (0 + eps)),
    the validation error stays 0, no update improves on update 0, and every
    head stops after exactly `patience` updates."""
    rng = np.random.default_rng(73)
    tr, va, groups = _calib_case(rng)
    Lt = np.stack([np.tril(rng.standard_normal((3, 3))) * 0.7 for _ in range(2)])
    a, b, c = O.coeffs_from_factor(0.01, Lt)
    Yt = O.attention_direct(*tr, groups, a, b, c)
    Yv = O.attention_direct(*va, groups, a, b, c)
    plan = np.array([[u % 2] + list(rng.choice(12, 4, replace=False)) for u in range(30)])
    res = O.calibrate(tr, va, groups, 0.01, Lt[None], plan, validate_every=5, patience=10, targets=(Yt, Yv))
    assert np.array_equal(res["L"], Lt)
    assert (res["mse"] == 0).all() and (res["updates"] == 10).all()


def test_calibrate_selects_best_initial_candidate_at_zero_rate():
    """With lr = 0 the factors never move: each head's checkpoint is its
    initial factors, it stops after `patience` updates, and per head the
    candidate with the lowest initial validation MSE is chosen; the MSE and
    RelMSE are recomputed here from the metric definitions."""
    rng = np.random.default_rng(74)
    tr, va, groups = _calib_case(rng)
    inits = np.stack([np.stack([np.tril(rng.standard_normal((3, 3))) for _ in range(2)]) for _ in range(3)])
    plan = np.array([[u % 2] + list(rng.choice(12, 4, replace=False)) for u in range(40)])
    res = O.calibrate(tr, va, groups, 0.01, inits, plan, lr=0.0, validate_every=5, patience=15)
    Yv = O.softmax_attention(*va)
    mse = np.zeros((3, 2))
    rel = np.zeros((3, 2))
    for ci in range(3):
        a, b, c = O.coeffs_from_factor(0.01, inits[ci])
        Yh = O.attention_direct(*va, groups, a, b, c)
        for h in range(2):
            e = ((Yh[0, h] - Yv[0, h]) ** 2).sum()
            mse[ci, h] = e / Yv[0, h].size
            rel[ci, h] = e / (Yv[0, h] ** 2).sum()
    pick = mse.argmin(axis=0)
    assert np.array_equal(res["init"], pick)
    assert np.allclose(res["mse"], mse[pick, [0, 1]], rtol=1e-12)
    assert np.allclose(res["relmse"], rel[pick, [0, 1]], rtol=1e-12)
    assert (res["updates"] == 15).all()
    for h in range(2):
        assert np.array_equal(res["L"][h], np.tril(inits[pick[h], h]))


def test_calibrate_lowers_validation_error_from_taylor_start():
    """From the second-order Taylor factors (a = 1, b_g = 1, c_gh = 1/2,
    a Cholesky factor of that PSD matrix with a small ridge) on softmax
    targets, the fit ends with a lower validation MSE for every head than the
    starting factors, and early stopping ends it before the plan runs out."""
    rng = np.random.default_rng(75)
    T, H, N, d, dv, G = 2, 2, 24, 4, 3, 2
    tr = tuple(rng.standard_normal((T, H, N, x)) for x in (d, d, dv))
    va = tuple(rng.standard_normal((1, H, N, x)) for x in (d, d, dv))
    groups = np.array([np.arange(d) % G, (np.arange(d) + 1) % G])
    M = np.full((G + 1, G + 1), 0.5)
    M[0, 0] = 1.0
    L0 = np.linalg.cholesky(M + 1e-3 * np.eye(G + 1))
    inits = np.stack([np.stack([L0] * H)])
    plan = np.array([[u % T] + list(rng.choice(N, 8, replace=False)) for u in range(200)])
    res = O.calibrate(tr, va, groups, 1e-3, inits, plan, validate_every=20, patience=80)
    start, _ = O.validation_errors(inits[0], 1e-3, groups, *va, O.softmax_attention(*va))
    assert (res["mse"] < 0.6 * start).all()
    assert (res["updates"] < 200).all()
