"""Plain, slow fp64 CPU oracle for OAL causal attention -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module.  It shares no code with the HIP path and imports nothing from it.

Sources (cited by title and section/equation, never by file position):
  [OAL]     "Not All Dimensions Are Equal: Outlier-Aware Attention Linearization
            with Grouped Quadratic Kernels" (arXiv 2610.13674).
  [Slides]  the research discussion deck on the same paper.
  [ReBased] "Linear Transformers with Learnable Kernel Functions" (blog post).

What is computed (restated, not quoted):
  For a query head h reading KV head h // (Hq/Hkv), a query q and key k:
    x_r   = q_r k_r / sqrt(d_h)                          [OAL] sec. 4.1
    s_g   = sum of x_r over the dimensions r of group g   [OAL] sec. 4.2
    kappa = a + sum_g b_g s_g + sum_{g,h} c_gh s_g s_h    grouped form of the
            dimension-aware kernel ([Slides] "Relax sharing ...", Eq. (3)) with
            b_r = b_g(r) and C_rt = c_g(r)g(t) ([Slides] "A squared quadratic
            form guarantees positive weights").
  Causal normalised output ([OAL] sec. 2, linear attention; causal pair set of
  Eq. (2) includes j = i):
    y_i = sum_{j<=i} kappa(q_i,k_j) v_j / sum_{j<=i} kappa(q_i,k_j)

Forms provided:
  * ``attention_direct``: the definition above, O(N^2) per head (the direct
    pairwise evaluation of [OAL] sec. 4.4).  This is the reference.
  * ``attention_recurrent_packed``: prefix states of [OAL] Eq. (5) stored
    symmetric-packed ([OAL] App. D, "Exact state and parameter counts") and
    read out with Eq. (6).
  * ``attention_recurrent_ordered``: the same with ordered-pair states (full
    d_h x d_h second moment), Eq. (5)-(6) literally.
  * ``chi_bruteforce`` / ``chi_separable``: the contribution score of Eq. (2).

Readings of the pages (listed with reasons in the design notes):
  * The score is scaled by 1/sqrt(d_h) everywhere; the Based polynomial
    1 + t + t^2/2 of [ReBased] is the G = 1 case evaluated at s = t.
  * ReBased's norm(x) is LayerNorm over d_h without its own affine, biased
    variance, epsilon 1e-5, followed by ReBased's gamma/beta.
  * Packed feature order (also the library's state layout): feature 0 is the
    constant, feature 1 + r the linear term r, then the pairs r <= t in
    row-major upper-triangle order.  The state keeps raw Eq. (5) moments;
    multiplicity 2 for r < t and the coefficients belong to the query side.

Parity pins: see tests/test_oracle_pins.py.  Every public function here is
pinned by at least one check that does not reuse this module's arithmetic.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "coeffs_from_factor",
    "premap",
    "group_scores",
    "kappa_from_scores",
    "kappa",
    "attention_direct",
    "attention_backward",
    "feature_count",
    "packed_pairs",
    "phi_k_packed",
    "phi_q_packed",
    "attention_recurrent_packed",
    "attention_recurrent_ordered",
    "state_from_prefix",
    "decode_step",
    "chi_bruteforce",
    "chi_separable",
    "abi_state_from_matrix",
    "matrix_from_abi_state",
    "group_dims_bootstrap",
    "group_dims_budget",
    "groups_sorted_split",
    "softmax_attention",
    "factor_grad",
    "adam_clip_step",
    "validation_errors",
    "calibrate",
]


# --------------------------------------------------------------------------
# coefficients
# --------------------------------------------------------------------------

def coeffs_from_factor(eps, L):
    """(epsilon, L) -> (a, b_g, c_gh) for the positive group-aware kernel.

    [OAL] sec. 4.3, Eq. (7): kappa = eps + sbar^T L L^T sbar with
    sbar = [1, s_1..s_G]; [Slides] "A squared quadratic form guarantees
    positive weights": with M = L L^T, a = eps + M_00, b_g = 2 M_0g and
    c_gh = M_gh.  ``L`` is [H, G+1, G+1] (or [G+1, G+1]).
    """
    L = np.asarray(L, dtype=np.float64)
    single = L.ndim == 2
    if single:
        L = L[None]
    M = np.matmul(L, np.transpose(L, (0, 2, 1)))
    a = eps + M[:, 0, 0]
    b = 2.0 * M[:, 0, 1:]
    c = M[:, 1:, 1:].copy()
    if single:
        return a[0], b[0], c[0]
    return a, b, c


# --------------------------------------------------------------------------
# kernel evaluation
# --------------------------------------------------------------------------

def premap(x, gamma, beta, ln_eps=1e-5, kind="layernorm"):
    """Pre-map gamma * norm(x) + beta along the last axis.

    kind "layernorm": [ReBased] section "Let training place the parabola":
    the feature map is (gamma * norm(x) + beta) squared elementwise; this
    returns the part inside the square.  norm is LayerNorm (mean and biased
    variance over d_h, eps added to the variance).

    kind "l2": the TaylorShift-style map of [OAL] App. F.1 (the TaylorShift
    baseline): queries and keys are scaled to unit l2 norm, norm(x) =
    x / sqrt(sum_r x_r^2 + eps) (reading: eps inside the root, as for
    LayerNorm).  With gamma = tau * sqrt(d_h) on the queries, gamma = 1 on
    the keys and beta = 0, the scaled dot product q~.k~ / sqrt(d_h) is that
    baseline's s = tau * qhat.khat, and a = 1, b = 1, c = 1/2 give its
    polynomial 1 + s + s^2 / 2.
    """
    x = np.asarray(x, dtype=np.float64)
    if kind == "layernorm":
        mu = x.mean(axis=-1, keepdims=True)
        var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
        xn = (x - mu) / np.sqrt(var + ln_eps)
    elif kind == "l2":
        xn = x / np.sqrt((x ** 2).sum(axis=-1, keepdims=True) + ln_eps)
    else:
        raise ValueError(f"unknown pre-map kind {kind!r}")
    return np.asarray(gamma, np.float64) * xn + np.asarray(beta, np.float64)


def _premap_p(x, p, which, head):
    """premap with the parameters of dict p for 'q' or 'k' of one head."""
    return premap(x, p["gamma_" + which][head], p["beta_" + which][head], p["ln_eps"], p.get("kind", "layernorm"))


def group_scores(q, k, group_of_dim, n_groups):
    """Group-restricted scaled dot products s_g for all (query, key) pairs.

    [OAL] sec. 4.2: s_g is the sum over r in group g of q_r k_r / sqrt(d_h).
    q: [n, d], k: [m, d] -> [G, n, m].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    d = q.shape[-1]
    g = np.asarray(group_of_dim)
    out = np.zeros((n_groups, q.shape[0], k.shape[0]))
    for gi in range(n_groups):
        dims = np.nonzero(g == gi)[0]
        if dims.size:
            out[gi] = (q[:, dims] @ k[:, dims].T) / math.sqrt(d)
    return out


def kappa_from_scores(s, a, b, c):
    """kappa = a + sum_g b_g s_g + sum_g sum_h c_gh s_g s_h for score stacks s [G, ...]."""
    G = s.shape[0]
    out = np.full(s.shape[1:], float(a))
    for g in range(G):
        out = out + float(b[g]) * s[g]
    for g in range(G):
        for h in range(G):
            out = out + float(c[g][h]) * s[g] * s[h]
    return out


def kappa(q, k, group_of_dim, a, b, c):
    """Kernel value for one query/key pair (vectors of length d_h)."""
    s = group_scores(np.atleast_2d(q), np.atleast_2d(k), group_of_dim, len(b))
    return float(kappa_from_scores(s, a, b, c)[0, 0])


def _kv_head(h, n_q_heads, n_kv_heads):
    # query heads share KV heads in consecutive blocks (GQA, [OAL] App. B)
    return h // (n_q_heads // n_kv_heads)


def attention_direct(Q, K, V, group_of_dim, a, b, c, premap_params=None, rows=None,
                     return_parts=False):
    """Causal normalised OAL attention by the O(N^2) definition.

    Q: [B, Hq, N, d]; K: [B, Hkv, N, d]; V: [B, Hkv, N, dv]; group_of_dim:
    [Hq, d]; a: [Hq]; b: [Hq, G]; c: [Hq, G, G]; premap_params: None or the
    pre-map {"gamma_q", "beta_q", "gamma_k", "beta_k", "ln_eps"[, "kind"]}
    (kind "layernorm", the default, or "l2"; see ``premap``).
    ``rows``: optional sorted array of output positions (0-based) to evaluate;
    each y_i is computed from its own definition, so any subset is exact.
    Returns y [B, Hq, R, dv] (and num [.., dv], den [..] if return_parts).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    dv = V.shape[-1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    R = rows.size
    y = np.zeros((B, Hq, R, dv))
    num = np.zeros((B, Hq, R, dv))
    den = np.zeros((B, Hq, R))
    causal = (np.arange(N)[None, :] <= rows[:, None])  # j <= i, [R, N]
    for bi in range(B):
        for h in range(Hq):
            kh = _kv_head(h, Hq, Hkv)
            q = Q[bi, h, rows]
            k = K[bi, kh]
            if premap_params is not None:
                p = premap_params
                q = _premap_p(q, p, "q", h)
                k = _premap_p(k, p, "k", kh)
            G = len(b[h])
            s = group_scores(q, k, group_of_dim[h], G)
            w = kappa_from_scores(s, a[h], b[h], c[h]) * causal
            num[bi, h] = w @ V[bi, kh]
            den[bi, h] = w.sum(axis=1)
            y[bi, h] = num[bi, h] / den[bi, h][:, None]
    if return_parts:
        return y, num, den
    return y


# --------------------------------------------------------------------------
# feature-space (HD state) forms
# --------------------------------------------------------------------------

def attention_backward(Q, K, V, dY, group_of_dim, a, b, c):
    """Gradients of sum(dY * y) for the causal normalised attention of
    ``attention_direct`` (no pre-map), by the chain rule on its definition.

    The backward pass the calibration of [OAL] App. B (Eq. (20), the
    output-matching fit of L) and the joint adaptation of App. F.2 need:
        y_i = num_i / den_i,  num_i = sum_{j<=i} kappa_ij v_j,  den_i = sum_{j<=i} kappa_ij
        dnum_i = dY_i / den_i,  dden_i = -(dY_i . y_i) / den_i
        dkappa_ij = [j <= i] (dnum_i . v_j + dden_i)
        dV_j = sum_i kappa_ij dnum_i
        dkappa/ds_g = b_g + sum_h (c_gh + c_hg) s_h
        dQ_ir = sum_j dkappa_ij (dkappa/ds_g(r))_ij k_jr / sqrt(d)   (dK likewise with q_ir)
        da = sum dkappa,  db_g = sum dkappa s_g,  dc_gh = sum dkappa s_g s_h
    (the coefficient gradients summed over the batch).  Q, K, V, dY as in
    ``attention_direct`` (dY: [B, Hq, N, dv]).  Returns dQ, dK, dV (fp64, the
    input shapes), da [Hq], db [Hq, G], dc [Hq, G, G].
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dY = np.asarray(dY, np.float64)
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    G = len(b[0])
    da, db, dc = np.zeros(Hq), np.zeros((Hq, G)), np.zeros((Hq, G, G))
    causal = np.tril(np.ones((N, N)))
    for bi in range(B):
        for h in range(Hq):
            kh = _kv_head(h, Hq, Hkv)
            q, k, v = Q[bi, h], K[bi, kh], V[bi, kh]
            gd = np.asarray(group_of_dim[h])
            s = group_scores(q, k, gd, G)
            w = kappa_from_scores(s, a[h], b[h], c[h]) * causal
            num, den = w @ v, w.sum(axis=1)
            y = num / den[:, None]
            dnum = dY[bi, h] / den[:, None]
            dden = -(dY[bi, h] * y).sum(axis=1) / den
            dk = (dnum @ v.T + dden[:, None]) * causal
            dV[bi, kh] += w.T @ dnum
            cs = np.asarray(c[h], np.float64)
            for g in range(G):
                dks = float(b[h][g]) + sum((cs[g, hh] + cs[hh, g]) * s[hh] for hh in range(G))
                m = dk * dks
                dims = np.nonzero(gd == g)[0]
                dQ[bi, h][:, dims] += (m @ k[:, dims]) / math.sqrt(d)
                dK[bi, kh][:, dims] += (m.T @ q[:, dims]) / math.sqrt(d)
                db[h, g] += (dk * s[g]).sum()
                for hh in range(G):
                    dc[h, g, hh] += (dk * s[g] * s[hh]).sum()
            da[h] += dk.sum()
    return dQ, dK, dV, da, db, dc


def feature_count(d):
    """Packed feature count 1 + d + d(d+1)/2 ([OAL] App. D)."""
    return 1 + d + d * (d + 1) // 2


def packed_pairs(d):
    """List of (r, t), r <= t, in row-major upper-triangle order."""
    return [(r, t) for r in range(d) for t in range(r, d)]


def phi_k_packed(k):
    """Key features [1, k_r, k_r k_t (r <= t)] ([OAL] Eq. (5) moments, packed)."""
    k = np.asarray(k, np.float64)
    d = k.shape[-1]
    f = [np.ones(k.shape[:-1])]
    f += [k[..., r] for r in range(d)]
    f += [k[..., r] * k[..., t] for (r, t) in packed_pairs(d)]
    return np.stack(f, axis=-1)


def phi_q_packed(q, group_of_dim, a, b, c):
    """Query features carrying the coefficients of [OAL] Eq. (6).

    [a, b_g(r) q_r / sqrt(d), m_rt c_g(r)g(t) q_r q_t / d] with multiplicity
    m_rt = 1 on the diagonal and 2 off it ([OAL] App. D, packed readout).
    """
    q = np.asarray(q, np.float64)
    d = q.shape[-1]
    g = np.asarray(group_of_dim)
    sd = math.sqrt(d)
    f = [np.full(q.shape[:-1], float(a))]
    f += [float(b[g[r]]) * q[..., r] / sd for r in range(d)]
    for (r, t) in packed_pairs(d):
        m = 1.0 if r == t else 2.0
        f.append(m * float(c[g[r]][g[t]]) * q[..., r] * q[..., t] / d)
    return np.stack(f, axis=-1)


def attention_recurrent_packed(Q, K, V, group_of_dim, a, b, c, premap_params=None,
                               state_in=None, return_state=False):
    """Causal attention through packed prefix states, token by token.

    State per (batch, KV head): S [D, dv+1] = sum_j phi_k(k_j) [v_j, 1]^T
    ([OAL] Eq. (5) with u_j = [v_j; 1]); readout u~_i = phi_q(q_i)^T S_i and
    y_i = u~_i[:dv] / u~_i[dv] ([OAL] Eq. (6)).  ``state_in``: [B, Hkv, D, dv+1]
    initial states (zeros if None).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    dv = V.shape[-1]
    D = feature_count(d)
    S = np.zeros((B, Hkv, D, dv + 1)) if state_in is None else np.array(state_in, np.float64)
    y = np.zeros((B, Hq, N, dv))
    for bi in range(B):
        for kh in range(Hkv):
            heads = [h for h in range(Hq) if _kv_head(h, Hq, Hkv) == kh]
            k = K[bi, kh]
            if premap_params is not None:
                p = premap_params
                k = _premap_p(k, p, "k", kh)
            fk = phi_k_packed(k)
            fq = {}
            for h in heads:
                q = Q[bi, h]
                if premap_params is not None:
                    q = _premap_p(q, premap_params, "q", h)
                fq[h] = phi_q_packed(q, group_of_dim[h], a[h], b[h], c[h])
            st = S[bi, kh]
            for i in range(N):
                u = np.concatenate([V[bi, kh, i], [1.0]])
                st += np.outer(fk[i], u)
                for h in heads:
                    ut = fq[h][i] @ st
                    y[bi, h, i] = ut[:dv] / ut[dv]
    if return_state:
        return y, S
    return y


def attention_recurrent_ordered(Q, K, V, group_of_dim, a, b, c):
    """Eq. (5)-(6) of [OAL] with ordered-pair states (no packing).

    H0 = sum u_j, H1_r = sum k_jr u_j, H2_rt = sum k_jr k_jt u_j over j <= i;
    u~_i = a H0 + (1/sqrt d) sum_r b_r q_r H1_r + (1/d) sum_{r,t} C_rt q_r q_t H2_rt
    with b_r = b_g(r), C_rt = c_g(r)g(t).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    dv = V.shape[-1]
    y = np.zeros((B, Hq, N, dv))
    for bi in range(B):
        for h in range(Hq):
            kh = _kv_head(h, Hq, Hkv)
            g = np.asarray(group_of_dim[h])
            br = np.array([b[h][g[r]] for r in range(d)], dtype=np.float64)
            C = np.array([[c[h][g[r]][g[t]] for t in range(d)] for r in range(d)], dtype=np.float64)
            H0 = np.zeros(dv + 1)
            H1 = np.zeros((d, dv + 1))
            H2 = np.zeros((d, d, dv + 1))
            for i in range(N):
                kk = K[bi, kh, i]
                u = np.concatenate([V[bi, kh, i], [1.0]])
                H0 += u
                H1 += np.outer(kk, u)
                H2 += np.einsum("r,t,l->rtl", kk, kk, u)
                q = Q[bi, h, i]
                ut = a[h] * H0
                ut = ut + np.einsum("r,rl->l", br * q, H1) / math.sqrt(d)
                ut = ut + np.einsum("rt,r,t,rtl->l", C, q, q, H2) / d
                y[bi, h, i] = ut[:dv] / ut[dv]
    return y


def state_from_prefix(K, V, premap_k=None, ln_eps=1e-5, kind="layernorm"):
    """Packed state sum_j phi_k(k_j) [v_j, 1]^T of one (sequence, KV head).

    K: [n, d], V: [n, dv]; premap_k: optional (gamma_k, beta_k) for the
    ReBased pre-map.  Returns [D, dv+1].
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if premap_k is not None:
        K = premap(K, premap_k[0], premap_k[1], ln_eps, kind)
    fk = phi_k_packed(K)
    U = np.concatenate([V, np.ones((V.shape[0], 1))], axis=1)
    return fk.T @ U


def decode_step(state, q, k, v, group_of_dim, a, b, c, n_q_heads, premap_params=None):
    """One recurrent decode step ([OAL] Eq. (5)-(6) for a single new token).

    state: [S, Hkv, D, dv+1] (fp64, updated copy returned); q: [S, Hq, d];
    k: [S, Hkv, d]; v: [S, Hkv, dv].  The new token is part of its own causal
    prefix (j <= i), so the state is updated before the readout.
    Returns (y [S, Hq, dv], new_state).
    """
    st = np.array(state, np.float64)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S, Hkv = k.shape[0], k.shape[1]
    dv = v.shape[-1]
    y = np.zeros((S, n_q_heads, dv))
    for s in range(S):
        for kh in range(Hkv):
            kk = k[s, kh]
            if premap_params is not None:
                p = premap_params
                kk = _premap_p(kk, p, "k", kh)
            st[s, kh] += np.outer(phi_k_packed(kk), np.concatenate([v[s, kh], [1.0]]))
        for h in range(n_q_heads):
            kh = _kv_head(h, n_q_heads, Hkv)
            qq = q[s, h]
            if premap_params is not None:
                p = premap_params
                qq = _premap_p(qq, p, "q", h)
            ut = phi_q_packed(qq, group_of_dim[h], a[h], b[h], c[h]) @ st[s, kh]
            y[s, h] = ut[:dv] / ut[dv]
    return y, st


def abi_state_from_matrix(S):
    """[..., D, dv+1] -> flat library layout [..., D*dv + D]: H rows then z."""
    S = np.asarray(S)
    H = S[..., :-1]
    z = S[..., -1]
    return np.concatenate([H.reshape(H.shape[:-2] + (-1,)), z], axis=-1)


def matrix_from_abi_state(flat, D, dv):
    """Inverse of abi_state_from_matrix."""
    flat = np.asarray(flat)
    H = flat[..., : D * dv].reshape(flat.shape[:-1] + (D, dv))
    z = flat[..., D * dv:]
    return np.concatenate([H, z[..., None]], axis=-1)


# --------------------------------------------------------------------------
# contribution score (Eq. (2))
# --------------------------------------------------------------------------

def chi_bruteforce(Q, K, lengths=None):
    """chi_{p,r} and chi_r by the definition of [OAL] Eq. (2).

    chi_{p,r} = mean over causal pairs j <= i < N_p of |q_ir k_jr| / sqrt(d);
    chi_r = equal-weight mean over prompts p.  Query head h uses KV head
    h // (Hq/Hkv) (the native GQA map, [OAL] App. B).  Q: [P, Hq, N, d],
    K: [P, Hkv, N, d]; lengths: [P] (default N).  O(N^2 d): tiny inputs only.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    P, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    lengths = np.full(P, N) if lengths is None else np.asarray(lengths)
    per = np.zeros((P, Hq, d))
    for p in range(P):
        n = int(lengths[p])
        pairs = [(i, j) for i in range(n) for j in range(i + 1)]
        for h in range(Hq):
            kh = _kv_head(h, Hq, Hkv)
            for r in range(d):
                tot = 0.0
                for (i, j) in pairs:
                    tot += abs(Q[p, h, i, r] * K[p, kh, j, r]) / math.sqrt(d)
                per[p, h, r] = tot / len(pairs)
    return per, per.mean(axis=0)


def chi_separable(Q, K, lengths=None):
    """Same quantity as chi_bruteforce, summed as sum_i |q_ir| * sum_{j<=i} |k_jr|."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    P, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    lengths = np.full(P, N) if lengths is None else np.asarray(lengths)
    per = np.zeros((P, Hq, d))
    for p in range(P):
        n = int(lengths[p])
        npairs = n * (n + 1) / 2.0
        for h in range(Hq):
            kh = _kv_head(h, Hq, Hkv)
            pre = np.cumsum(np.abs(K[p, kh, :n]), axis=0)
            per[p, h] = (np.abs(Q[p, h, :n]) * pre).sum(axis=0) / (math.sqrt(d) * npairs)
    return per, per.mean(axis=0)


# --------------------------------------------------------------------------
# outlier-aware dimension grouping ([OAL] App. B, "Dimension grouping")
# --------------------------------------------------------------------------

def _sorted_order(chi):
    """pi: dimension indices by ascending chi, ties kept in index order (a
    stable sort, [OAL] App. B)."""
    return sorted(range(len(chi)), key=lambda r: chi[r])


def _groups_from_cuts(pi, cuts):
    """Group id of every dimension for retained cuts k_1 < ... < k_{G-1}:
    group g (0-based) holds sorted positions k_{g-1}+1 .. k_g (1-based
    positions, k_0 = 0, k_G = d_h), mapped back to dimension indices."""
    d = len(pi)
    bounds = [0] + sorted(cuts) + [d]
    gid = [0] * d
    for g in range(len(bounds) - 1):
        for pos in range(bounds[g], bounds[g + 1]):
            gid[pi[pos]] = g
    return gid


def group_dims_bootstrap(chi_pp, boot, alpha, gamma, tau=1.5, g_min=2, eps=1e-12):
    """Outlier-aware grouping of one query head ([OAL] App. B).

    chi_pp: [P][d] per-prompt contribution scores chi_{p,r} (Eq. (2)).
    boot:   [B][P] prompt indices of the B bootstrap replicates (drawn with
            replacement by the caller; repeated indices count repeatedly).
    Steps, in the appendix's order:
      1. chi_r = equal-weight mean over prompts; pi = stable ascending order.
      2. m = ceil(alpha d); candidate cuts k = d - m .. d - 1 (and k >= 1), a
         cut at k separating sorted positions 1..k from k+1..d.
      3. rho_k = chi_{pi_{k+1}} / max(chi_{pi_k}, eps).
      4. per replicate b, chi^(b) = mean of chi_p over the sampled prompts (pi
         kept fixed); R_k^(b) = min over the upper side of chi^(b) / max(max
         over the lower side of chi^(b), eps) (the deck's backup slide on
         bootstrap support); S_k = fraction of replicates with R_k^(b) >= tau.
      5. natural cuts: rho_k >= tau and S_k >= gamma.
      6. fewer than g_min groups: add unused candidates in descending
         lexicographic order of (S_k, rho_k), ties in candidate order, until
         g_min groups or no candidate is left.
      7. groups = contiguous runs of the sorted order between the cuts.
    Returns (group id per dimension, G, {k: rho_k}, {k: S_k}), in fp64.
    """
    P = len(chi_pp)
    d = len(chi_pp[0])
    chi = []
    for r in range(d):
        tot = 0.0
        for p in range(P):
            tot += float(chi_pp[p][r])
        chi.append(tot / P)
    pi = _sorted_order(chi)
    m = math.ceil(alpha * d)
    cands = [k for k in range(d - m, d) if k >= 1]
    rho, sup = {}, {}
    for k in cands:
        rho[k] = chi[pi[k]] / max(chi[pi[k - 1]], eps)  # 1-based pi_{k+1} / pi_k
    counts = {k: 0 for k in cands}
    for idx in boot:
        chib = []
        for r in range(d):
            tot = 0.0
            for i in idx:
                tot += float(chi_pp[int(i)][r])
            chib.append(tot / len(idx))
        for k in cands:
            lo = max(chib[pi[pos]] for pos in range(k))
            up = min(chib[pi[pos]] for pos in range(k, d))
            if up / max(lo, eps) >= tau:
                counts[k] += 1
    for k in cands:
        sup[k] = counts[k] / len(boot)
    cuts = [k for k in cands if rho[k] >= tau and sup[k] >= gamma]
    if len(cuts) + 1 < g_min:
        rest = [k for k in cands if k not in cuts]
        rest = sorted(rest, key=lambda k: (-sup[k], -rho[k]))  # stable: ties in candidate order
        for k in rest:
            if len(cuts) + 1 >= g_min:
                break
            cuts.append(k)
    gid = _groups_from_cuts(pi, cuts)
    return gid, len(cuts) + 1, rho, sup


def group_dims_budget(chi, n_groups, eps=1e-12):
    """Fixed-budget grouping ([OAL] App. B, "Group-budget diagnostic"): the
    G - 1 largest adjacent gaps of the stably sorted profile become the
    boundaries.  The gap at cut k is the appendix's adjacent contribution gap
    rho_k = chi_{pi_{k+1}} / max(chi_{pi_k}, eps), over every k = 1..d-1;
    equal gaps are taken in cut order.  Returns (group id per dimension, rho)."""
    d = len(chi)
    chi = [float(x) for x in chi]
    pi = _sorted_order(chi)
    rho = {k: chi[pi[k]] / max(chi[pi[k - 1]], eps) for k in range(1, d)}
    order = sorted(range(1, d), key=lambda k: -rho[k])  # stable
    cuts = order[:n_groups - 1]
    return _groups_from_cuts(pi, cuts), rho


def groups_sorted_split(chi, bulk_sizes, n_tail):
    """Contribution-sorted split with a fixed group budget, one head at a time.

    The grouping of the long-context workload: [OAL] sec. 4.2 and App. B sort
    the dimensions of a head by ascending chi_r (Eq. (2)) with a stable sort
    (equal scores keep index order) and place the boundaries in that order.
    Here the budget is fixed: the last ``n_tail`` sorted positions become
    singleton groups and the rest, still in sorted order, are cut into
    contiguous runs of ``bulk_sizes``.  Group ids: 0, 1, ... for the bulk runs
    (lowest contribution first), then the tail singletons in ascending chi.

    chi: [H][d] scores -> [H][d] group ids (pure Python loops).
    """
    out = []
    for row in chi:
        d = len(row)
        if sum(bulk_sizes) + n_tail != d:
            raise ValueError("bulk sizes plus tail must cover the head dimensions")
        pi = _sorted_order([float(x) for x in row])
        gid = [0] * d
        pos = 0
        for g, size in enumerate(bulk_sizes):
            for _ in range(size):
                gid[pi[pos]] = g
                pos += 1
        for i in range(n_tail):
            gid[pi[pos]] = len(bulk_sizes) + i
            pos += 1
        out.append(gid)
    return np.array(out, dtype=np.int64)


# --------------------------------------------------------------------------
# output-matching calibration of the factors ([OAL] App. B, Eq. (20) and
# "Coefficient-calibration settings")
# --------------------------------------------------------------------------

def softmax_attention(Q, K, V):
    """Causal softmax attention, the calibration target y^softmax of [OAL]
    Eq. (20): y_i = sum_{j<=i} w_ij v_j with w_ij proportional to
    exp(q_i . k_j / sqrt(d_h)) over the causal prefix.  fp64; shapes as in
    ``attention_direct`` (query head h reads KV head h // (Hq / Hkv))."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    out = np.zeros((B, Hq, N, V.shape[3]))
    mask = np.tril(np.ones((N, N), bool))
    for bi in range(B):
        for h in range(Hq):
            kh = _kv_head(h, Hq, Hkv)
            s = (Q[bi, h] @ K[bi, kh].T) / math.sqrt(d)
            s = np.where(mask, s, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            out[bi, h] = (w @ V[bi, kh]) / w.sum(axis=1, keepdims=True)
    return out


def factor_grad(L, da, db, dc):
    """Gradient with respect to the factor L (lower triangle, [G+1, G+1]) of
    an objective that depends on L only through (a, b, c) =
    ``coeffs_from_factor(eps, L)``, given its gradients da, db [G], dc [G, G].
    With M = L L^T, a = eps + M_00, b_g = 2 M_0g, c_gh = M_gh, the objective
    reads the entries Mbar = [[da, 2 db^T], [0, dc]] of M, and
    d/dL = (Mbar + Mbar^T) L restricted to the lower triangle."""
    L = np.tril(np.asarray(L, np.float64))
    G = len(db)
    Mbar = np.zeros((G + 1, G + 1))
    Mbar[0, 0] = da
    Mbar[0, 1:] = 2.0 * np.asarray(db, np.float64)
    Mbar[1:, 1:] = np.asarray(dc, np.float64)
    return np.tril((Mbar + Mbar.T) @ L)


def adam_clip_step(theta, grad, m, v, t, lr, clip, beta1=0.9, beta2=0.999, eps=1e-8):
    """One Adam update of the parameter vector theta (the settings' optimiser:
    Adam at learning rate lr, gradient norm clipped at clip).  The gradient is
    first scaled by clip / (||grad|| + 1e-6) when its norm exceeds clip; then
    the bias-corrected moments of step t (t >= 1) give
    theta - lr * mhat / (sqrt(vhat) + eps).  Returns (theta, m, v)."""
    grad = np.asarray(grad, np.float64)
    norm = float(np.sqrt((grad * grad).sum()))
    if norm > clip:
        grad = grad * (clip / (norm + 1e-6))
    m = beta1 * m + (1.0 - beta1) * grad
    v = beta2 * v + (1.0 - beta2) * grad * grad
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    return theta - lr * mhat / (np.sqrt(vhat) + eps), m, v


def _tril_index(n):
    return np.tril_indices(n)


def validation_errors(L, eps, group_of_dim, Qv, Kv, Vv, Yv):
    """Per-head MSE and RelMSE of the OAL outputs with factors L [H, G+1, G+1]
    against the targets Yv over whole validation sequences ([OAL] metric
    definitions: the mean over sequences of ||Yhat_b - Y_b||_F^2 / n_b, n_b
    the scalar output elements, and of ||Yhat_b - Y_b||_F^2 / ||Y_b||_F^2)."""
    a, b, c = coeffs_from_factor(eps, L)
    Yh = attention_direct(Qv, Kv, Vv, group_of_dim, a, b, c)
    err = ((Yh - Yv) ** 2).sum(axis=(2, 3))      # [V, H]
    n = Yv.shape[2] * Yv.shape[3]
    mse = (err / n).mean(axis=0)
    rel = (err / (Yv ** 2).sum(axis=(2, 3))).mean(axis=0)
    return mse, rel


def calibrate(train, val, group_of_dim, eps, inits, plan, lr=0.02, clip=10.0, validate_every=100,
              patience=400, targets=None):
    """Output-matching calibration of the factors L of every head ([OAL]
    App. B, Eq. (20)), following the coefficient-calibration settings: Adam
    at lr, gradient norm clipped at clip, one training sequence and the
    sampled causal query positions per update, validation every
    ``validate_every`` updates, early stop after ``patience`` updates without
    improvement, the lowest-validation-MSE checkpoint kept per head within
    each initialisation candidate and the best candidate chosen per head.

    Readings (the settings leave them open): each head is its own objective
    and optimiser (independent coefficients per head; its gradient norm is
    clipped alone and it stops alone); an update's objective is the mean over
    its sampled positions of ||yhat_i - y_i||^2; validation runs on whole
    sequences, also before the first update (update 0), so the initial
    factors are a checkpoint; every candidate follows the same plan.

    train, val: (Q, K, V) arrays [T, H, N, d] / [V, H, N, d] (heads with their
    own keys); inits [n_init, H, G+1, G+1]; plan [U, 1 + P] int: per update,
    the training sequence and P distinct positions.  targets: optional
    (Y_train, Y_val) in place of the softmax outputs.  Returns a dict with
    the chosen factors "L" [H, G+1, G+1], "mse", "relmse", "init" [H], and per
    candidate "cand_mse" [n_init, H], "cand_L", "updates" [n_init, H] (the
    updates each head ran)."""
    Qt, Kt, Vt = (np.asarray(x, np.float64) for x in train)
    Qv, Kv, Vv = (np.asarray(x, np.float64) for x in val)
    inits = np.asarray(inits, np.float64)
    plan = np.asarray(plan)
    n_init, H, n, _ = inits.shape
    G = n - 1
    if targets is None:
        Yt, Yv = softmax_attention(Qt, Kt, Vt), softmax_attention(Qv, Kv, Vv)
    else:
        Yt, Yv = (np.asarray(x, np.float64) for x in targets)
    ti = _tril_index(n)
    cand_mse = np.zeros((n_init, H))
    cand_rel = np.zeros((n_init, H))
    cand_L = np.zeros((n_init, H, n, n))
    cand_upd = np.zeros((n_init, H), np.int64)
    for ci in range(n_init):
        L = np.stack([np.tril(inits[ci, h]) for h in range(H)])
        m = np.zeros((H, len(ti[0])))
        v = np.zeros((H, len(ti[0])))
        best, best_rel = validation_errors(L, eps, group_of_dim, Qv, Kv, Vv, Yv)
        best_L = L.copy()
        last = np.zeros(H, np.int64)
        active = np.ones(H, bool)
        done = np.zeros(H, np.int64)
        for u in range(1, len(plan) + 1):
            if not active.any():
                break
            seq, pos = int(plan[u - 1, 0]), np.asarray(plan[u - 1, 1:])
            a, b, c = coeffs_from_factor(eps, L)
            sl = slice(seq, seq + 1)
            y = attention_direct(Qt[sl], Kt[sl], Vt[sl], group_of_dim, a, b, c)
            dY = np.zeros_like(y)
            dY[0][:, pos] = 2.0 * (y[0][:, pos] - Yt[seq][:, pos]) / len(pos)
            _, _, _, da, db, dc = attention_backward(Qt[sl], Kt[sl], Vt[sl], dY, group_of_dim, a, b, c)
            for h in range(H):
                if not active[h]:
                    continue
                gL = factor_grad(L[h], da[h], db[h], dc[h])
                th, m[h], v[h] = adam_clip_step(L[h][ti], gL[ti], m[h], v[h], u, lr, clip)
                L[h][ti] = th
                done[h] = u
            if u % validate_every == 0:
                mse, rel = validation_errors(L, eps, group_of_dim, Qv, Kv, Vv, Yv)
                for h in range(H):
                    if not active[h]:
                        continue
                    if mse[h] < best[h]:
                        best[h], best_rel[h], best_L[h], last[h] = mse[h], rel[h], L[h], u
                    elif u - last[h] >= patience:
                        active[h] = False
        cand_mse[ci], cand_rel[ci], cand_L[ci], cand_upd[ci] = best, best_rel, best_L, done
    pick = cand_mse.argmin(axis=0)
    hs = np.arange(H)
    return {"L": cand_L[pick, hs], "mse": cand_mse[pick, hs], "relmse": cand_rel[pick, hs], "init": pick,
            "cand_mse": cand_mse, "cand_L": cand_L, "updates": cand_upd}
