"""Shared helpers for the GPU parity tests (no method arithmetic here).

Coefficient maps are taken separately for each side: the oracle maps (eps, L)
with its own fp64 routine, the HIP path with the library's host helper.
"""

from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402

# Tolerances of the parity bar: max relative error (row-infinity normalised)
TOL = {"f32": 2e-3, "bf16": 2e-2}


def torch_mod():
    import torch
    return torch


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def require_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def to_dev(x, dtype_name):
    torch = torch_mod()
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dt).contiguous()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_coeffs(wl):
    if wl.coeff["kind"] == "factor":
        return O.coeffs_from_factor(wl.coeff["eps"], wl.coeff["L"])
    return (np.asarray(wl.coeff["a"], np.float64), np.asarray(wl.coeff["b"], np.float64),
            np.asarray(wl.coeff["c"], np.float64))


def gpu_coeffs(wl, groups):
    import grouped_quadratic_softmax_amd as oal
    if wl.coeff["kind"] == "factor":
        a, b, c = oal.coeffs_from_factor(wl.coeff["eps"], wl.coeff["L"])
    else:
        a, b, c = wl.coeff["a"], wl.coeff["b"], wl.coeff["c"]
    return oal.Coeffs(groups, a, b, c)


def gpu_prep(wl):
    import grouped_quadratic_softmax_amd as oal
    if wl.premap is None:
        return None
    p = wl.premap
    return oal.Prep(p["gamma_q"], p["beta_q"], p["gamma_k"], p["beta_k"], p["ln_eps"], kind=p.get("kind", "layernorm"))


def oracle_prep(wl):
    if wl.premap is None:
        return None
    return {k: (np.asarray(v, np.float64) if not isinstance(v, (float, str)) else v) for k, v in wl.premap.items()}


def with_l2_premap(wl, seed, tau=None):
    """Give workload wl the TaylorShift-style pre-map (unit l2 norm, then the
    affine).  tau given: that baseline's parameters, gamma_q = tau sqrt(d_h),
    gamma_k = 1, beta = 0 (tau per query head); else seeded gamma ~ 1 +
    N(0, 0.1^2) and beta ~ N(0, 0.1^2) per head and dimension."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, d = wl.n_q_heads, wl.n_kv_heads, wl.d_h
    if tau is not None:
        tq = np.broadcast_to(np.asarray(tau, np.float64), (Hq,))
        p = {"gamma_q": np.repeat((tq * np.sqrt(d))[:, None], d, 1), "beta_q": np.zeros((Hq, d)),
             "gamma_k": np.ones((Hkv, d)), "beta_k": np.zeros((Hkv, d))}
    else:
        p = {"gamma_q": 1 + 0.1 * rng.standard_normal((Hq, d)), "beta_q": 0.1 * rng.standard_normal((Hq, d)),
             "gamma_k": 1 + 0.1 * rng.standard_normal((Hkv, d)), "beta_k": 0.1 * rng.standard_normal((Hkv, d))}
    p = {k: v.astype(np.float32).astype(np.float64) for k, v in p.items()}
    p["ln_eps"] = 1e-6
    p["kind"] = "l2"
    wl.premap = p
    return wl


def rel_err(y, ref):
    """max over rows of max_l |y - ref| / max(max_l |ref|, 1e-30) (last axis = l)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(y - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def sample_rows(N, C, n_random, seed):
    """Every chunk's first and last row, the final row and a seeded random set."""
    rng = np.random.default_rng(seed)
    rows = set()
    for start in range(0, N, C):
        rows.add(start)
        rows.add(min(start + C - 1, N - 1))
    rows.add(N - 1)
    rows.update(rng.integers(0, N, size=n_random).tolist())
    return np.array(sorted(rows))


def log(msg):
    print(msg, flush=True)


def diag_form_mask(d, dv):
    """Boolean mask over a packed state block of the entries the dimension-wise
    form reads and writes: rows of the constant, linear and squared features
    (H rows [D][dv], then z [D])."""
    D = O.feature_count(d)
    rows = np.zeros(D, bool)
    rows[: 1 + d] = True
    for r in range(d):
        rows[1 + d + r * d - r * (r - 1) // 2] = True  # pair (r, r) in row-major upper-triangle order
    return np.concatenate([np.repeat(rows, dv), rows])
