"""Output-matching calibration (oal_calibrate) against the oracle's
``calibrate`` ([OAL] App. B, Eq. (20) and its coefficient-calibration
settings), the oracle pinned by the closed forms and finite differences of
its steps.  Both sides take the same inputs, initial factors and sampling
plan; the library runs the targets, forward and backward passes on the GPU in
fp32 and the optimiser in fp32, the oracle everything in fp64, so the two
trajectories agree to about the fp32 rounding of a few hundred Adam steps."""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import log, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _taylor_factor(G):
    """Cholesky factor of the second-order Taylor coefficients (a = 1,
    b_g = 1, c_gh = 1/2) with a small ridge."""
    M = np.full((G + 1, G + 1), 0.5)
    M[0, 0] = 1.0
    return np.linalg.cholesky(M + 1e-3 * np.eye(G + 1))


def _case(dtype, seed, T=3, V=2, H=2, N=96, G=4):
    rng = np.random.default_rng(seed)
    draw = lambda *shape: (S.bf16_round(rng.standard_normal(shape)) if dtype == "bf16"
                           else rng.standard_normal(shape).astype(np.float32)).astype(np.float64)
    # halving keeps bf16 draws bf16-exact
    tr = (draw(T, H, N, 16) * 0.5, draw(T, H, N, 16) * 0.5, draw(T, H, N, 64))
    va = (draw(V, H, N, 16) * 0.5, draw(V, H, N, 16) * 0.5, draw(V, H, N, 64))
    groups = np.stack([rng.permutation(np.arange(16) % G) for _ in range(H)]).astype(np.int32)
    L0 = _taylor_factor(G)
    Lr = np.stack([np.tril(rng.standard_normal((G + 1, G + 1))) * 0.4 + np.eye(G + 1) * 0.6 for _ in range(H)])
    inits = np.stack([np.stack([L0] * H), Lr])
    return tr, va, groups, inits


def _gpu(tr, va, groups, inits, plan, dtype, **kw):
    import grouped_quadratic_softmax_amd as oal
    dev = lambda t: tuple(to_dev(x, dtype) for x in t)
    return oal.calibrate(dev(tr), dev(va), groups, inits, plan, **kw)


def test_calibrate_matches_oracle():
    """fp32 inputs, two candidates (the Taylor factors and a random factor),
    40 updates of 16 positions, validation every 10 with patience 20: the
    chosen candidates, the updates each head ran (early stops included),
    checkpoint MSE / RelMSE and factors agree with the oracle's."""
    require_gpu()
    tr, va, groups, inits = _case("f32", 2201)
    plan = S.calibration_plan(3, 96, 16, 40, seed=2202)
    kw = dict(lr=0.02, clip=10.0, eps=1e-3, validate_every=10, patience=20)
    log("[calib] f32: T=3 V=2 H=2 N=96 G=4, 2 candidates, 40 updates")
    got = _gpu(tr, va, groups, inits, plan, "f32", **kw)
    ref = O.calibrate(tr, va, groups, kw["eps"], inits, plan, lr=kw["lr"], clip=kw["clip"],
                      validate_every=kw["validate_every"], patience=kw["patience"])
    log(f"[calib]   mse gpu {got['mse']} oracle {ref['mse']}; init gpu {got['init']} oracle {ref['init']}")
    log(f"[calib]   max |L - L_ref| {np.abs(got['L'] - ref['L']).max():.3e}; updates {got['updates'].tolist()}")
    assert np.array_equal(got["init"], ref["init"])
    assert np.array_equal(got["updates"], ref["updates"])
    assert np.allclose(got["mse"], ref["mse"], rtol=2e-4)
    assert np.allclose(got["relmse"], ref["relmse"], rtol=2e-4)
    assert np.allclose(got["cand_mse"], ref["cand_mse"], rtol=2e-4)
    assert np.abs(got["L"] - ref["L"]).max() <= 2e-4
    assert (np.triu(got["L"], 1) == 0).all()


def test_calibrate_bf16_reaches_the_oracles_quality():
    """bf16 inputs: the bf16 forward rounds its features and state to bf16,
    so the fit follows a slightly different objective and its trajectory is
    not the oracle's.  What must hold: the factors it picks, evaluated by the
    oracle in fp64, are within 15% of the validation MSE of the oracle's own
    calibration and better than the starting factors, and the MSE the library
    reports for them is the oracle's evaluation of the same factors to 10%."""
    require_gpu()
    tr, va, groups, inits = _case("bf16", 2201)
    plan = S.calibration_plan(3, 96, 16, 40, seed=2202)
    kw = dict(lr=0.02, clip=10.0, eps=1e-3, validate_every=10, patience=20)
    got = _gpu(tr, va, groups, inits, plan, "bf16", **kw)
    ref = O.calibrate(tr, va, groups, kw["eps"], inits, plan, lr=kw["lr"], clip=kw["clip"],
                      validate_every=kw["validate_every"], patience=kw["patience"])
    Yv = O.softmax_attention(*va)
    mine, _ = O.validation_errors(got["L"], kw["eps"], groups, *va, Yv)
    start = np.min([O.validation_errors(inits[c], kw["eps"], groups, *va, Yv)[0] for c in range(2)], axis=0)
    log(f"[calib] bf16: oracle-evaluated {mine}, oracle best {ref['mse']}, start {start}, reported {got['mse']}")
    assert (mine <= 1.15 * ref["mse"]).all()
    assert (mine < start).all()
    assert np.allclose(got["mse"], mine, rtol=0.1)


def test_calibrate_early_stop_and_selection_at_zero_rate():
    """lr = 0: every head keeps its initial factors, stops after `patience`
    updates, and takes the candidate with the lower initial validation MSE,
    which matches the oracle's (fp32 inputs)."""
    require_gpu()
    tr, va, groups, inits = _case("f32", 2203)
    plan = S.calibration_plan(3, 96, 8, 30, seed=2204)
    got = _gpu(tr, va, groups, inits, plan, "f32", lr=0.0, validate_every=5, patience=10)
    ref = O.calibrate(tr, va, groups, 1e-3, inits, plan, lr=0.0, validate_every=5, patience=10)
    assert (got["updates"] == 10).all()
    assert np.array_equal(got["init"], ref["init"])
    for h in range(2):
        assert np.allclose(got["L"][h], np.tril(inits[got["init"][h], h]), rtol=1e-6, atol=1e-7)
    assert np.allclose(got["mse"], ref["mse"], rtol=1e-4)
