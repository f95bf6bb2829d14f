"""Host-side checks of the C ABI: the library loads, exports every declared
entry point, and its host helpers and argument validation behave as
documented.  No call here reaches a GPU: every error path returns before any
launch."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oal.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def L():
    from grouped_quadratic_softmax_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from grouped_quadratic_softmax_amd.build import build
        build()
    return _lib


def declared_functions(headers=(HEADER,)):
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(oal_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("oal_fwd", "oal_decode_step", "oal_contrib"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    names = declared_functions(HEADERS)
    assert "oal_ceiling_stream_rw" in names and "oal_ceiling_mfma" in names
    for name in names:
        assert hasattr(lib, name), name


def test_versions_and_counts(L):
    lib = L.lib()
    assert b"gfx950" in lib.oal_version()
    assert L.status_str(L.OAL_ERR_WORKSPACE) == "OAL_ERR_WORKSPACE"
    for d in (16, 32, 64):
        assert lib.oal_feature_count(d) == O.feature_count(d)
        assert lib.oal_state_floats(d, 64) == O.feature_count(d) * 65
    assert lib.oal_state_floats(64, 64) == 139425  # OAL slides, state-size slide


def test_coeffs_from_factor_matches_oracle(L):
    import grouped_quadratic_softmax_amd as oal
    rng = np.random.default_rng(3)
    for G in (1, 4, 8):
        Lf = np.tril(rng.uniform(-1, 1, size=(3, G + 1, G + 1)))
        a, b, c = oal.coeffs_from_factor(1e-3, Lf)
        ao, bo, co = O.coeffs_from_factor(1e-3, Lf)
        assert np.allclose(a, ao, rtol=1e-6) and np.allclose(b, bo, rtol=1e-6, atol=1e-7)
        assert np.allclose(c, co, rtol=1e-6, atol=1e-7)


def _dims(L, B=1, Hq=2, Hkv=1, N=8, d=64, dv=64, G=2, dt=1):
    return L.OalDims(B, Hq, Hkv, N, d, dv, G, dt)


def test_check_coeffs(L):
    lib = L.lib()
    d = _dims(L)
    g = np.zeros((2, 64), np.int32)
    c = np.ones((2, 2, 2), np.float32)
    vp = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    assert lib.oal_check_coeffs(ctypes.byref(d), vp(g), vp(c)) == L.OAL_OK
    g[1, 7] = 2
    assert lib.oal_check_coeffs(ctypes.byref(d), vp(g), vp(c)) == L.OAL_ERR_INVALID_ARG
    g[1, 7] = -1
    assert lib.oal_check_coeffs(ctypes.byref(d), vp(g), vp(c)) == L.OAL_ERR_INVALID_ARG
    g[1, 7] = 0
    c[0, 1, 0] = np.inf
    assert lib.oal_check_coeffs(ctypes.byref(d), vp(g), vp(c)) == L.OAL_ERR_INVALID_ARG
    with pytest.raises(L.OalError):
        import grouped_quadratic_softmax_amd as oal
        oal.Coeffs(np.full((1, 64), 3, np.int32), [1.0], [[1.0, 1.0]], [[[1, 0], [0, 1]]], device="cpu")


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation first


@pytest.fixture
def no_device():
    """The validation tests below pass fake device pointers that every check
    must reject before anything is enqueued.  Where a GPU is visible, a
    regression in one of those checks would launch a kernel on them, so these
    tests run only where no device is visible (the CPU suite)."""
    try:
        import torch
        if torch.cuda.device_count() > 0:
            pytest.skip("fake-pointer validation runs only without a visible GPU")
    except ImportError:
        pass


def _mis(off):
    """A fake device pointer off the 16-byte grid."""
    return ctypes.c_void_p(0x1000 + off)


def _fwd(L, dims, coeffs=True, ws=(FAKE, 1 << 40), q=FAKE, y=FAKE, state_in=None, state_out=None, prep=None):
    lib = L.lib()
    cs = L.OalCoeffs(0x1000, 0x1000, 0x1000, 0x1000) if coeffs else None
    return lib.oal_fwd(ctypes.byref(dims) if dims is not None else None, q, FAKE, FAKE,
                       ctypes.byref(cs) if cs is not None else None,
                       ctypes.byref(prep) if prep is not None else None, state_in, state_out, y, ws[0],
                       ctypes.c_size_t(ws[1]), None)


def test_fwd_validation_errors(L, no_device):
    E, U, W = L.OAL_ERR_INVALID_ARG, L.OAL_ERR_UNSUPPORTED, L.OAL_ERR_WORKSPACE
    assert _fwd(L, None) == E
    assert _fwd(L, _dims(L, Hq=3, Hkv=2)) == E           # Hq % Hkv
    assert _fwd(L, _dims(L, N=-1)) == E
    assert _fwd(L, _dims(L, B=-1)) == E
    assert _fwd(L, _dims(L, dt=7)) == E
    assert _fwd(L, _dims(L, d=48)) == U                  # unsupported head dim
    assert _fwd(L, _dims(L, dv=32)) == U
    assert _fwd(L, _dims(L, G=0)) == E
    assert _fwd(L, _dims(L, G=65)) == E
    assert _fwd(L, _dims(L, G=9)) == U
    # more than eight groups: only the one-wave d_h = 16 build (heads with
    # their own keys, bf16, no pre-map) takes them
    assert _fwd(L, _dims(L, d=16, Hq=4, Hkv=2, G=9)) == U
    assert _fwd(L, _dims(L, d=16, G=9, dt=0)) == U
    assert _fwd(L, _dims(L), coeffs=False) == E
    assert _fwd(L, _dims(L), q=None) == E
    assert _fwd(L, _dims(L), y=None) == E
    assert _fwd(L, _dims(L), ws=(None, 0)) == W
    need = L.lib().oal_fwd_workspace_bytes(ctypes.byref(_dims(L)))
    assert need > 0
    assert _fwd(L, _dims(L), ws=(FAKE, need - 1)) == W
    assert _fwd(L, _dims(L), state_in=FAKE, state_out=FAKE) == E  # aliasing
    assert _fwd(L, _dims(L), q=_mis(2)) == E                      # 16-byte alignment
    assert _fwd(L, _dims(L), y=_mis(8)) == E
    assert _fwd(L, _dims(L), state_out=_mis(4)) == E
    bad_prep = L.OalPrep(0x1000, 0, 0x1000, 0x1000, 1e-5)
    assert _fwd(L, _dims(L), prep=bad_prep) == E
    # per-sequence lengths: a null length array is refused before any launch
    lib = L.lib()
    cs = L.OalCoeffs(0x1000, 0x1000, 0x1000, 0x1000)
    assert lib.oal_fwd_varlen(ctypes.byref(_dims(L)), None, FAKE, FAKE, FAKE, ctypes.byref(cs), None, None, None,
                              FAKE, FAKE, ctypes.c_size_t(need), None) == E
    assert lib.oal_fwd_varlen_workspace_bytes_for(ctypes.byref(_dims(L)), ctypes.byref(cs)) == need
    for kind in (-1, 2):  # pre-map kinds: 0 LayerNorm, 1 unit l2 norm
        assert _fwd(L, _dims(L), prep=L.OalPrep(0x1000, 0x1000, 0x1000, 0x1000, 1e-5, kind)) == E
    assert _fwd(L, _dims(L, B=0)) == L.OAL_OK                     # empty batch: nothing enqueued


def test_workspace_sizes(L):
    lib = L.lib()
    # one internal snapshot per 64-token chunk and (batch, KV head), bf16
    d = _dims(L, B=4, Hq=14, Hkv=2, N=2048, G=4)
    # one fp16 snapshot of 70 K-blocks x 65 columns x 32 features per (chunk,
    # sequence, KV head), plus small per-snapshot exponent and constant rows
    snaps = 32 * 8
    snap_bytes = snaps * 70 * 65 * 32 * 2
    got = lib.oal_fwd_workspace_bytes(ctypes.byref(d))
    # plus per-head coefficient tables (14 heads x 70 x 32 fp16 + small rows)
    small = snaps * (72 + 65 + 2) * 4 + 14 * (70 * 32 * 2 + 73 * 4 + 4) + 6 * 256
    assert snap_bytes <= got <= snap_bytes + small
    assert lib.oal_fwd_workspace_bytes(None) == 0
    assert lib.oal_contrib_workspace_bytes(ctypes.byref(_dims(L, B=2, N=3000))) > 0


def test_decode_and_contrib_validation(L, no_device):
    lib = L.lib()
    cs = L.OalCoeffs(0x1000, 0x1000, 0x1000, 0x1000)
    d = _dims(L, B=2)
    z = ctypes.c_size_t(0)
    assert lib.oal_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None, z, None) == \
        L.OAL_ERR_INVALID_ARG
    assert lib.oal_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(cs), None, None, FAKE, None, z,
                               None) == L.OAL_ERR_INVALID_ARG
    assert lib.oal_decode_step(ctypes.byref(_dims(L, Hq=18, Hkv=2)), FAKE, FAKE, FAKE, ctypes.byref(cs), None,
                               FAKE, FAKE, None, z, None) == L.OAL_ERR_UNSUPPORTED
    assert lib.oal_decode_step(ctypes.byref(_dims(L, B=0)), FAKE, FAKE, FAKE, ctypes.byref(cs), None, FAKE, FAKE,
                               None, z, None) == L.OAL_OK
    # a few sequences: the state rows are split into slices whose partial
    # readouts need a workspace
    need = lib.oal_decode_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert lib.oal_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(cs), None, FAKE, FAKE, FAKE,
                               ctypes.c_size_t(need - 1), None) == L.OAL_ERR_WORKSPACE
    assert lib.oal_decode_step(ctypes.byref(d), FAKE, _mis(2), FAKE, ctypes.byref(cs), None, FAKE, FAKE, FAKE,
                               ctypes.c_size_t(need), None) == L.OAL_ERR_INVALID_ARG
    ws = ctypes.c_size_t(1 << 30)
    assert lib.oal_contrib(ctypes.byref(d), _mis(8), FAKE, None, None, FAKE, FAKE, ws, None) == \
        L.OAL_ERR_INVALID_ARG
    assert lib.oal_contrib(ctypes.byref(_dims(L, B=0)), FAKE, FAKE, None, None, FAKE, FAKE, ws, None) == \
        L.OAL_ERR_INVALID_ARG
    assert lib.oal_contrib(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, ws, None) == L.OAL_ERR_INVALID_ARG
    assert lib.oal_contrib(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, None, ctypes.c_size_t(0), None) == \
        L.OAL_ERR_WORKSPACE


def _bwd(L, dims, coeffs=True, diagonal=0, ws=(FAKE, 1 << 40), dq=FAKE, da=FAKE, dy=FAKE):
    lib = L.lib()
    cs = L.OalCoeffs(0x1000, 0x1000, 0x1000, 0x1000, diagonal) if coeffs else None
    return lib.oal_bwd(ctypes.byref(dims) if dims is not None else None, FAKE, FAKE, FAKE, dy,
                       ctypes.byref(cs) if cs is not None else None, dq, FAKE, FAKE, da, FAKE, FAKE, ws[0],
                       ctypes.c_size_t(ws[1]), None)


def test_bwd_validation_errors(L, no_device):
    E, U, W = L.OAL_ERR_INVALID_ARG, L.OAL_ERR_UNSUPPORTED, L.OAL_ERR_WORKSPACE
    ok = _dims(L, B=2, d=16, Hq=4, Hkv=4, G=16, N=300)
    assert _bwd(L, None) == E
    assert _bwd(L, _dims(L, d=16, G=17)) == E                  # G > d_h
    assert _bwd(L, _dims(L, d=64, Hq=4, Hkv=4)) == U           # only d_h = 16
    assert _bwd(L, _dims(L, d=16, Hq=4, Hkv=2)) == U           # heads with their own keys only
    assert _bwd(L, ok, diagonal=1) == U                        # the grouped kernel only
    assert _bwd(L, ok, coeffs=False) == E
    assert _bwd(L, ok, dy=None) == E
    assert _bwd(L, ok, dq=None) == E
    assert _bwd(L, ok, da=None) == E
    assert _bwd(L, ok, dy=_mis(4)) == E                        # 16-byte alignment
    need = L.lib().oal_bwd_workspace_bytes(ctypes.byref(ok))
    # the recomputed dL/d[num, den] rows, plus per-segment state sums (at
    # most eight segments of at most eight parts per sequence x head, 160
    # padded features x 65 columns) and coefficient sums (160 per segment)
    rows = 2 * 4 * 300 * 65 * 4
    seg = 2 * 4 * (64 * 160 * 65 + 8 * 160) * 4
    assert rows <= need <= rows + seg + 3 * 256
    assert _bwd(L, ok, ws=(None, 0)) == W
    assert _bwd(L, ok, ws=(FAKE, need - 1)) == W
    assert L.lib().oal_bwd_workspace_bytes(ctypes.byref(_dims(L, d=32, Hq=4, Hkv=4))) == 0
    assert L.lib().oal_bwd_workspace_bytes(None) == 0


def test_calibrate_validation_errors(L, no_device):
    """oal_calibrate refuses bad shapes, settings and plans before any work."""
    import numpy as np
    lib = L.lib()
    E, U, W = L.OAL_ERR_INVALID_ARG, L.OAL_ERR_UNSUPPORTED, L.OAL_ERR_WORKSPACE
    G, H, N, P = 2, 2, 40, 4
    ok = _dims(L, B=3, d=16, Hq=H, Hkv=H, G=G, N=N)
    inits = np.zeros((1, H, G + 1, G + 1))
    plan = np.array([[0, 1, 2, 3, 4], [2, 39, 0, 5, 7]], dtype=np.int32)
    outs = [np.zeros(H * (G + 1) ** 2), np.zeros(H), np.zeros(H), np.zeros(H, np.int32)]
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)

    def call(dims, plan=plan, prm=None, ws=(FAKE, 1 << 40), n_val=1):
        prm = prm or L.OalCalibParams(0.02, 10.0, 1e-3, P, 100, 400)
        return lib.oal_calibrate(ctypes.byref(dims), FAKE, FAKE, FAKE, n_val, FAKE, FAKE, FAKE, FAKE, 1, vp(inits),
                                 len(plan), vp(plan), ctypes.byref(prm), *[vp(o) for o in outs], None, None,
                                 ws[0], ctypes.c_size_t(ws[1]), None)

    assert call(_dims(L, B=3, d=64, Hq=H, Hkv=H, G=G, N=N)) == U   # the backward pass is d_h = 16 only
    assert call(_dims(L, B=3, d=16, Hq=4, Hkv=2, G=G, N=N)) == U   # heads with their own keys
    assert call(ok, n_val=0) == E
    assert call(ok, prm=L.OalCalibParams(0.02, 0.0, 1e-3, P, 100, 400)) == E   # clip must be > 0
    assert call(ok, prm=L.OalCalibParams(0.02, 10.0, 1e-3, N + 1, 100, 400)) == E
    assert call(ok, plan=np.array([[3, 1, 2, 3, 4]], dtype=np.int32)) == E   # sequence out of range
    assert call(ok, plan=np.array([[0, 1, 2, 2, 4]], dtype=np.int32)) == E   # repeated position
    assert call(ok, plan=np.array([[0, 1, 2, 3, 40]], dtype=np.int32)) == E  # position out of range
    assert call(ok, ws=(None, 0)) == W
    assert lib.oal_calibrate_workspace_bytes(ctypes.byref(ok), 1, FAKE) > 0
    assert lib.oal_calibrate_workspace_bytes(ctypes.byref(_dims(L, B=3, d=64, Hq=H, Hkv=H, G=G, N=N)), 1, FAKE) == 0


def test_binding_refuses_cpu_tensors(L):
    import torch
    import grouped_quadratic_softmax_amd as oal
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        oal.contrib(x, x)
