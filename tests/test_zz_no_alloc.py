"""GPU check of oal_decode_step_noalloc (the decode step on the library's own
scratch array, for callers that cannot allocate) against oal_decode_step with
a caller workspace: identical outputs and states, bit for bit, on two calls
in a row (the second smaller), and a clear refusal of a size beyond the
array."""

import ctypes

import numpy as np
import pytest

import synthetic as S
from helpers import log, require_gpu

pytestmark = pytest.mark.gpu


def _noalloc(oal, L, q, k, v, co, state, y):
    import torch
    from grouped_quadratic_softmax_amd.ops import _dims, _ptr
    B, Hq, d = q.shape
    Hkv, dv = k.shape[1], v.shape[2]
    dims = _dims(B, Hq, Hkv, 0, d, dv, co.n_groups, q.dtype)
    cs = co.struct()
    return L.lib().oal_decode_step_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs), None,
                                           _ptr(state), _ptr(y),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_decode_matches_workspace_decode(dtype):
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    from grouped_quadratic_softmax_amd import _lib as L
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(77)
    # (sequences, query heads, KV heads, d_h, groups): the second call smaller;
    # the third, at d_h = 16 (one slice per state), needs no scratch at all
    for B, Hq, Hkv, d, G in ((96, 8, 2, 64, 4), (5, 3, 3, 32, 2), (5, 3, 3, 16, 2)):
        groups = np.stack([rng.permutation(np.arange(d) % G) for _ in range(Hq)]).astype(np.int32)
        a, b, c = oal.coeffs_from_factor(1e-3, rng.standard_normal((Hq, G + 1, G + 1)) * 0.5)
        co = oal.Coeffs(groups, a, b, c)
        need = oal.decode_workspace_bytes(B, Hq, Hkv, d, 64, G, dt)
        if d > 16:
            assert 0 < need <= 32 << 20, need  # the scratch is really used
        else:
            assert need == 0, need
        g = torch.Generator(device="cuda").manual_seed(B)
        q = torch.randn((B, Hq, d), generator=g, device="cuda").to(dt)
        k = torch.randn((B, Hkv, d), generator=g, device="cuda").to(dt)
        v = torch.randn((B, Hkv, 64), generator=g, device="cuda").to(dt)
        s0 = torch.rand((B, Hkv, oal.state_floats(d, 64)), generator=g, device="cuda")
        s_ref, s_new = s0.clone(), s0.clone()
        y_ref = oal.decode_step(q, k, v, co, s_ref)
        y_new = torch.full_like(y_ref, float("nan"))
        st = _noalloc(oal, L, q, k, v, co, s_new, y_new)
        torch.cuda.synchronize()
        assert st == L.OAL_OK, L.status_str(st)
        log(f"[noalloc] {dtype} B={B} Hq={Hq} Hkv={Hkv} d={d} G={G} scratch bytes {need}: "
            f"y equal {bool(torch.equal(y_new, y_ref))}, state equal {bool(torch.equal(s_new, s_ref))}")
        assert torch.equal(y_new, y_ref)
        assert torch.equal(s_new, s_ref)


def test_noalloc_decode_refuses_sizes_beyond_its_scratch():
    require_gpu()
    import torch
    import grouped_quadratic_softmax_amd as oal
    from grouped_quadratic_softmax_amd import _lib as L
    from grouped_quadratic_softmax_amd.ops import _dims
    dims = _dims(2048, 128, 16, 0, 64, 64, 4, torch.bfloat16)
    assert int(L.lib().oal_decode_workspace_bytes(ctypes.byref(dims))) > 32 << 20
    co = oal.Coeffs(np.zeros((128, 64), np.int32), np.ones(128), np.ones((128, 4)), np.zeros((128, 4, 4)))
    cs = co.struct()
    # refused on the size alone, before any pointer is looked at or a kernel launched
    st = L.lib().oal_decode_step_noalloc(ctypes.byref(dims), None, None, None, ctypes.byref(cs), None, None, None,
                                         None)
    assert st == L.OAL_ERR_WORKSPACE
