"""GPU check of the machine-ceiling probes (include/oal_ceilings.h): the
stream probe applies its update exactly once per element, the MFMA probe
writes finite values, and both reject bad arguments before any launch."""

import ctypes

import pytest

from helpers import log, require_gpu

pytestmark = pytest.mark.gpu


def test_stream_probe_updates_every_element_once():
    require_gpu()
    import torch
    from grouped_quadratic_softmax_amd import _lib as L
    lib = L.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for n in (4, 1028, 1 << 20, (1 << 20) + 4 * 1000):
        x = torch.arange(n, device="cuda", dtype=torch.float32)
        L.check(lib.oal_ceiling_stream_rw(ctypes.c_void_p(x.data_ptr()), ctypes.c_size_t(n), st), "stream")
        want = torch.arange(n, dtype=torch.float64) * float(torch.tensor(0.999)) + float(torch.tensor(1e-3))
        # once, not twice or never: the update changes every value by far more than its rounding
        assert torch.allclose(x.cpu().double(), want, rtol=2e-7, atol=1e-9), n
    assert lib.oal_ceiling_stream_rw(ctypes.c_void_p(x.data_ptr()), ctypes.c_size_t(6), st) == L.OAL_ERR_INVALID_ARG


def test_mfma_probe_runs():
    require_gpu()
    import torch
    from grouped_quadratic_softmax_amd import _lib as L
    lib = L.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.full((8 * 256,), float("nan"), device="cuda", dtype=torch.float32)
    L.check(lib.oal_ceiling_mfma(ctypes.c_void_p(out.data_ptr()), 8, 32, st), "mfma")
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert lib.oal_ceiling_mfma(ctypes.c_void_p(out.data_ptr()), 8, 30, st) == L.OAL_ERR_INVALID_ARG
    assert lib.oal_ceiling_mfma_flops(8, 32) == 8 * 4 * 32 * 8 * 2 * 16 * 16 * 32
    log("[ceilings] probes ran")
