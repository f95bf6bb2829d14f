"""ctypes view of the C ABI declared in include/oal.h and include/oal_ceilings.h.

Loads the in-tree ``liboal.so``.  There is no fallback: if the library is
missing or fails to load, every entry point raises.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboal.so")

OAL_OK = 0
OAL_ERR_INVALID_ARG = -1
OAL_ERR_UNSUPPORTED = -2
OAL_ERR_WORKSPACE = -3
OAL_ERR_HIP = -4
OAL_F32 = 0
OAL_BF16 = 1


class OalDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "n_q_heads", "n_kv_heads", "seq_len", "d_h", "d_v", "n_groups", "dtype")]


class OalCoeffs(ctypes.Structure):
    _fields_ = [("group_of_dim", ctypes.c_void_p), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("c", ctypes.c_void_p), ("diagonal", ctypes.c_int32)]


class OalCalibParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("clip", ctypes.c_double), ("eps", ctypes.c_double),
                ("n_positions", ctypes.c_int32), ("validate_every", ctypes.c_int32), ("patience", ctypes.c_int32)]


class OalPrep(ctypes.Structure):
    _fields_ = [("gamma_q", ctypes.c_void_p), ("beta_q", ctypes.c_void_p), ("gamma_k", ctypes.c_void_p),
                ("beta_k", ctypes.c_void_p), ("ln_eps", ctypes.c_float), ("kind", ctypes.c_int32)]


class OalGroupParams(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_double), ("gamma", ctypes.c_double), ("tau", ctypes.c_double),
                ("eps", ctypes.c_double), ("g_min", ctypes.c_int32)]


class OalError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where} failed: {status_str(status)} ({status})")


_lib = None

_P = ctypes.c_void_p
_SIGS = {
    "oal_version": ([], ctypes.c_char_p),
    "oal_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "oal_feature_count": ([ctypes.c_int32], ctypes.c_int64),
    "oal_state_floats": ([ctypes.c_int32, ctypes.c_int32], ctypes.c_int64),
    "oal_coeffs_from_factor": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_double, _P, _P, _P, _P], ctypes.c_int),
    "oal_check_coeffs": ([_P, _P, _P], ctypes.c_int),
    "oal_fwd_workspace_bytes": ([_P], ctypes.c_size_t),
    "oal_fwd_workspace_bytes_for": ([_P, _P], ctypes.c_size_t),
    "oal_fwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "oal_fwd_varlen_workspace_bytes_for": ([_P, _P], ctypes.c_size_t),
    "oal_fwd_varlen": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "oal_fwd_states": ([_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "oal_fwd_outputs": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "oal_decode_workspace_bytes": ([_P], ctypes.c_size_t),
    "oal_decode_step": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "oal_decode_step_noalloc": ([_P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "oal_contrib_workspace_bytes": ([_P], ctypes.c_size_t),
    "oal_contrib": ([_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "oal_bwd_workspace_bytes": ([_P], ctypes.c_size_t),
    "oal_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "oal_calibrate_workspace_bytes": ([_P, ctypes.c_int32, _P], ctypes.c_size_t),
    "oal_calibrate": ([_P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_int32, _P, _P,
                       _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "oal_group_dims": ([ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P, _P, _P], ctypes.c_int),
    "oal_group_dims_budget": ([ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_double, _P], ctypes.c_int),
    # include/oal_ceilings.h
    "oal_ceiling_stream_rw": ([_P, ctypes.c_size_t, _P], ctypes.c_int),
    "oal_ceiling_mfma": ([_P, ctypes.c_int, ctypes.c_int, _P], ctypes.c_int),
    "oal_ceiling_mfma_flops": ([ctypes.c_int, ctypes.c_int], ctypes.c_double),
}


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"OAL HIP library not found at {LIB_PATH}; build it with "
                "`python -m grouped_quadratic_softmax_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().oal_status_str(int(status)).decode()


def check(status: int, where: str):
    if status != OAL_OK:
        raise OalError(status, where)
