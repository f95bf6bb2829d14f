"""Torch-facing binding of the OAL C ABI (argument marshalling only).

Every computation happens in the HIP kernels of ``liboal.so``; this module
checks tensor placement/shape/dtype, allocates outputs and workspaces with
torch (device memory plumbing) and passes raw pointers plus the current HIP
stream to the library.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _lib as L

_DT = {torch.float32: L.OAL_F32, torch.bfloat16: L.OAL_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(t, name, dtype=None, ndim=None):
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _need(t.is_cuda, f"{name} must be on the GPU")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None:
        _need(t.dim() == ndim, f"{name} must have {ndim} dims")
    return t


class Coeffs:
    """Device copies of the grouped-kernel coefficients of every query head.

    group_of_dim [Hq, d_h] int32 in [0, G), a [Hq], b [Hq, G], c [Hq, G, G]
    float32.  Host copies are checked with the library's validator before
    upload.
    """

    def __init__(self, group_of_dim, a, b, c, device="cuda", diagonal=None):
        g = np.ascontiguousarray(np.asarray(group_of_dim, dtype=np.int32))
        a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
        b = np.ascontiguousarray(np.asarray(b, dtype=np.float32))
        c = np.ascontiguousarray(np.asarray(c, dtype=np.float32))
        Hq, d = g.shape
        G = b.shape[1]
        _need(a.shape == (Hq,) and b.shape == (Hq, G) and c.shape == (Hq, G, G), "coefficient shapes")
        dims = L.OalDims(1, Hq, 1, 1, d, 64, G, 0)
        L.check(L.lib().oal_check_coeffs(ctypes.byref(dims), g.ctypes.data_as(ctypes.c_void_p),
                                         c.ctypes.data_as(ctypes.c_void_p)), "oal_check_coeffs")
        self.n_heads, self.d_h, self.n_groups = Hq, d, G
        # c without off-diagonal entries: the grouped kernel equals the
        # dimension-wise form read from the same coefficients
        self.offdiag_zero = not np.any(c * (1.0 - np.eye(G, dtype=np.float32)))
        if diagonal is None:
            # the dimension-wise form is exact when every group is one
            # dimension and c is diagonal; it is required beyond 8 groups
            singletons = G == d and all(np.array_equal(np.sort(row), np.arange(d)) for row in g)
            diagonal = bool(singletons and self.offdiag_zero)
        self.diagonal = bool(diagonal)
        self.group_of_dim = torch.from_numpy(g).to(device)
        self.a = torch.from_numpy(a).to(device)
        self.b = torch.from_numpy(b).to(device)
        self.c = torch.from_numpy(c).to(device)

    def struct(self):
        return L.OalCoeffs(self.group_of_dim.data_ptr(), self.a.data_ptr(), self.b.data_ptr(),
                           self.c.data_ptr(), 1 if self.diagonal else 0)


_PREMAP_KINDS = {"layernorm": 0, "l2": 1}


class Prep:
    """Pre-map parameters (device float32): gamma * norm(x) + beta on q and k,
    norm = LayerNorm (kind "layernorm", the ReBased map) or the unit l2 norm
    (kind "l2", the TaylorShift-style map)."""

    def __init__(self, gamma_q, beta_q, gamma_k, beta_k, ln_eps=1e-5, device="cuda", kind="layernorm"):
        _need(kind in _PREMAP_KINDS, f"pre-map kind must be one of {sorted(_PREMAP_KINDS)}")
        conv = lambda x: torch.as_tensor(np.asarray(x, dtype=np.float32)).contiguous().to(device)
        self.gamma_q, self.beta_q = conv(gamma_q), conv(beta_q)
        self.gamma_k, self.beta_k = conv(gamma_k), conv(beta_k)
        self.ln_eps = float(ln_eps)
        self.kind = kind

    def struct(self):
        return L.OalPrep(self.gamma_q.data_ptr(), self.beta_q.data_ptr(), self.gamma_k.data_ptr(),
                         self.beta_k.data_ptr(), self.ln_eps, _PREMAP_KINDS[self.kind])


def coeffs_from_factor(eps: float, Lf) -> tuple:
    """(eps, L [H, G+1, G+1]) -> (a [H], b [H, G], c [H, G, G]) float32, host side."""
    Lf = np.ascontiguousarray(np.asarray(Lf, dtype=np.float64))
    H, n, _ = Lf.shape
    G = n - 1
    a = np.zeros(H, np.float32)
    b = np.zeros((H, G), np.float32)
    c = np.zeros((H, G, G), np.float32)
    vp = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    L.check(L.lib().oal_coeffs_from_factor(H, G, float(eps), vp(Lf), vp(a), vp(b), vp(c)),
            "oal_coeffs_from_factor")
    return a, b, c


def feature_count(d_h: int) -> int:
    return int(L.lib().oal_feature_count(d_h))


def state_floats(d_h: int, d_v: int) -> int:
    return int(L.lib().oal_state_floats(d_h, d_v))


def _dims(B, Hq, Hkv, N, d, dv, G, dtype):
    return L.OalDims(B, Hq, Hkv, N, d, dv, G, _DT[dtype])


def fwd_workspace_bytes(B, Hq, Hkv, N, d_h, d_v, G, dtype) -> int:
    dims = _dims(B, Hq, Hkv, N, d_h, d_v, G, dtype)
    return int(L.lib().oal_fwd_workspace_bytes(ctypes.byref(dims)))


def fwd_workspace_bytes_for(q, k, v, coeffs: Coeffs, varlen=False) -> int:
    """Workspace oal_fwd (varlen: oal_fwd_varlen) uses at full parallelism
    for these tensors and coefficients."""
    B, Hq, N, d = q.shape
    dims = _dims(B, Hq, k.shape[1], N, d, v.shape[3], coeffs.n_groups, q.dtype)
    cs = coeffs.struct()
    fn = L.lib().oal_fwd_varlen_workspace_bytes_for if varlen else L.lib().oal_fwd_workspace_bytes_for
    return int(fn(ctypes.byref(dims), ctypes.byref(cs)))


def fwd(q, k, v, coeffs: Coeffs, prep: Optional[Prep] = None, state_in=None, return_state=False,
        y=None, state_out=None, workspace=None, seq_lens=None):
    """Causal OAL prefill.  q [B, Hq, N, d], k [B, Hkv, N, d], v [B, Hkv, N, 64].

    seq_lens: optional device int32 [B]; sequence b then uses its first
    seq_lens[b] rows (oal_fwd_varlen: the other rows of y are not written).
    Returns y (and the final state [B, Hkv, state_floats] when return_state).
    """
    _dev(q, "q", ndim=4)
    _need(q.dtype in _DT, "q must be float32 or bfloat16")
    _dev(k, "k", q.dtype, 4)
    _dev(v, "v", q.dtype, 4)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dv = v.shape[3]
    _need(k.shape == (B, Hkv, N, d) and v.shape == (B, Hkv, N, dv), "k/v shapes")
    _need(coeffs.n_heads == Hq and coeffs.d_h == d, "coefficients do not match q")
    dims = _dims(B, Hq, Hkv, N, d, dv, coeffs.n_groups, q.dtype)
    if y is None:
        y = torch.empty((B, Hq, N, dv), dtype=q.dtype, device=q.device)
    sf = state_floats(d, dv)
    if state_in is not None:
        _dev(state_in, "state_in", torch.float32)
        _need(state_in.numel() == B * Hkv * sf, "state_in size")
    if return_state and state_out is None:
        state_out = torch.empty((B, Hkv, sf), dtype=torch.float32, device=q.device)
    cs = coeffs.struct()
    if seq_lens is not None:
        _dev(seq_lens, "seq_lens", torch.int32, 1)
        _need(seq_lens.numel() == B, "seq_lens must hold one length per sequence")
    if workspace is None:  # a caller's workspace is passed as given
        size_fn = (L.lib().oal_fwd_varlen_workspace_bytes_for if seq_lens is not None
                   else L.lib().oal_fwd_workspace_bytes_for)
        nbytes = int(size_fn(ctypes.byref(dims), ctypes.byref(cs)))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    else:
        _dev(workspace, "workspace", torch.uint8)
    ps = prep.struct() if prep is not None else None
    args = (_ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs), ctypes.byref(ps) if ps is not None else None,
            _ptr(state_in), _ptr(state_out), _ptr(y), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream())
    if seq_lens is None:
        L.check(L.lib().oal_fwd(ctypes.byref(dims), *args), "oal_fwd")
    else:
        L.check(L.lib().oal_fwd_varlen(ctypes.byref(dims), _ptr(seq_lens), *args), "oal_fwd_varlen")
    return (y, state_out) if return_state else y


def decode_workspace_bytes(B, Hq, Hkv, d_h, d_v, G, dtype) -> int:
    dims = _dims(B, Hq, Hkv, 0, d_h, d_v, G, dtype)
    return int(L.lib().oal_decode_workspace_bytes(ctypes.byref(dims)))


def decode_step(q, k, v, coeffs: Coeffs, state, prep: Optional[Prep] = None, y=None, workspace=None):
    """One decode step.  q [B, Hq, d], k [B, Hkv, d], v [B, Hkv, 64];
    state [B, Hkv, state_floats] float32 updated in place.  Returns y [B, Hq, 64]."""
    _dev(q, "q", ndim=3)
    _need(q.dtype in _DT, "q must be float32 or bfloat16")
    _dev(k, "k", q.dtype, 3)
    _dev(v, "v", q.dtype, 3)
    _dev(state, "state", torch.float32)
    B, Hq, d = q.shape
    Hkv, dv = k.shape[1], v.shape[2]
    _need(state.numel() == B * Hkv * state_floats(d, dv), "state size")
    dims = _dims(B, Hq, Hkv, 0, d, dv, coeffs.n_groups, q.dtype)
    if y is None:
        y = torch.empty((B, Hq, dv), dtype=q.dtype, device=q.device)
    nbytes = int(L.lib().oal_decode_workspace_bytes(ctypes.byref(dims)))
    if nbytes > 0 and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    cs = coeffs.struct()
    ps = prep.struct() if prep is not None else None
    st = L.lib().oal_decode_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs),
                                 ctypes.byref(ps) if ps is not None else None, _ptr(state), _ptr(y),
                                 _ptr(workspace), ctypes.c_size_t(0 if workspace is None else workspace.numel()),
                                 _stream())
    L.check(st, "oal_decode_step")
    return y


def contrib(q, k, seq_lens=None, per_prompt=False, workspace=None):
    """Contribution scores chi [Hq, d] (and chi per prompt [P, Hq, d]).

    q [P, Hq, N, d], k [P, Hkv, N, d]; seq_lens: None or int32 device [P]."""
    _dev(q, "q", ndim=4)
    _need(q.dtype in _DT, "q must be float32 or bfloat16")
    _dev(k, "k", q.dtype, 4)
    P, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if seq_lens is not None:
        _dev(seq_lens, "seq_lens", torch.int32, 1)
    dims = _dims(P, Hq, Hkv, N, d, 64, 1, q.dtype)
    chi = torch.empty((Hq, d), dtype=torch.float32, device=q.device)
    chip = torch.empty((P, Hq, d), dtype=torch.float32, device=q.device) if per_prompt else None
    nbytes = int(L.lib().oal_contrib_workspace_bytes(ctypes.byref(dims)))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = L.lib().oal_contrib(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(seq_lens), _ptr(chip), _ptr(chi),
                             _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream())
    L.check(st, "oal_contrib")
    return (chi, chip) if per_prompt else chi


def bwd_workspace_bytes(B, H, N, d_h, d_v, G, dtype) -> int:
    dims = _dims(B, H, H, N, d_h, d_v, G, dtype)
    return int(L.lib().oal_bwd_workspace_bytes(ctypes.byref(dims)))


def bwd(q, k, v, dy, coeffs: Coeffs, workspace=None, out=None):
    """Gradients of sum(dy * y) for y = fwd(q, k, v, coeffs) (oal_bwd).

    q, k [B, H, N, 16], v, dy [B, H, N, 64], one dtype.  Returns dq, dk, dv
    (float32, the input shapes) and da [H], db [H, G], dc [H, G, G] (float32,
    summed over the batch), written into `out` (those six tensors) when
    given."""
    _dev(q, "q", ndim=4)
    _need(q.dtype in _DT, "q must be float32 or bfloat16")
    _dev(k, "k", q.dtype, 4)
    _dev(v, "v", q.dtype, 4)
    _dev(dy, "dy", q.dtype, 4)
    B, H, N, d = q.shape
    dv = v.shape[3]
    _need(k.shape == q.shape and v.shape == (B, H, N, dv) and dy.shape == v.shape, "k/v/dy shapes")
    _need(coeffs.n_heads == H and coeffs.d_h == d, "coefficients do not match q")
    G = coeffs.n_groups
    dims = _dims(B, H, H, N, d, dv, G, q.dtype)
    f32 = dict(dtype=torch.float32, device=q.device)
    shapes = (q.shape, k.shape, v.shape, (H,), (H, G), (H, G, G))
    if out is None:
        out = tuple(torch.empty(sh, **f32) for sh in shapes)
    _need(len(out) == 6, "out must hold dq, dk, dv, da, db, dc")
    for t, sh, name in zip(out, shapes, ("dq", "dk", "dv", "da", "db", "dc")):
        _dev(t, name, torch.float32)
        _need(tuple(t.shape) == tuple(sh), f"{name} shape")
    dq, dk, dvv, da, db, dc = out
    nbytes = int(L.lib().oal_bwd_workspace_bytes(ctypes.byref(dims)))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    cs = coeffs.struct()
    if coeffs.diagonal:  # the backward takes the grouped kernel, which is the same kernel here
        _need(coeffs.offdiag_zero, "bwd: the dimension-wise form with off-diagonal c entries has no backward")
        cs.diagonal = 0
    st = L.lib().oal_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(dy), ctypes.byref(cs), _ptr(dq),
                         _ptr(dk), _ptr(dvv), _ptr(da), _ptr(db), _ptr(dc), _ptr(workspace),
                         ctypes.c_size_t(workspace.numel()), _stream())
    L.check(st, "oal_bwd")
    return dq, dk, dvv, da, db, dc


def calibrate(train, val, group_of_dim, inits, plan, lr=0.02, clip=10.0, eps=1e-3, validate_every=100,
              patience=400, workspace=None):
    """Output-matching calibration of the factors L of every head
    (oal_calibrate).  train, val: (q, k, v) device tensors [T, H, N, d] and
    [V, H, N, d] of one dtype (heads with their own keys); group_of_dim
    [H, d] ints; inits [n_init, H, G+1, G+1]; plan [U, 1 + P] ints (per
    update a training sequence and P distinct positions).  Returns a dict of
    numpy arrays: "L" [H, G+1, G+1], "mse", "relmse", "init" [H],
    "cand_mse" and "updates" [n_init, H]."""
    qt, kt, vt = train
    qv, kv, vv = val
    for name, t in (("q_train", qt), ("k_train", kt), ("v_train", vt), ("q_val", qv), ("k_val", kv), ("v_val", vv)):
        _dev(t, name, qt.dtype, 4)
    _need(qt.dtype in _DT, "activations must be float32 or bfloat16")
    T, H, N, d = qt.shape
    _need(kt.shape == qt.shape and vt.shape[:3] == (T, H, N), "training shapes")
    _need(qv.shape[1:] == qt.shape[1:] and kv.shape == qv.shape and vv.shape[:3] == qv.shape[:3], "validation shapes")
    dv = vt.shape[3]
    n_val = qv.shape[0]
    g = np.ascontiguousarray(np.asarray(group_of_dim, dtype=np.int32))
    inits = np.ascontiguousarray(np.asarray(inits, dtype=np.float64))
    plan = np.ascontiguousarray(np.asarray(plan, dtype=np.int32))
    n_init, Hi, n, _ = inits.shape
    G = n - 1
    _need(Hi == H and g.shape == (H, d), "inits and group map must match the heads")
    _need(plan.ndim == 2 and plan.shape[1] >= 2, "plan must be [updates, 1 + positions]")
    P = plan.shape[1] - 1
    dims = _dims(T, H, H, N, d, dv, G, qt.dtype)
    gd = torch.from_numpy(g).to(qt.device)
    nbytes = int(L.lib().oal_calibrate_workspace_bytes(ctypes.byref(dims), n_val, _ptr(gd)))
    _need(nbytes > 0, "calibration not supported for these shapes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=qt.device)
    prm = L.OalCalibParams(float(lr), float(clip), float(eps), P, int(validate_every), int(patience))
    L_out = np.zeros((H, n, n))
    mse, rel = np.zeros(H), np.zeros(H)
    init = np.zeros(H, np.int32)
    cand = np.zeros((n_init, H))
    upd = np.zeros((n_init, H), np.int32)
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = L.lib().oal_calibrate(ctypes.byref(dims), _ptr(qt), _ptr(kt), _ptr(vt), n_val, _ptr(qv), _ptr(kv), _ptr(vv),
                               _ptr(gd), n_init, vp(inits), plan.shape[0], vp(plan), ctypes.byref(prm), vp(L_out),
                               vp(mse), vp(rel), vp(init), vp(cand), vp(upd), _ptr(workspace),
                               ctypes.c_size_t(workspace.numel()), _stream())
    L.check(st, "oal_calibrate")
    return {"L": L_out, "mse": mse, "relmse": rel, "init": init, "cand_mse": cand, "updates": upd}


class PrefillPlan:
    """Pre-marshalled oal_fwd arguments for repeated calls on fixed buffers.

    ``run()`` enqueues one oal_fwd call on the stream that is current at
    construction time; ``states()`` and ``outputs()`` enqueue its two stages
    separately (not available for coefficients in the dimension-wise form).
    With ``staged=False`` the workspace is sized for ``run()`` alone, which
    for the one-pass paths is far smaller than the two stages need.
    """

    def __init__(self, q, k, v, coeffs: Coeffs, prep: Optional[Prep] = None, state_in=None,
                 with_state=True, staged=True):
        import torch
        B, Hq, N, d = q.shape
        Hkv, dv = k.shape[1], v.shape[3]
        self.q, self.k, self.v, self.coeffs, self.prep = q, k, v, coeffs, prep
        self.y = torch.empty((B, Hq, N, dv), dtype=q.dtype, device=q.device)
        self.state_in = state_in
        self.state_out = (torch.empty((B, Hkv, state_floats(d, dv)), dtype=torch.float32, device=q.device)
                          if with_state else None)
        self.dims = _dims(B, Hq, Hkv, N, d, dv, coeffs.n_groups, q.dtype)
        self._cs = coeffs.struct()
        lib = L.lib()
        nbytes = int(lib.oal_fwd_workspace_bytes_for(ctypes.byref(self.dims), ctypes.byref(self._cs)))
        if staged and not coeffs.diagonal:  # the two stages need the full workspace
            nbytes = max(nbytes, int(lib.oal_fwd_workspace_bytes(ctypes.byref(self.dims))))
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        self._ps = prep.struct() if prep is not None else None
        pp = ctypes.byref(self._ps) if self._ps is not None else None
        ws = (_ptr(self.workspace), ctypes.c_size_t(self.workspace.numel()))
        st = _stream()
        self._states_args = (ctypes.byref(self.dims), _ptr(k), _ptr(v), pp, _ptr(state_in), _ptr(self.state_out),
                             *ws, st)
        self._out_args = (ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(self._cs), pp,
                          _ptr(state_in), _ptr(self.y), *ws, st)
        self._fwd_args = (ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(self._cs), pp,
                          _ptr(state_in), _ptr(self.state_out), _ptr(self.y), *ws, st)
        self._lib = L.lib()
        self._staged = staged

    def states(self):
        _need(self._staged, "PrefillPlan(staged=False) has no separate stages")
        L.check(self._lib.oal_fwd_states(*self._states_args), "oal_fwd_states")

    def outputs(self):
        _need(self._staged, "PrefillPlan(staged=False) has no separate stages")
        L.check(self._lib.oal_fwd_outputs(*self._out_args), "oal_fwd_outputs")

    def run(self):
        L.check(self._lib.oal_fwd(*self._fwd_args), "oal_fwd")
        return self.y


class DecodePlan:
    """Pre-marshalled oal_decode_step arguments (state updated in place)."""

    def __init__(self, q, k, v, coeffs: Coeffs, state, prep: Optional[Prep] = None):
        import torch
        B, Hq, d = q.shape
        Hkv, dv = k.shape[1], v.shape[2]
        self.y = torch.empty((B, Hq, dv), dtype=q.dtype, device=q.device)
        self.dims = _dims(B, Hq, Hkv, 0, d, dv, coeffs.n_groups, q.dtype)
        nbytes = int(L.lib().oal_decode_workspace_bytes(ctypes.byref(self.dims)))
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        self._keep = (q, k, v, coeffs, state, prep)
        self._cs = coeffs.struct()
        self._ps = prep.struct() if prep is not None else None
        pp = ctypes.byref(self._ps) if self._ps is not None else None
        self._args = (ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(self._cs), pp, _ptr(state),
                      _ptr(self.y), _ptr(self.workspace), ctypes.c_size_t(self.workspace.numel()), _stream())
        self._lib = L.lib()

    def run(self):
        L.check(self._lib.oal_decode_step(*self._args), "oal_decode_step")
        return self.y


class ContribPlan:
    """Pre-marshalled oal_contrib arguments."""

    def __init__(self, q, k, seq_lens=None, per_prompt=False):
        import torch
        P, Hq, N, d = q.shape
        Hkv = k.shape[1]
        self.dims = _dims(P, Hq, Hkv, N, d, 64, 1, q.dtype)
        self.chi = torch.empty((Hq, d), dtype=torch.float32, device=q.device)
        self.chi_per_prompt = torch.empty((P, Hq, d), dtype=torch.float32, device=q.device) if per_prompt else None
        nbytes = int(L.lib().oal_contrib_workspace_bytes(ctypes.byref(self.dims)))
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        self._keep = (q, k, seq_lens)
        self._args = (ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(seq_lens), _ptr(self.chi_per_prompt),
                      _ptr(self.chi), _ptr(self.workspace), ctypes.c_size_t(self.workspace.numel()), _stream())
        self._lib = L.lib()

    def run(self):
        L.check(self._lib.oal_contrib(*self._args), "oal_contrib")
        return self.chi


class StepPlan:
    """One pass of the hot path on fixed buffers, spread over two streams.

    A batch of prompts ``q, k, v [B, H, N, d]`` is prefilled (one oal_fwd
    call keeping the final states), each sequence then decodes one token
    ``qn, kn, vn [B, H, d]`` on the prefill's final state, and chi (the
    per-dimension contribution of the prompts' q and k) is reduced.

    The prefill and the decode step run in that order on the stream current
    at construction.  Chi reads only q and k, so a second stream of default
    priority runs it from the start of the step, on the compute units that
    the prefill's first launch leaves idle.  ``run()`` starts with the
    second stream waiting for the first (so chi sees inputs produced earlier
    on it, and the previous step's consumers of the chi buffer are done) and
    ends with the first stream waiting for the second.  (The decode step stays behind the prefill:
    when the prefill has one workgroup per compute unit, a decode launched
    beside it holds compute units that the prefill then waits for.)
    """

    def __init__(self, q, k, v, qn, kn, vn, coeffs: Coeffs, prep: Optional[Prep] = None):
        import torch
        self.main = torch.cuda.current_stream()
        self.side = torch.cuda.Stream()
        self.prefill = PrefillPlan(q, k, v, coeffs, prep, staged=False)
        self.decode = DecodePlan(qn, kn, vn, coeffs, self.prefill.state_out, prep)
        with torch.cuda.stream(self.side):
            self.chi = ContribPlan(q, k)

    def run(self):
        self.side.wait_stream(self.main)
        self.prefill.run()
        self.chi.run()
        self.decode.run()
        self.main.wait_stream(self.side)
