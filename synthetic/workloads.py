"""Seeded synthetic stand-ins for the workloads the OAL method is measured on.

The pages measure on frozen post-RoPE Q/K/V of pretrained models (Qwen2.5-0.5B,
GPT-2 Medium) over WikiText; none of that is available here, so every input is
drawn from a seeded generator with the same shapes and the same kind of
structure: Gaussian coordinates with a few planted high-magnitude dimensions,
mirroring the concentrated per-dimension contribution profile the OAL paper
reports (section 3.1 and Table 4 of "Not All Dimensions Are Equal:
Outlier-Aware Attention Linearization with Grouped Quadratic Kernels").

Draw order per workload (fixed so that every consumer sees identical data):
Q, K, V, outlier dimensions, coefficient draws, pre-map affine draws.  Values
are drawn in float32, outlier dimensions are scaled, and the result is rounded
to bfloat16 (round to nearest even) when the workload is a bf16 one.  Arrays
are returned as float32 numpy arrays whose values are exactly representable in
the workload dtype, so a consumer can convert them without further rounding.

Coefficients are returned as raw draws.  Workloads 2 and 5 draw the factor of
the positive group-aware kernel (a lower-triangular L and epsilon, OAL paper
section 4.3, Eq. (7)); mapping them to (a, b_g, c_gh) is the method's own
arithmetic and is done by each consumer.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

CONFIG_NAMES = {
    1: "c1_fp32_single_head",
    2: "c2_qwen_gqa",
    3: "c3_based_taylor",
    4: "c4_rebased",
    5: "c5_gpt2m_long",
}

#: Seeds: workload k draws from numpy's PCG64 seeded with 1000 + k.
SEED_BASE = 1000


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    d_h: int
    d_v: int
    dtype: str  # "f32" or "bf16"
    q: np.ndarray  # [B, Hq, N, d_h] float32
    k: np.ndarray  # [B, Hkv, N, d_h] float32
    v: np.ndarray  # [B, Hkv, N, d_v] float32
    n_groups: int
    #: [Hq, d_h] int32 group id per dimension, or None when the grouping is to
    #: be derived from contribution scores (see ``group_budget``).
    group_of_dim: Optional[np.ndarray]
    #: {"kind": "abc", "a": [Hq], "b": [Hq, G], "c": [Hq, G, G]} or
    #: {"kind": "factor", "eps": float, "L": [Hq, G+1, G+1] lower triangular}
    coeff: dict
    #: None or {"gamma_q": [Hq, d], "beta_q": [Hq, d], "gamma_k": [Hkv, d],
    #: "beta_k": [Hkv, d], "ln_eps": float}
    premap: Optional[dict] = None
    #: For contribution-derived groups: {"bulk_sizes": [...], "n_tail": int}
    group_budget: Optional[dict] = None
    #: planted outlier dimensions per KV head, [Hkv, n] int
    outlier_dims: Optional[np.ndarray] = None

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len


def _normal(rng, shape, std=1.0):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _factor_draw(rng, n_heads, G):
    """Lower-triangular (G+1)x(G+1) factors: diagonal U(0.5,1.5), strictly lower U(0,0.5)."""
    n = G + 1
    L = np.zeros((n_heads, n, n), dtype=np.float64)
    for h in range(n_heads):
        for i in range(n):
            for j in range(i + 1):
                L[h, i, j] = rng.uniform(0.5, 1.5) if i == j else rng.uniform(0.0, 0.5)
    return L


def _finish(x, dtype):
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def make(config: int, *, batch=None, seq_len=None, n_q_heads=None, n_kv_heads=None,
         seed=None, dtype=None, rebased_reading: str = "e") -> Workload:
    """Build workload ``config`` (1..5) with optional size overrides.

    Overrides shrink a workload for tests while keeping its structure; the
    seed defaults to 1000 + config.
    """
    if config not in CONFIG_NAMES:
        raise ValueError(f"unknown workload {config}")
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + config if seed is None else seed))

    if config == 1:
        # Single head, fp32; dims 26 and 58 planted x8 in Q and K; groups
        # {26}, {58}, then the remaining dims in index order as two groups of 31.
        B, Hq, Hkv, N, d, dv = 1, 1, 1, 256, 64, 64
        B, N = batch or B, seq_len or N
        Hq, Hkv = n_q_heads or Hq, n_kv_heads or Hkv
        dt = dtype or "f32"
        q = _normal(rng, (B, Hq, N, d))
        k = _normal(rng, (B, Hkv, N, d))
        v = _normal(rng, (B, Hkv, N, dv))
        outl = np.array([[26, 58]] * Hkv, dtype=np.int64)
        q[..., [26, 58]] *= 8.0
        k[..., [26, 58]] *= 8.0
        G = 4
        rest = [r for r in range(d) if r not in (26, 58)]
        gmap = np.zeros(d, dtype=np.int32)
        gmap[26], gmap[58] = 0, 1
        gmap[rest[:31]] = 2
        gmap[rest[31:]] = 3
        groups = np.tile(gmap, (Hq, 1))
        A = rng.uniform(0.0, 0.1, size=(Hq, G, G))
        c = 0.5 + np.einsum("hij,hkj->hik", A, A)
        coeff = {"kind": "abc", "a": np.ones(Hq), "b": np.ones((Hq, G)), "c": c}
        return Workload(CONFIG_NAMES[1], B, Hq, Hkv, N, d, dv, dt, _finish(q, dt), _finish(k, dt),
                        _finish(v, dt), G, groups, coeff, outlier_dims=outl)

    if config == 2:
        # Qwen2.5-0.5B-shaped layer: 14 query heads over 2 KV heads, two planted
        # outlier dims per KV head (x10 in K and in the Q of its query heads).
        B, Hq, Hkv, N, d, dv = 4, 14, 2, 2048, 64, 64
        B, N = batch or B, seq_len or N
        Hq, Hkv = n_q_heads or Hq, n_kv_heads or Hkv
        dt = dtype or "bf16"
        q = _normal(rng, (B, Hq, N, d))
        k = _normal(rng, (B, Hkv, N, d))
        v = _normal(rng, (B, Hkv, N, dv))
        rep = Hq // Hkv
        outl = np.stack([rng.choice(d, size=2, replace=False) for _ in range(Hkv)])
        G = 4
        groups = np.zeros((Hq, d), dtype=np.int32)
        for kh in range(Hkv):
            o1, o2 = int(outl[kh, 0]), int(outl[kh, 1])
            k[:, kh, :, [o1, o2]] *= 10.0
            rest = [r for r in range(d) if r not in (o1, o2)]
            for h in range(kh * rep, (kh + 1) * rep):
                q[:, h, :, [o1, o2]] *= 10.0
                groups[h, o1], groups[h, o2] = 0, 1
                groups[h, rest[:31]] = 2
                groups[h, rest[31:]] = 3
        coeff = {"kind": "factor", "eps": 1e-3, "L": _factor_draw(rng, Hq, G)}
        return Workload(CONFIG_NAMES[2], B, Hq, Hkv, N, d, dv, dt, _finish(q, dt), _finish(k, dt),
                        _finish(v, dt), G, groups, coeff, outlier_dims=outl)

    if config == 3:
        # Based Taylor kernel on a 16-dim projected feature space.
        B, Hq, Hkv, N, d, dv = 8, 16, 16, 8192, 16, 64
        B, N = batch or B, seq_len or N
        Hq, Hkv = n_q_heads or Hq, n_kv_heads or Hkv
        dt = dtype or "bf16"
        q = _normal(rng, (B, Hq, N, d), std=0.25)
        k = _normal(rng, (B, Hkv, N, d), std=0.25)
        v = _normal(rng, (B, Hkv, N, dv))
        G = 1
        groups = np.zeros((Hq, d), dtype=np.int32)
        coeff = {"kind": "abc", "a": np.ones(Hq), "b": np.ones((Hq, 1)), "c": np.full((Hq, 1, 1), 0.5)}
        return Workload(CONFIG_NAMES[3], B, Hq, Hkv, N, d, dv, dt, _finish(q, dt), _finish(k, dt),
                        _finish(v, dt), G, groups, coeff)

    if config == 4:
        # ReBased: (gamma * LayerNorm(x) + beta)^2 feature map, separate affine
        # for queries and keys; gamma ~ N(1, 0.1), beta ~ N(0, 0.1) (variances).
        B, Hq, Hkv, N, d, dv = 16, 8, 8, 2048, 64, 64
        B, N = batch or B, seq_len or N
        Hq, Hkv = n_q_heads or Hq, n_kv_heads or Hkv
        dt = dtype or "bf16"
        q = _normal(rng, (B, Hq, N, d))
        k = _normal(rng, (B, Hkv, N, d))
        v = _normal(rng, (B, Hkv, N, dv))
        sd = float(np.sqrt(0.1))
        premap = {
            "gamma_q": (1.0 + _normal(rng, (Hq, d), sd)).astype(np.float32),
            "beta_q": _normal(rng, (Hq, d), sd),
            "gamma_k": (1.0 + _normal(rng, (Hkv, d), sd)).astype(np.float32),
            "beta_k": _normal(rng, (Hkv, d), sd),
            "ln_eps": 1e-5,
        }
        if rebased_reading == "e":
            # elementwise square: one singleton group per dimension, c = d * I
            G = d
            groups = np.tile(np.arange(d, dtype=np.int32), (Hq, 1))
            coeff = {"kind": "abc", "a": np.zeros(Hq), "b": np.zeros((Hq, G)),
                     "c": np.tile(np.eye(G) * d, (Hq, 1, 1))}
        elif rebased_reading == "d":
            # squared dot product of the mapped vectors: one group, c = d
            G = 1
            groups = np.zeros((Hq, d), dtype=np.int32)
            coeff = {"kind": "abc", "a": np.zeros(Hq), "b": np.zeros((Hq, 1)),
                     "c": np.full((Hq, 1, 1), float(d))}
        else:
            raise ValueError("rebased_reading must be 'e' or 'd'")
        return Workload(CONFIG_NAMES[4] + ("" if rebased_reading == "e" else "_alt"), B, Hq, Hkv, N,
                        d, dv, dt, _finish(q, dt), _finish(k, dt), _finish(v, dt), G, groups, coeff,
                        premap=premap)

    # config 5: GPT-2-Medium-shaped long context, 16 heads, two planted outlier
    # dims per head (x10), 8 groups derived from contribution scores: the top-2
    # dims as singletons, the other 62 in ascending-contribution order split
    # into bulk groups of 11, 11, 10, 10, 10, 10.
    B, Hq, Hkv, N, d, dv = 1, 16, 16, 32768, 64, 64
    B, N = batch or B, seq_len or N
    Hq, Hkv = n_q_heads or Hq, n_kv_heads or Hkv
    dt = dtype or "bf16"
    q = _normal(rng, (B, Hq, N, d))
    k = _normal(rng, (B, Hkv, N, d))
    v = _normal(rng, (B, Hkv, N, dv))
    rep = Hq // Hkv
    outl = np.stack([rng.choice(d, size=2, replace=False) for _ in range(Hkv)])
    for kh in range(Hkv):
        k[:, kh, :, outl[kh]] *= 10.0
        for h in range(kh * rep, (kh + 1) * rep):
            q[:, h, :, outl[kh]] *= 10.0
    G = 8
    coeff = {"kind": "factor", "eps": 1e-3, "L": _factor_draw(rng, Hq, G)}
    return Workload(CONFIG_NAMES[5], B, Hq, Hkv, N, d, dv, dt, _finish(q, dt), _finish(k, dt),
                    _finish(v, dt), G, None, coeff,
                    group_budget={"bulk_sizes": [11, 11, 10, 10, 10, 10], "n_tail": 2},
                    outlier_dims=outl)


def decode_prefix_lengths(n_seq: int, max_len: int = 512, seed: int = 1105) -> np.ndarray:
    """Seeded prefix lengths in [1, max_len] for the batched decode workload."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(1, max_len + 1, size=n_seq).astype(np.int32)


def calibration_plan(n_train: int, seq_len: int, n_positions: int, n_updates: int, seed: int = 2200) -> np.ndarray:
    """Seeded sampling plan of a calibration run: per update, one training
    sequence and n_positions distinct causal query positions (the pages'
    settings draw one sequence and 32 positions per update).  int32
    [n_updates, 1 + n_positions]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    plan = np.zeros((n_updates, 1 + n_positions), dtype=np.int32)
    for u in range(n_updates):
        plan[u, 0] = rng.integers(0, n_train)
        plan[u, 1:] = rng.choice(seq_len, size=n_positions, replace=False)
    return plan
