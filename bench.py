#!/usr/bin/env python3
"""Causal OAL attention throughput on one MI355X.

Workload (default): the Based Taylor kernel (one group, a = 1, b = 1,
c = 1/2) on a d_h = 16 projected feature space -- B = 8 sequences of N = 8192
tokens, 16 heads, d_v = 64, bf16, seeded synthetic inputs.  One step is one
pass of the whole hot path over that batch: contribution scores chi
(Eq. (2)), the causal prefill keeping the final states (Eqs. (5)-(6)), and one
recurrent decode step per sequence on those states.

Prints ONE JSON line.  `value` is tokens/s over the whole step (prefill tokens
plus decoded tokens).  `roofline` is the prefill (its HBM fraction binds;
its bf16 MFMA fraction is given beside it), timed with HIP events on its
own stream; `roofline_decode` is the batched decode step of 256 sequences x
16 heads with fp32 states (HBM-bound); `ceilings` are the in-place stream and
MFMA-chain probes measured in the same run; `cpu_baseline` is the fp64
oracle on the host.  Secondary lines (under "secondary") time the other
workloads' hot kernels: the Qwen-shaped GQA layer, the ReBased prefill, the
32k-token prefill, the backward pass of the timed prefill, and the
output-matching calibration.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3   # MI355X dense fp32 matrix cores (256 CUs x 2.4 GHz x 256 flops per cycle)
COPY_BYTES = 1 << 30        # calibration copy for the HBM byte counters
STREAM_BYTES = 2 << 30      # in-place stream probe (read and written once each)
METRIC = "causal OAL attention tokens/s at 1 GPU; % bf16 MFMA peak (prefill), % HBM BW (decode)"
DV = 64
DECODE_SEQS, DECODE_HEADS = 256, 16


def feature_count(d):
    return 1 + d + d * (d + 1) // 2


def load_traffic(key):
    """HBM bytes per launch measured with rocprofv3 counters, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    from grouped_quadratic_softmax_amd.profiling import source_hash
    if not rec or rec.get("source_sha256") != source_hash(rec.get("sources")):
        return None
    return rec.get("bytes_per_launch")


def device_inputs(wl):
    import torch
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = lambda x: torch.from_numpy(x).to("cuda").to(dt).contiguous()
    return dev(wl.q), dev(wl.k), dev(wl.v)


def coeffs_for(wl, groups=None):
    import grouped_quadratic_softmax_amd as oal
    if wl.coeff["kind"] == "factor":
        a, b, c = oal.coeffs_from_factor(wl.coeff["eps"], wl.coeff["L"])
    else:
        a, b, c = wl.coeff["a"], wl.coeff["b"], wl.coeff["c"]
    return oal.Coeffs(wl.group_of_dim if groups is None else groups, a, b, c)


def bwd_flops_per_token(d, N, C=32):
    """Algorithmic flops per (token, head) of the backward pass in the packed
    feature space (D features, d_v + 1 columns with the normaliser), counted
    from its definition (2 flops per multiply-add): the six state products
    of D x (d_v + 1) per token (the readout it recomputes against S, S g, the
    state update, R u, R^T m(k) and the R update), and per causal pair within
    a C-token chunk (C / 2 pairs per token on average): kappa twice (2 D
    each), dkappa twice (2 (d_v + 1) each), the readout's pair term (d_v + 1),
    the dq and dk pair terms (2 D each) and dv's (d_v).  The segment sums
    that let segments run in parallel are not counted."""
    D = feature_count(d)
    state = 6 * 2 * D * (DV + 1)
    pair = 2 * (2 * D) + 2 * (2 * (DV + 1)) + 2 * (DV + 1) + 2 * (2 * D) + 2 * DV
    return state + pair * min(C, N) / 2


def time_events(fn, steps, warmup):
    """Mean duration (ms) of fn() over `steps` calls, HIP events recorded on
    the current stream (the stream the plans below launch on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    return sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / steps  # ms


def settle_with(fn, ms=60.0):
    """Run `fn` back to back, untimed, for about `ms` before it is timed.
    The clocks drop within a second of idling (host-side setup between the
    timed regions does that) and after the ceiling probes (the MFMA chain
    draws the chip's full power) take some tens of milliseconds of load to
    climb back: without this the first ~60 steps run about 12% slower than
    every later one."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def measure_ceilings(reps=40):
    """The in-place read+write stream probe over 2 GiB and the bf16 MFMA
    chain probe (include/oal_ceilings.h), each timed with HIP events over
    `reps` calls (about 50 ms of sustained load in all)."""
    import ctypes
    import torch
    from grouped_quadratic_softmax_amd import _lib as L
    lib = L.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.zeros(STREAM_BYTES // 4, device="cuda", dtype=torch.float32)
    ms = time_events(lambda: L.check(lib.oal_ceiling_stream_rw(ctypes.c_void_p(buf.data_ptr()),
                                                                ctypes.c_size_t(buf.numel()), stream),
                                     "oal_ceiling_stream_rw"), reps, 3)
    stream_gbs = 2 * STREAM_BYTES / (ms * 1e-3) / 1e9
    del buf
    wgs, iters = 4096, 512
    out = torch.empty(wgs * 256, device="cuda", dtype=torch.float32)
    ms_m = time_events(lambda: L.check(lib.oal_ceiling_mfma(ctypes.c_void_p(out.data_ptr()), wgs, iters, stream),
                                       "oal_ceiling_mfma"), reps, 3)
    tflops = lib.oal_ceiling_mfma_flops(wgs, iters) / (ms_m * 1e-3) / 1e12
    return {"stream_rw_GBs": stream_gbs, "stream_rw_bytes": 2 * STREAM_BYTES, "stream_rw_ms": ms,
            "mfma_bf16_TFLOPs": tflops, "mfma_probe": f"{wgs} workgroups x 4 waves x {iters} x 8 "
                                                       "v_mfma_f32_16x16x32_bf16", "mfma_ms": ms_m}


def run_main(args):
    import torch
    import grouped_quadratic_softmax_amd as oal
    import synthetic as S

    wl = S.make(3, seq_len=8192 + 1)  # token N is the decoded one
    B, Hq, Hkv, N1, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.seq_len, wl.d_h
    N = N1 - 1
    q_all, k_all, v_all = device_inputs(wl)
    q, k, v = (t[:, :, :N].contiguous() for t in (q_all, k_all, v_all))
    qn, kn, vn = (t[:, :, N].contiguous() for t in (q_all, k_all, v_all))
    co = coeffs_for(wl)

    # The timed step (oal.StepPlan) runs chi on a second stream of default
    # priority beside the prefill; the decode step follows the prefill on the
    # main stream, which waits for chi at the end of every step.
    plan = oal.StepPlan(q, k, v, qn, kn, vn, co)
    chi_main = oal.ContribPlan(q, k)  # the same reduction on the main stream, for the per-stage timing

    run_step = plan.run
    if args.no_overlap:
        def run_step():
            chi_main.run()
            plan.prefill.run()
            plan.decode.run()
    # The machine ceilings are measured here, right before the steps: the
    # probes' sustained load (about 50 ms) also brings the clocks, which drop
    # within a second of idling, to the level a sustained workload runs at.
    ce = measure_ceilings()
    print("[bench] ceilings done", file=sys.stderr, flush=True)
    settle_with(run_step)
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-stage durations with HIP events on the main stream (separate pass)
    stage_ms = {"contrib": time_events(chi_main.run, args.steps, 2),
                "prefill": time_events(plan.prefill.run, args.steps, 2),
                "decode": time_events(plan.decode.run, args.steps, 2)}
    pre_ms = stage_ms["prefill"]

    D = feature_count(d)
    tokens_per_step = B * N + B
    ms_per_step = elapsed / args.steps * 1e3
    io_bytes = B * N * Hq * d * 2 + B * N * Hkv * (d * 2 + DV * 2) + B * N * Hq * DV * 2  # q, k, v, y
    flops = B * N * Hq * 2 * D * (DV + 1) + B * N * Hkv * 2 * D * (DV + 1)  # readout + state update
    gbs = io_bytes / (pre_ms * 1e-3) / 1e9
    tfl = flops / (pre_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": tokens_per_step / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "mfma_format": "v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulation)",
        "data": "synthetic (seeded Gaussian Q, K ~ N(0, 1/16), V ~ N(0, 1); no pretrained weights)",
        "config": {"workload": "Based Taylor kernel (G=1, a=1, b=1, c=1/2): B=8, H=16, N=8192, d_h=16, d_v=64, "
                               "bf16; step = chi + prefill(+final state) + 1 decode token/seq",
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "roofline": {
            "kernel": "onepass16w_kernel (oal_fwd prefill at d_h=16 in one launch: segment sums and outputs of "
                      "four segments per workgroup, two chained workgroups per sequence)",
            "bound": "hbm",
            "achieved": gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS,
            "traffic": load_traffic("onepass16_based_prefill"),
            "algorithmic_bytes_per_launch": io_bytes,
            "avg_launch_ms": pre_ms,
            "mfma_achieved_TFLOPs": tfl,
            "mfma_frac": tfl / PEAK_BF16_TFLOPS,
            "algorithmic_flops_per_launch": flops,
        },
        "schedule": ("one stream" if args.no_overlap else
                     "chi on a second stream beside the prefill; the second stream waits for the first at the "
                     "start of every step and the first for the second at its end"),
        "stages_ms": stage_ms,
    }
    del plan, chi_main, q, k, v, q_all, k_all, v_all
    return result, wl, ce


def run_decode(args):
    """The batched decode step: 256 sequences x 16 heads, d_h = d_v = 64,
    eight groups, fp32 states of (1 + 64 + 2080) x 65 each, updated in place."""
    import torch
    import grouped_quadratic_softmax_amd as oal
    import synthetic as S

    S_, H = DECODE_SEQS, DECODE_HEADS
    D = feature_count(64)
    g = torch.Generator(device="cuda").manual_seed(1205)
    state = torch.rand((S_, H, D * (DV + 1)), generator=g, device="cuda", dtype=torch.float32)
    mk = lambda *shape: torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    qd, kd, vd = mk(S_, H, 64), mk(S_, H, 64), mk(S_, H, 64)
    groups = ((torch.arange(64) * 8) // 64).repeat(H, 1).numpy()
    wl5 = S.make(5, seq_len=8, batch=1)
    dec = oal.DecodePlan(qd, kd, vd, coeffs_for(wl5, groups), state)
    settle_with(dec.run)
    ms = time_events(dec.run, max(10, args.steps), 3)
    nbytes = 2 * S_ * H * D * (DV + 1) * 4 + (3 * S_ * H * 64 + S_ * H * 64) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "decode_kernel (oal_decode_step, 256 sequences x 16 heads, G=8, fp32 states)",
            "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "traffic": load_traffic("decode_256x16"), "algorithmic_bytes_per_launch": nbytes,
            "avg_launch_ms": ms, "tokens_per_s": S_ / (ms * 1e-3)}


def run_secondary(args):
    import numpy as np
    import torch
    import grouped_quadratic_softmax_amd as oal
    import synthetic as S

    out = {}
    steps, warm = max(3, args.steps // 5), 2
    # the Qwen2.5-0.5B-shaped GQA layer (B=4, N=2048, Hq=14, Hkv=2, d_h=64,
    # G=4): the whole step, and its chunk readout (the MFMA-bound kernel)
    wl = S.make(2, seq_len=2048 + 1)
    N = wl.seq_len - 1
    q_all, k_all, v_all = device_inputs(wl)
    q, k, v = (t[:, :, :N].contiguous() for t in (q_all, k_all, v_all))
    qn, kn, vn = (t[:, :, N].contiguous() for t in (q_all, k_all, v_all))
    plan = oal.StepPlan(q, k, v, qn, kn, vn, coeffs_for(wl))
    settle_with(plan.run)
    step_ms = time_events(plan.run, steps, warm)
    pre = oal.PrefillPlan(q, k, v, coeffs_for(wl))
    st_ms = time_events(pre.states, steps, warm)
    out_ms = time_events(pre.outputs, steps, warm)
    D = feature_count(64)
    rd_flops = wl.batch * N * wl.n_q_heads * 2 * D * (DV + 1)
    up_flops = wl.batch * N * wl.n_kv_heads * 2 * D * (DV + 1)
    out["c2_qwen_layer"] = {"step_ms": step_ms, "tokens_per_s": wl.batch * (N + 1) / (step_ms * 1e-3),
                            "states_ms": st_ms, "readout_ms": out_ms,
                            "readout_mfma_frac": rd_flops / (out_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                            "readout_traffic": load_traffic("readout_kernel_qwen_layer"),
                            "prefill_mfma_frac": (rd_flops + up_flops) / ((st_ms + out_ms) * 1e-3) / 1e12
                                                 / PEAK_BF16_TFLOPS}
    del plan, pre
    # the same layer with eight groups of eight dimensions: the readout alone
    # (its eight-group build)
    rng = np.random.default_rng(2048)
    a8, b8, c8 = oal.coeffs_from_factor(1e-3, rng.standard_normal((wl.n_q_heads, 9, 9)))
    g8 = np.repeat(np.arange(8, dtype=np.int32), 8)[None, :].repeat(wl.n_q_heads, 0)
    pre = oal.PrefillPlan(q, k, v, oal.Coeffs(g8, a8, b8, c8))
    pre.states()
    settle_with(pre.outputs)
    ms = time_events(pre.outputs, steps, warm)
    out["c2_gqa_g8_readout"] = {"ms": ms, "mfma_frac": rd_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del pre, q, k, v, q_all, k_all, v_all
    # ReBased elementwise-square prefill, B=16, H=8, N=2048 (dimension-wise
    # form: features [1, k, k^2], HBM-bound)
    wl = S.make(4)
    q, k, v = device_inputs(wl)
    p = wl.premap
    pre = oal.PrefillPlan(q, k, v, coeffs_for(wl),
                          oal.Prep(p["gamma_q"], p["beta_q"], p["gamma_k"], p["beta_k"], p["ln_eps"]))
    settle_with(pre.run)
    ms = time_events(pre.run, steps, warm)
    tok = wl.batch * wl.seq_len
    io = tok * wl.n_q_heads * (2 * 64 * 2) + tok * wl.n_kv_heads * (2 * 64 * 2)
    out["c4_rebased_prefill"] = {"ms": ms, "tokens_per_s": tok / (ms * 1e-3),
                                 "hbm_frac": io / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                 "kernel": "dimw_kernel (one launch, chained segment groups)",
                                 "traffic": load_traffic("dimw_rebased_prefill")}
    del pre, q, k, v
    # 32k-token prefill, 16 heads, 8 contribution-sorted groups
    wl = S.make(5)
    q, k, v = device_inputs(wl)
    chi = oal.contrib(q, k).cpu().numpy()
    groups = oal.groups_from_contribution(chi, wl.group_budget["bulk_sizes"], wl.group_budget["n_tail"])
    pre = oal.PrefillPlan(q, k, v, coeffs_for(wl, groups))
    settle_with(pre.run)
    ms = time_events(pre.run, steps, warm)
    tok = wl.batch * wl.seq_len
    flops = tok * 2 * wl.n_q_heads * 2 * D * (DV + 1)
    out["c5_long_prefill"] = {"ms": ms, "tokens_per_s": tok / (ms * 1e-3),
                              "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del pre, q, k, v
    # the backward pass of the Based prefill (B=8, H=16, N=8192, d_h=16):
    # fp32 matrix-core products over the packed features
    wl = S.make(3)
    q, k, v = device_inputs(wl)
    dy = torch.randn(v.shape, generator=torch.Generator(device="cuda").manual_seed(2102), device="cuda").to(v.dtype)
    co = coeffs_for(wl)
    B_, H_, N_ = wl.batch, wl.n_q_heads, wl.seq_len
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = (torch.empty(q.shape, **f32), torch.empty(k.shape, **f32), torch.empty(v.shape, **f32),
            torch.empty((H_,), **f32), torch.empty((H_, 1), **f32), torch.empty((H_, 1, 1), **f32))
    ws = torch.empty(max(oal.bwd_workspace_bytes(B_, H_, N_, 16, DV, 1, q.dtype), 1), dtype=torch.uint8,
                     device="cuda")
    settle_with(lambda: oal.bwd(q, k, v, dy, co, workspace=ws, out=outs))
    ms = time_events(lambda: oal.bwd(q, k, v, dy, co, workspace=ws, out=outs), steps, warm)
    flops = B_ * H_ * N_ * bwd_flops_per_token(16, N_)
    out["f2_based_backward"] = {"ms": ms, "tokens_per_s": B_ * N_ / (ms * 1e-3),
                                "fp32_mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
                                "traffic": load_traffic("bwd16_based_backward"),
                                "kernels": "bwd16_segsum_kernel x2, bwd16_fwd_kernel, bwd16_rev_kernel, "
                                           "bwd16_coef_kernel (fp32 MFMA)"}
    del q, k, v, dy, outs, ws
    out["f3_calibration"] = run_calibration()
    return out


def calibration_case():
    """The calibration run timed here: the Based shape at the settings' scale
    (8 training and 2 validation sequences of 4096 tokens, 16 heads, d_h = 16,
    bf16; four groups of four dimensions; 32 positions per update; the
    Taylor factors as the one candidate)."""
    import numpy as np
    import synthetic as S
    T, V, N, H, G = 8, 2, 4096, 16, 4
    wl = S.make(3, batch=T + V, seq_len=N)
    groups = np.repeat(np.arange(G, dtype=np.int32), 16 // G)[None, :].repeat(H, 0)
    M = np.full((G + 1, G + 1), 0.5)
    M[0, 0] = 1.0
    L0 = np.linalg.cholesky(M + 1e-3 * np.eye(G + 1))
    inits = np.stack([np.stack([L0] * H)])
    return wl, T, groups, inits


def run_calibration(n_updates=100):
    """oal_calibrate on calibration_case(): one call with no update (targets
    and the initial validation) and one with n_updates updates and a second
    validation; the difference over n_updates is the cost of an update."""
    import numpy as np
    import torch
    import grouped_quadratic_softmax_amd as oal
    import synthetic as S
    wl, T, groups, inits = calibration_case()
    q, k, v = device_inputs(wl)
    tr, va = (q[:T], k[:T], v[:T]), (q[T:], k[T:], v[T:])
    plan = S.calibration_plan(T, wl.seq_len, 32, n_updates)
    times = []
    for U in (0, n_updates):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = oal.calibrate(tr, va, groups, inits, plan[:U], validate_every=n_updates, patience=4 * n_updates)
        times.append(time.perf_counter() - t0)
    per = (times[1] - times[0]) / n_updates
    return {"ms_per_update": per * 1e3, "targets_and_validation_ms": times[0] * 1e3,
            "protocol_3x1000_s": 3 * (times[0] + 1000 * per),
            "mse_after": float(np.mean(res["mse"])), "shape": "T=8, V=2, N=4096, H=16, d_h=16, G=4, bf16, P=32"}


def run_pmc_target(args):
    """Launch only one kernel repeatedly, for rocprofv3 counter passes.

    ``based16``: the prefill of the timed workload (B=8, H=16, N=8192,
    d_h=16: the one-launch chained kernel); ``decode``: the
    batched decode step (256 sequences x 16 heads, fp32 states);
    ``readout`` / ``states``: the chunk readout / chunk scan of the
    Qwen-shaped GQA layer (B=4, N=2048, Hq=14, Hkv=2, d_h=64);
    ``rebased``: the one-launch prefill of the ReBased workload in the
    dimension-wise form (B=16, H=8, N=2048); ``long``: the prefill of the
    long-context multi-head workload (B=1, H=16, N=32768, d_h=64, eight
    groups from its contribution scores); ``copy``: a plain device copy of
    1 GiB (fp32), whose FETCH_SIZE and WRITE_SIZE readings calibrate the
    counters against a known byte count; ``mfma``: the bf16 MFMA chain probe,
    whose MFMA counters calibrate the busy fraction of the prefill kernels;
    ``stream``: the in-place stream probe over 2 GiB; ``bwd``: the backward
    pass of the timed workload's prefill (B=8, H=16, N=8192, d_h=16);
    ``calib``: one calibration run of ``--steps`` updates on
    calibration_case()."""
    import ctypes
    import torch
    import grouped_quadratic_softmax_amd as oal
    import synthetic as S

    def repeat(fn):
        torch.cuda.synchronize()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"pmc_target": args.pmc_target, "launches": args.steps}), flush=True)

    t = args.pmc_target
    if t == "copy":
        n = COPY_BYTES // 4
        src = torch.ones(n, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        repeat(lambda: dst.copy_(src))
        return
    if t in ("mfma", "stream"):
        from grouped_quadratic_softmax_amd import _lib as L
        lib = L.lib()
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if t == "mfma":
            out = torch.empty(4096 * 256, device="cuda", dtype=torch.float32)
            repeat(lambda: L.check(lib.oal_ceiling_mfma(ctypes.c_void_p(out.data_ptr()), 4096, 512, st), t))
        else:
            buf = torch.zeros(STREAM_BYTES // 4, device="cuda", dtype=torch.float32)
            repeat(lambda: L.check(lib.oal_ceiling_stream_rw(ctypes.c_void_p(buf.data_ptr()),
                                                             ctypes.c_size_t(buf.numel()), st), t))
        return
    if t == "decode":
        S_, H = DECODE_SEQS, DECODE_HEADS
        D = feature_count(64)
        g = torch.Generator(device="cuda").manual_seed(1205)
        state = torch.rand((S_, H, D * (DV + 1)), generator=g, device="cuda", dtype=torch.float32)
        mk = lambda *shape: torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
        groups = ((torch.arange(64) * 8) // 64).repeat(H, 1).numpy()
        dec = oal.DecodePlan(mk(S_, H, 64), mk(S_, H, 64), mk(S_, H, 64),
                             coeffs_for(S.make(5, seq_len=8, batch=1), groups), state)
        repeat(dec.run)
        return
    if t == "long":
        wl = S.make(5)
        q, k, v = device_inputs(wl)
        chi = oal.contrib(q, k).cpu().numpy()
        groups = oal.groups_from_contribution(chi, wl.group_budget["bulk_sizes"], wl.group_budget["n_tail"])
        pre = oal.PrefillPlan(q, k, v, coeffs_for(wl, groups), staged=False)
        repeat(pre.run)
        return
    if t == "calib":
        import synthetic as S2
        wl, T, groups, inits = calibration_case()
        q, k, v = device_inputs(wl)
        plan = S2.calibration_plan(T, wl.seq_len, 32, args.steps)
        res = oal.calibrate((q[:T], k[:T], v[:T]), (q[T:], k[T:], v[T:]), groups, inits, plan,
                            validate_every=max(args.steps, 1))
        print(json.dumps({"pmc_target": t, "updates": args.steps, "mse": float(res["mse"].mean())}), flush=True)
        return
    if t == "bwd":
        wl = S.make(3)
        q, k, v = device_inputs(wl)
        dy = torch.randn(v.shape, generator=torch.Generator(device="cuda").manual_seed(2102),
                         device="cuda").to(v.dtype)
        co = coeffs_for(wl)
        f32 = dict(dtype=torch.float32, device="cuda")
        H_ = wl.n_q_heads
        outs = (torch.empty(q.shape, **f32), torch.empty(k.shape, **f32), torch.empty(v.shape, **f32),
                torch.empty((H_,), **f32), torch.empty((H_, 1), **f32), torch.empty((H_, 1, 1), **f32))
        repeat(lambda: oal.bwd(q, k, v, dy, co, out=outs))
        return
    if t in ("based16", "rebased"):
        wl = S.make(3 if t == "based16" else 4)
        q, k, v = device_inputs(wl)
        p = wl.premap
        prep = (oal.Prep(p["gamma_q"], p["beta_q"], p["gamma_k"], p["beta_k"], p["ln_eps"])
                if p is not None else None)
        pre = oal.PrefillPlan(q, k, v, coeffs_for(wl), prep, staged=False)
        repeat(pre.run)
        return
    wl = S.make(2, seq_len=2048 + 1)
    N = wl.seq_len - 1
    q, k, v = (t_[:, :, :N].contiguous() for t_ in device_inputs(wl))
    pre = oal.PrefillPlan(q, k, v, coeffs_for(wl))
    pre.states()
    repeat(pre.outputs if t == "readout" else pre.states)


def cpu_baseline(wl, min_seconds=10.0):
    """The fp64 oracle (as it stands) on a bounded sample of the same
    workload: whole sequences of it (every head, every token), each through
    chi (separable form), the prefix-recurrence attention (the oracle's
    linear-time form), the final states and one decode step, repeated until
    at least ``min_seconds`` of host time have passed."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    N = wl.seq_len - 1
    a, b, c = wl.coeff["a"], wl.coeff["b"], wl.coeff["c"]
    done = 0
    t0 = time.perf_counter()
    while True:
        bi = done % wl.batch
        qs, ks, vs = (x[bi:bi + 1, :, :N] for x in (wl.q, wl.k, wl.v))
        O.chi_separable(qs, ks)
        _, st = O.attention_recurrent_packed(qs, ks, vs, wl.group_of_dim, a, b, c, return_state=True)
        O.decode_step(st, wl.q[bi:bi + 1, :, N], wl.k[bi:bi + 1, :, N], wl.v[bi:bi + 1, :, N], wl.group_of_dim,
                      a, b, c, wl.n_q_heads)
        done += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    tokens = done * (N + 1)
    return {"value": tokens / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "blas_threads": blas_threads, "seconds": dt,
            "sample": f"{done} sequence(s) of the workload ({N} prefill tokens + 1 decoded token each, all "
                      f"{wl.n_q_heads} heads): chi (separable form), fp64 prefix-recurrence attention with the "
                      f"final states, one decode step; repeated until >= {min_seconds:g} s of host time"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run chi, prefill and decode back to back on one stream")
    ap.add_argument("--pmc-target", default=None,
                    choices=("based16", "decode", "readout", "states", "rebased", "long", "copy", "mfma", "stream", "bwd",
                             "calib"),
                    help="only launch this kernel --steps times (for rocprofv3 counter passes)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the OAL library and this benchmark run on one GPU; no figures for more GPUs are "
              "produced (batch x KV-head sharding needs no communication and is not implemented).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.pmc_target:
        run_pmc_target(args)
        return
    result, wl, ce = run_main(args)
    print(f"[bench] main done: {result['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
    result["roofline_decode"] = run_decode(args)
    result["ceilings"] = ce
    result["roofline"]["frac_of_stream_ceiling"] = result["roofline"]["achieved"] / ce["stream_rw_GBs"]
    result["roofline"]["mfma_frac_of_probe"] = result["roofline"]["mfma_achieved_TFLOPs"] / ce["mfma_bf16_TFLOPs"]
    result["roofline_decode"]["frac_of_stream_ceiling"] = result["roofline_decode"]["achieved"] / ce["stream_rw_GBs"]
    print("[bench] decode done", file=sys.stderr, flush=True)
    if not args.no_secondary:
        result["secondary"] = run_secondary(args)
        print("[bench] secondary done", file=sys.stderr, flush=True)
    result["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
