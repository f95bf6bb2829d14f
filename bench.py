#!/usr/bin/env python3
"""Causal OAL attention throughput on one MI355X.

Workload (default): the Qwen2.5-0.5B-shaped attention layer -- B = 4 sequences
of N = 2048 tokens, 14 query heads over 2 KV heads (GQA), d_h = d_v = 64,
bf16, 4 dimension groups (two planted outlier singletons + two bulk groups),
seeded synthetic inputs.  One step is one pass of the whole hot path over that
batch: contribution scores chi (Eq. (2)), the chunked causal prefill (chunk
states, then readout + within-chunk pairs + normalisation) keeping the final
states, and one recurrent decode step per sequence on those states.

Prints ONE JSON line.  `value` is tokens/s over the whole step (prefill tokens
plus decoded tokens); `roofline` is the dominant kernel (the chunk readout)
timed with HIP events on its own stream; `cpu_baseline` is the fp64 oracle on
the host.  Secondary lines (under "secondary") time the other workloads' hot
kernels: the d_h = 16 Based prefill (HBM-bound), the 32k-token prefill and the
batched decode step with 256 x 16 fp32 states (HBM-bound).
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
COPY_BYTES = 1 << 30        # calibration copy for the HBM byte counters
METRIC = "causal OAL attention tokens/s at 1 GPU; % bf16 MFMA peak (prefill), % HBM BW (decode)"
DV = 64


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
    if not rec or rec.get("source_sha256") != source_hash():
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


def time_events(fn, steps, warmup):
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


def run_main(args):
    import torch
    import grouped_quadratic_softmax_amd as oal
    import synthetic as S

    wl = S.make(2, seq_len=2048 + 1)  # token N is the decoded one
    B, Hq, Hkv, N1, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.seq_len, wl.d_h
    N = N1 - 1
    q_all, k_all, v_all = device_inputs(wl)
    q, k, v = (t[:, :, :N].contiguous() for t in (q_all, k_all, v_all))
    qn, kn, vn = (t[:, :, N].contiguous() for t in (q_all, k_all, v_all))
    co = coeffs_for(wl)

    chi_plan = oal.ContribPlan(q, k)
    pre = oal.PrefillPlan(q, k, v, co)
    dec = oal.DecodePlan(qn, kn, vn, co, pre.state_out)
    # The timed step (oal.StepPlan) runs chi on a second stream of default
    # priority beside the scan; the readout and the decode step follow the
    # scan on the main stream, which waits for chi at the end of every step.
    overlapped = oal.StepPlan(q, k, v, qn, kn, vn, co)
    step_overlapped = overlapped.run

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    stage_ms = [0.0, 0.0, 0.0, 0.0]

    def step(record):
        if record:
            ev[0].record()
        chi_plan.run()
        if record:
            ev[1].record()
        pre.states()
        if record:
            ev[2].record()
        pre.outputs()
        if record:
            ev[3].record()
        dec.run()
        if record:
            ev[4].record()

    run_step = (lambda: step(False)) if args.no_overlap else step_overlapped
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    # per-stage durations with HIP events on the same stream (separate pass)
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        for i in range(4):
            stage_ms[i] += ev[i].elapsed_time(ev[i + 1]) / args.steps
    out_ms = stage_ms[2]

    D = feature_count(d)
    tokens_per_step = B * N + B
    ms_per_step = elapsed / args.steps * 1e3
    readout_flops = B * N * Hq * 2 * D * (DV + 1)         # one launch of the readout kernel
    update_flops = B * N * Hkv * 2 * D * (DV + 1)
    achieved = readout_flops / (out_ms * 1e-3) / 1e12
    traffic = load_traffic("readout_kernel_qwen_layer")
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
        "data": "synthetic (seeded Gaussian Q/K/V with planted outlier dims; no pretrained weights)",
        "config": {"workload": "qwen2.5-0.5b-shaped OAL layer: B=4, N=2048, Hq=14, Hkv=2, d_h=d_v=64, G=4, "
                               "bf16; step = chi + prefill(+final state) + 1 decode token/seq",
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "roofline": {
            "kernel": "readout_kernel (oal_fwd_outputs: coefficient tables, chunk readout, intra-chunk block, normalise)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "algorithmic_flops_per_launch": readout_flops,
            "avg_launch_ms": out_ms,
        },
        "schedule": ("one stream" if args.no_overlap else
                     "chi on a second stream beside the chunk scan; streams joined every step"),
        "stages_ms": {"contrib": stage_ms[0], "prefill_states": stage_ms[1], "prefill_outputs": stage_ms[2],
                      "decode": stage_ms[3]},
        "prefill_mfma_frac": (readout_flops + update_flops) / ((stage_ms[1] + stage_ms[2]) * 1e-3) / 1e12
                             / PEAK_BF16_TFLOPS,
    }
    return result, wl


def run_secondary(args):
    import numpy as np
    import torch
    import grouped_quadratic_softmax_amd as oal
    import synthetic as S

    out = {}
    steps, warm = max(3, args.steps // 5), 2
    # the same GQA layer (B=4, N=2048, Hq=14, Hkv=2) with eight groups of
    # eight dimensions: the readout alone (its eight-group build)
    wl = S.make(2, seq_len=2048)
    q, k, v = device_inputs(wl)
    rng = np.random.default_rng(2048)
    a8, b8, c8 = oal.coeffs_from_factor(1e-3, rng.standard_normal((wl.n_q_heads, 9, 9)))
    g8 = np.repeat(np.arange(8, dtype=np.int32), 8)[None, :].repeat(wl.n_q_heads, 0)
    pre = oal.PrefillPlan(q, k, v, oal.Coeffs(g8, a8, b8, c8))
    pre.states()
    ms = time_events(pre.outputs, steps, warm)
    flops = wl.batch * wl.seq_len * wl.n_q_heads * 2 * feature_count(64) * (DV + 1)
    out["c2_gqa_g8_readout"] = {"ms": ms, "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del pre, q, k, v
    # d_h = 16 Based Taylor prefill, B=8, H=16, N=8192 (HBM-bound)
    wl = S.make(3)
    q, k, v = device_inputs(wl)
    pre = oal.PrefillPlan(q, k, v, coeffs_for(wl))
    ms = time_events(pre.run, steps, warm)
    tok = wl.batch * wl.seq_len
    D = feature_count(16)
    flops = tok * 2 * wl.n_q_heads * 2 * D * (DV + 1)
    io = tok * wl.n_q_heads * (16 * 2 * 2 + DV * 2 * 2)
    out["c3_based_prefill"] = {"ms": ms, "tokens_per_s": tok / (ms * 1e-3),
                               "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                               "hbm_frac": io / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del pre, q, k, v
    # ReBased elementwise-square prefill, B=16, H=8, N=2048 (dimension-wise
    # form: features [1, k, k^2], HBM-bound)
    wl = S.make(4)
    q, k, v = device_inputs(wl)
    p = wl.premap
    pre = oal.PrefillPlan(q, k, v, coeffs_for(wl),
                          oal.Prep(p["gamma_q"], p["beta_q"], p["gamma_k"], p["beta_k"], p["ln_eps"]))
    ms = time_events(pre.run, steps, warm)
    tok = wl.batch * wl.seq_len
    io = tok * wl.n_q_heads * (2 * 64 * 2) + tok * wl.n_kv_heads * (2 * 64 * 2)
    out["c4_rebased_prefill"] = {"ms": ms, "tokens_per_s": tok / (ms * 1e-3),
                                 "hbm_frac": io / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del pre, q, k, v
    # 32k-token prefill, 16 heads, 8 contribution-sorted groups
    wl = S.make(5)
    q, k, v = device_inputs(wl)
    chi = oal.contrib(q, k).cpu().numpy()
    groups = oal.groups_from_contribution(chi, wl.group_budget["bulk_sizes"], wl.group_budget["n_tail"])
    pre = oal.PrefillPlan(q, k, v, coeffs_for(wl, groups))
    ms = time_events(pre.run, steps, warm)
    tok = wl.batch * wl.seq_len
    D = feature_count(64)
    flops = tok * 2 * wl.n_q_heads * 2 * D * (DV + 1)
    out["c5_long_prefill"] = {"ms": ms, "tokens_per_s": tok / (ms * 1e-3),
                              "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del pre, q, k, v
    # batched decode: 256 sequences x 16 heads, fp32 states (2145 x 65 each)
    S_, H = 256, 16
    g = torch.Generator(device="cuda").manual_seed(1205)
    state = torch.rand((S_, H, D * (DV + 1)), generator=g, device="cuda", dtype=torch.float32)
    mk = lambda *shape: torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    qd, kd, vd = mk(S_, H, 64), mk(S_, H, 64), mk(S_, H, 64)
    groups = ((torch.arange(64) * 8) // 64).repeat(H, 1).numpy()
    wl5 = S.make(5, seq_len=8, batch=1)
    dec = oal.DecodePlan(qd, kd, vd, coeffs_for(wl5, groups), state)
    ms = time_events(dec.run, max(10, args.steps), 3)
    nbytes = 2 * S_ * H * D * (DV + 1) * 4 + (3 * S_ * H * 64 + S_ * H * 64) * 2
    out["c5_decode_256x16"] = {"ms": ms, "tokens_per_s": S_ / (ms * 1e-3),
                               "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                               "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return out


def run_pmc_target(args):
    """Launch only one kernel repeatedly, for rocprofv3 counter passes.

    ``readout``: the chunk readout of the main workload (after one states
    pass); ``states``: the chunk scan of the main workload; ``based16``: the
    one-pass prefill of the d_h = 16 Based Taylor workload (B=8, H=16,
    N=8192); ``rebased``: the one-pass prefill of the ReBased workload in the
    dimension-wise form (B=16, H=8, N=2048); ``long``: the prefill of the
    long-context multi-head workload (B=1, H=16, N=32768, d_h=64, eight
    groups from its contribution scores); ``copy``: a plain device copy of
    1 GiB (fp32), whose FETCH_SIZE and WRITE_SIZE readings calibrate the
    counters against a known byte count."""
    import torch
    import grouped_quadratic_softmax_amd as oal
    import synthetic as S

    if args.pmc_target == "copy":
        n = COPY_BYTES // 4
        src = torch.ones(n, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_target": "copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                          "launches": args.steps}), flush=True)
        return
    if args.pmc_target == "long":
        wl = S.make(5)
        q, k, v = device_inputs(wl)
        chi = oal.contrib(q, k).cpu().numpy()
        groups = oal.groups_from_contribution(chi, wl.group_budget["bulk_sizes"], wl.group_budget["n_tail"])
        pre = oal.PrefillPlan(q, k, v, coeffs_for(wl, groups))
        torch.cuda.synchronize()
        for _ in range(args.steps):
            pre.run()
        torch.cuda.synchronize()
        print(json.dumps({"pmc_target": args.pmc_target, "launches": args.steps}), flush=True)
        return
    if args.pmc_target in ("based16", "rebased"):
        wl = S.make(3 if args.pmc_target == "based16" else 4)
        q, k, v = device_inputs(wl)
        p = wl.premap
        prep = (oal.Prep(p["gamma_q"], p["beta_q"], p["gamma_k"], p["beta_k"], p["ln_eps"])
                if p is not None else None)
        pre = oal.PrefillPlan(q, k, v, coeffs_for(wl), prep)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            pre.run()
        torch.cuda.synchronize()
        print(json.dumps({"pmc_target": args.pmc_target, "launches": args.steps}), flush=True)
        return
    wl = S.make(2, seq_len=2048 + 1)
    N = wl.seq_len - 1
    q, k, v = (t[:, :, :N].contiguous() for t in device_inputs(wl))
    pre = oal.PrefillPlan(q, k, v, coeffs_for(wl))
    pre.states()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        if args.pmc_target == "readout":
            pre.outputs()
        else:
            pre.states()
    torch.cuda.synchronize()
    print(json.dumps({"pmc_target": args.pmc_target, "launches": args.steps}), flush=True)


def cpu_baseline(wl, min_seconds=10.0):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload:
    whole sequences of it (every query head, every token), repeated until at
    least ``min_seconds`` of host time have passed."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    N = wl.seq_len - 1
    a, b, c = O.coeffs_from_factor(wl.coeff["eps"], wl.coeff["L"])
    done = 0
    t0 = time.perf_counter()
    while True:
        bi = done % wl.batch
        qs, ks, vs = (x[bi:bi + 1, :, :N] for x in (wl.q, wl.k, wl.v))
        O.chi_separable(qs, ks)
        O.attention_direct(qs, ks, vs, wl.group_of_dim, a, b, c)
        st = np.stack([np.stack([O.state_from_prefix(ks[0, kh], vs[0, kh]) for kh in range(wl.n_kv_heads)])])
        O.decode_step(st, wl.q[bi:bi + 1, :, N], wl.k[bi:bi + 1, :, N], wl.v[bi:bi + 1, :, N], wl.group_of_dim,
                      a, b, c, wl.n_q_heads)
        done += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    tokens = done * (N + 1)
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "seconds": dt,
            "sample": f"{done} sequence(s) of the workload ({N} prefill tokens + 1 decoded token each, all "
                      f"{wl.n_q_heads} query heads): chi (separable form), direct O(N^2) fp64 attention, prefix "
                      "states, one decode step; repeated until >= 10 s of host time"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run chi, prefill and decode back to back on one stream")
    ap.add_argument("--pmc-target", choices=("readout", "states", "based16", "rebased", "long", "copy"), default=None,
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
    result, wl = run_main(args)
    print(f"[bench] main done: {result['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
    if not args.no_secondary:
        result["secondary"] = run_secondary(args)
        print("[bench] secondary done", file=sys.stderr, flush=True)
    result["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
