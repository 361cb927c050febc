#!/usr/bin/env python3
"""Benchmark of the RIB window-attention hot path on one MI355X (gfx950).

One step is one pass of the forward hot path over the 96x96-window workload
(batch 4, 192x192 map, 6 heads, d_c = 32, r = 16, bf16; 16 windows, 96
(batch, window, head) units): posgen of (Q_p, K_p), the window gathers of
K_c and V, and the fused RIB attention kernel, which reads Q_c and writes O
in the map layout itself. Inputs are seeded synthetic tensors already
resident in HBM.

Reported (one JSON line): TFLOP/s of algorithmic work (2 N^2 (2 d_c + r) per
unit, padding and softmax not counted) over the whole step, windows/s, % of
the bf16 dense MFMA peak, a roofline entry for the attention kernel (timed
with HIP events on its own stream), per-kernel GB/s of the gathers and
posgen, and the float64 CPU oracle timed on a bounded sample of units as a
baseline; the relative-position-bias comparison kernel on the same inputs
(--no-rpb skips it); with --stack also the window-size stack (windows
16/32/64/96, forward + backward).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--stack]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "RIB window-attn TFLOP/s + windows/s at 96x96 bf16; % of MFMA bf16 peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_w96_traffic.json")
ATTN_SRC = os.path.join(ROOT, "windowed_attention_implicit_amd", "csrc", "attn_fwd.hip")


def fwd_flops(units: int, N: int, d_c: int, r: int) -> int:
    return units * 2 * N * N * (2 * d_c + r)


def bwd_flops(units: int, N: int, d_c: int, r: int) -> int:
    return units * 2 * N * N * (5 * d_c + 3 * r)


def to_gpu(t, dev):
    import numpy as np
    import torch
    if t.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(dev)


class FwdStep:
    """posgen + forward call with every buffer preallocated; run() enqueues one step."""

    def __init__(self, wl, x, dev):
        import torch
        import windowed_attention_implicit_amd as rib
        self.rib, self.wl = rib, wl
        self.q, self.k, self.v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
        self.w1 = torch.from_numpy(x["w1"]).to(dev)
        self.w2 = torch.from_numpy(x["w2"]).to(dev)
        self.mlp = rib._Mlp(wl.n_freq, wl.hidden, wl.r, self.w1.data_ptr(), None, self.w2.data_ptr(), None)
        dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        self.pos_code = rib.RIB_F32 if wl.dtype == "f32" else rib.RIB_BF16
        self.qp = torch.empty((wl.N, wl.r), dtype=dt, device=dev)
        self.kp = torch.empty_like(self.qp)
        self.plan = rib.FwdPlan(self.q, self.k, self.v, self.qp, self.kp, wl.w)

    def run(self):
        L = self.rib.lib()
        st = self.rib._stream(self.q.device)
        self.rib._check(L.rib_posgen(self.wl.w, ctypes.byref(self.mlp), self.pos_code,
                                     ctypes.c_void_p(self.qp.data_ptr()), ctypes.c_void_p(self.kp.data_ptr()), st))
        self.plan.run()


def time_steps(fn, steps: int, warmup: int, after_warmup=None):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if after_warmup is not None:
        after_warmup()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall / steps * 1e3


def kernel_avg_ms(rib, group):
    ms, n = rib.kernel_timing_read(group)
    return (ms / n if n else None), n


def cold_kernel_ms(fn, rib, groups, dev, n: int = 10):
    """Average kernel time of each group with the 256 MB last-level cache (MALL) flushed before every
    call: a 512 MiB buffer is overwritten between calls, so the inputs come from HBM."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    tot = {g: 0.0 for g in groups}
    for _ in range(n):
        flush.fill_(1)
        torch.cuda.synchronize()
        for g in groups:
            rib.kernel_timing_read(g)
        fn()
        for g in groups:
            tot[g] += rib.kernel_timing_read(g)[0]
    del flush
    return {g: tot[g] / n for g in groups}


def counter_record():
    """The committed counter run of the attention kernel (HBM bytes per launch, the shader clock and
    MFMA-busy fraction under counters), only while the kernel source is the one it was taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
        return rec if rec.get("kernel_source_sha256") == sha else None
    except (OSError, ValueError):
        return None


def step_distribution(fn, n: int, rib):
    """Per-step times of n more steps, each bracketed by its own events (outside the timed region):
    p10 / median / p90 of the step and of the attention kernel launch."""
    import numpy as np
    import torch
    step, attn = [], []
    rib.kernel_timing_read("attn_fwd")
    for _ in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        step.append(a.elapsed_time(b))
        t, k = rib.kernel_timing_read("attn_fwd")
        attn.append(t / k if k else float("nan"))
    pct = lambda xs: {f"p{p}": round(float(np.percentile(xs, p)), 5) for p in (10, 50, 90)}
    return {"steps": n, "step_ms": pct(step), "attn_kernel_ms": pct(attn)}


def cpu_baseline(wl, x, n_units: int):
    """The float64 oracle, as it stands, on n_units (batch, window, head) units of the workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = max((p.get("num_threads", 1) for p in blas), default=1)
        blas_name = ",".join(f"{p.get('internal_api')} {p.get('version')}" for p in blas)
    except Exception:  # noqa: BLE001
        cores, blas_name = os.cpu_count(), "unknown"
    units = [(b, wy, wx, h) for b in range(wl.B) for wy in range(wl.H // wl.w)
             for wx in range(wl.W // wl.w) for h in range(wl.heads)]
    step = max(1, len(units) // n_units)
    sample = units[::step][:n_units]
    qc, kc, v = (x[n].f64() for n in ("q_c", "k_c", "v"))
    qp, kp = oracle.posgen(wl.w, wl.n_freq, x["w1"], None, x["w2"], None, wl.r)
    t0 = time.perf_counter()
    oracle.rib_window_attn_fwd(qc, kc, v, qp, kp, wl.w, units=sample)
    dt = time.perf_counter() - t0
    flops = fwd_flops(len(sample), wl.N, wl.d_c, wl.r)
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
        "sample": (f"{len(sample)} of {len(units)} (batch, window, head) units of the 96x96 workload, forward, "
                   f"float64 numpy with the explicit N x N score matrix; {dt:.2f} s"),
        "windows_per_s": len(sample) / wl.heads / dt, "seconds": dt, "blas": blas_name,
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def stack_measure(steps: int, warmup: int, dev):
    """One training step of the window-size stack (16, 32, 64, 96), per layer and total: posgen,
    attention forward, attention backward and the position-MLP weight gradients. The weights change
    every training step, so posgen runs every step (the forward plans keep the tokens of the same
    weights)."""
    import torch
    import rib_synth
    import windowed_attention_implicit_amd as rib
    xs = rib_synth.make_stack_inputs()
    layers = []
    for wl, x in zip(rib_synth.STACK, xs):
        q, k, v, do = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v", "d_o"))
        w1, w2 = torch.from_numpy(x["w1"]).to(dev), torch.from_numpy(x["w2"]).to(dev)
        qp, kp = rib.posgen(wl.w, w1, None, w2, None, wl.r, out_dtype=torch.bfloat16)
        fp = rib.FwdPlan(q, k, v, qp, kp, wl.w)
        o, lse = fp.run()
        bp = rib.BwdPlan(q, k, v, qp, kp, o, lse, do, wl.w)
        bp.run()

        def mlp_fwd(wl=wl, w1=w1, w2=w2):
            return rib.posgen(wl.w, w1, None, w2, None, wl.r, out_dtype=torch.bfloat16)

        def mlp_bwd(wl=wl, w1=w1, w2=w2, bp=bp):
            return rib.posgen_bwd(wl.w, w1, None, w2, None, wl.r, bp.dqp, bp.dkp)
        layers.append((wl, fp, bp, mlp_fwd, mlp_bwd))

    def run_all():
        for _, fp, bp, mlp_fwd, mlp_bwd in layers:
            mlp_fwd()
            fp.run()
            bp.run()
            mlp_bwd()

    def reset():
        for g in rib.KERNEL_GROUPS:
            rib.kernel_timing_read(g)

    # step and per-layer times with no kernel-timing events in the stream; the kernel breakdown
    # comes from loops of its own with every group timed
    rib.kernel_timing_enable(False)
    ms, _ = time_steps(run_all, steps, warmup, reset)
    rib.kernel_timing_enable(True)
    time_steps(run_all, steps, 2, reset)
    pg = [kernel_avg_ms(rib, g)[0] for g in ("posgen", "posgen_bwd")]
    per = []
    for wl, fp, bp, _, mlp_bwd in layers:
        rib.kernel_timing_enable(False)
        t_f, _ = time_steps(fp.run, steps, 2)
        t_b, _ = time_steps(bp.run, steps, 2)
        rib.kernel_timing_enable(True)
        time_steps(mlp_bwd, steps, 2, reset)
        pgb, _ = kernel_avg_ms(rib, "posgen_bwd")
        time_steps(fp.run, steps, 2, reset)
        fa, _ = kernel_avg_ms(rib, "attn_fwd")
        time_steps(bp.run, steps, 2, reset)
        dkv, _ = kernel_avg_ms(rib, "attn_bwd_dkv")
        dq, _ = kernel_avg_ms(rib, "attn_bwd_dq")
        gath, _ = kernel_avg_ms(rib, "partition")   # the one-pass backward gather (with -D, -LSE2)
        ff, bf = fwd_flops(wl.units, wl.N, wl.d_c, wl.r), bwd_flops(wl.units, wl.N, wl.d_c, wl.r)
        per.append({"w": wl.w, "fwd_ms": round(t_f, 4), "bwd_ms": round(t_b, 4),
                    "fwd_tflops": round(ff / t_f / 1e9, 1), "bwd_tflops": round(bf / t_b / 1e9, 1),
                    "attn_fwd_kernel_ms": fa and round(fa, 4), "bwd_dkv_kernel_ms": dkv and round(dkv, 4),
                    "bwd_dq_kernel_ms": dq and round(dq, 4), "bwd_gather_kernel_ms": gath and round(gath, 4),
                    "bwd_kernels_tflops": (dkv and dq) and round(bf / (dkv + dq) / 1e9, 1),
                    "posgen_bwd_kernels_ms": pgb and round(pgb, 4)})
    rib.kernel_timing_enable(False)
    total = sum(fwd_flops(wl.units, wl.N, wl.d_c, wl.r) + bwd_flops(wl.units, wl.N, wl.d_c, wl.r)
                for wl, *_ in layers)
    return {"workload": "window-size stack 16/32/64/96 on a 192x192 map, batch 2, 6 heads, d_c=32, r=16, bf16, "
                        "training step: posgen + forward + backward + position-MLP weight gradients",
            "ms_per_step": round(ms, 4), "tflops": round(total / ms / 1e9, 1),
            "posgen_ms_avg": pg[0] and round(pg[0], 4), "posgen_bwd_ms_avg": pg[1] and round(pg[1], 4),
            "layers": per}


def group_ms(fn, steps: int, groups):
    """Average per-call time of each kernel group of fn, from a loop of its own with every group timed."""
    import windowed_attention_implicit_amd as rib
    rib.kernel_timing_enable(True)
    for g in rib.KERNEL_GROUPS:
        rib.kernel_timing_read(g)
    time_steps(fn, steps, 2, lambda: [rib.kernel_timing_read(g) for g in rib.KERNEL_GROUPS])
    out = {}
    for g in groups:
        t, n = rib.kernel_timing_read(g)
        out[g] = round(t / steps, 5) if n else None
    rib.kernel_timing_enable(False)
    return out


def configs_measure(steps: int, dev):
    """The other forward workloads the method is measured on (single 16x16 window in float32; 32x32
    windows on a 256x256 map, 6 heads, r = 8; 64x64 windows on a 128x128 map x 8, r = 16): one
    step = posgen + gathers + attention (+ split-tail combine), the same step as the headline."""
    import rib_synth
    import windowed_attention_implicit_amd as rib
    out = {}
    for name in ("w16_single_fp32", "w32_map256_bf16", "w64_map128x8_bf16"):
        wl = rib_synth.WORKLOADS[name]
        x = rib_synth.make_inputs(wl)
        step = FwdStep(wl, x, dev)
        rib.kernel_timing_enable(False)
        ms, _ = time_steps(step.run, steps, 5)
        groups = group_ms(step.run, steps, ("posgen", "partition", "attn_fwd", "unpartition"))
        flops = fwd_flops(wl.units, wl.N, wl.d_c, wl.r)
        ktot = sum(v for v in groups.values() if v)
        out[name] = {
            "workload": (f"{wl.windows} window(s) of {wl.w}x{wl.w} (N={wl.N}) on a {wl.H}x{wl.W} map x {wl.B}, "
                         f"{wl.heads} heads, d_c={wl.d_c}, r={wl.r}, {wl.dtype}"),
            "ms_per_step": round(ms, 5), "tflops": round(flops / ms / 1e9, 3),
            "windows_per_s": round(wl.windows / (ms / 1e3), 1), "window_heads_per_s": round(wl.units / (ms / 1e3), 1),
            "pct_of_bf16_peak": round(100 * flops / ms / 1e9 / PEAK_BF16_TFLOPS, 2) if wl.dtype == "bf16" else None,
            "kernel_ms": groups,
            "attn_kernel_tflops": groups["attn_fwd"] and round(flops / groups["attn_fwd"] / 1e9, 1),
            "gather_share_of_kernel_time": groups["partition"] and round(groups["partition"] / ktot, 3),
            "note": ("kernel groups: posgen; partition = the K/V gather (+ packing of Q_p, K_p when r is not 16 or "
                     "32); attn_fwd = the attention kernel; unpartition = the split-tail combine (bf16) or the O "
                     "scatter (float32); the gaps between launches are the rest of the step"),
        }
    return out


def tiers_measure(wl, x, dev, steps: int):
    """What the bounded softmax costs when it cannot go unshifted, on the headline shape: Q_c and K_c
    scaled by 3 (score bounds above 64 log2 units: the shifted tier), and one key per window with 127
    in channel 0 (bounds ~150 log2 units above most rows' largest score: row sums underflow the guard
    and every workgroup leaves the fast pass after two key tiles for the exact online-softmax pass)."""
    import torch
    import windowed_attention_implicit_amd as rib
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    w1, w2 = torch.from_numpy(x["w1"]).to(dev), torch.from_numpy(x["w2"]).to(dev)
    qp, kp = rib.posgen(wl.w, w1, None, w2, None, wl.r, out_dtype=torch.bfloat16)
    k_big = k.clone()
    k_big[:, ::wl.w, ::wl.w, :, 0] = 127.0
    cases = {"unshifted (N(0,1) inputs)": (q, k), "shifted (Q_c, K_c x 3)": ((q.float() * 3).to(torch.bfloat16),
                                                                          (k.float() * 3).to(torch.bfloat16)),
             "exact pass (one key per window with 127 in channel 0)": (q, k_big)}
    plans = {name: rib.FwdPlan(qq, kk, v, qp, kp, wl.w) for name, (qq, kk) in cases.items()}
    rib.kernel_timing_select("attn_fwd")
    res = {}
    for name, plan in plans.items():
        for _ in range(2):
            plan.run()
        torch.cuda.synchronize()
        rib.kernel_timing_read("attn_fwd")
        for _ in range(steps):
            plan.run()
        t, n = rib.kernel_timing_read("attn_fwd")
        res[name] = round(t / n, 5)
    rib.kernel_timing_select()
    base = res["unshifted (N(0,1) inputs)"]
    return {"attn_kernel_ms": res, "slowdown": {k2: round(v2 / base, 3) for k2, v2 in res.items()}}


def rpb_compare(wl, x, dev, steps: int, rib_attn_ms: float):
    """The relative-position-bias attention that RIB replaces, on the same Q_c, K_c, V: the RPB
    kernel (bias gathered per score from an fp16 (2w-1)^2 table in LDS) against the RIB attention
    kernel, and the parameter / materialized-bias memory of both forms."""
    import torch
    import rib_synth
    import windowed_attention_implicit_amd as rib
    q, k, v = (to_gpu(x[n], dev) for n in ("q_c", "k_c", "v"))
    table = torch.from_numpy(rib_synth.make_rpb_table(wl.heads, wl.w, seed=96)).to(dev)
    plan = rib.RpbFwdPlan(q, k, v, table, wl.w)

    def reset():
        for g in rib.KERNEL_GROUPS:
            rib.kernel_timing_read(g)

    rib.kernel_timing_enable(True)
    ms, _ = time_steps(plan.run, steps, 3, reset)
    kern, _ = kernel_avg_ms(rib, "rpb_attn_fwd")
    rib.kernel_timing_enable(False)
    content_flops = 2 * wl.units * wl.N * wl.N * 2 * wl.d_c
    n_tab = (2 * wl.w - 1) ** 2
    return {"workload": "same Q_c, K_c, V as the headline workload; N(0,1) tables [heads, (2w-1)^2]",
            "rpb_call_ms": round(ms, 4), "rpb_attn_kernel_ms": kern and round(kern, 4),
            "rib_attn_kernel_ms": round(rib_attn_ms, 4),
            "rpb_over_rib_kernel_time": kern and round(kern / rib_attn_ms, 3),
            "rpb_content_tflops": kern and round(content_flops / kern / 1e9, 1),
            "rpb_table_params_per_layer": wl.heads * n_tab,
            "rib_mlp_params_per_layer": wl.hidden * 4 * wl.n_freq + wl.hidden + 2 * wl.r * wl.hidden + 2 * wl.r,
            "materialized_bias_bytes_bf16": wl.heads * wl.N * wl.N * 2}


def cla_gate_only(wl, dev, steps: int, warmup: int):
    """The CLA gate alone on the headline map (C = heads * d_c = 192): kernel time and rates."""
    import torch
    import rib_synth
    import windowed_attention_implicit_amd as rib
    C = wl.heads * wl.d_c
    xm = to_gpu(rib_synth.make_map(wl.B, wl.H, wl.W, C, "bf16", seed=192), dev)
    w = {k: torch.from_numpy(v).to(dev) for k, v in rib_synth.make_cla(C, seed=193).items()}
    g = torch.empty_like(xm)

    def gate():
        rib.cla_gate(xm, w["w_dw"], w["b_dw"], w["w_pw"], w["b_pw"], wl.heads, out=g)

    def reset():
        for grp in rib.KERNEL_GROUPS:
            rib.kernel_timing_read(grp)

    rib.kernel_timing_enable(True)
    time_steps(gate, steps, warmup, reset)
    gate_ms, n = kernel_avg_ms(rib, "cla_gate")
    rib.kernel_timing_enable(False)
    tensor_bytes = wl.B * wl.H * wl.W * C * 2
    flops = wl.B * wl.H * wl.W * (2 * 9 * C + 2 * C * C)
    return {"workload": f"gate of a [{wl.B}, {wl.H}, {wl.W}, {C}] bf16 map", "launches": n,
            "gate_kernel_ms": round(gate_ms, 5), "gate_GB/s": round(2 * tensor_bytes / gate_ms / 1e6, 1),
            "gate_frac_hbm": round(2 * tensor_bytes / gate_ms / 1e6 / PEAK_HBM_GBS, 3),
            "gate_tflops": round(flops / gate_ms / 1e9, 1)}


def cla_measure(wl, x, step, dev, steps: int):
    """The CLA gate on the headline map (C = heads * d_c = 192) and the forward with O' = O * G fused into
    the attention kernel's output stage."""
    import torch
    import rib_synth
    import windowed_attention_implicit_amd as rib
    C = wl.heads * wl.d_c
    xm = to_gpu(rib_synth.make_map(wl.B, wl.H, wl.W, C, "bf16", seed=192), dev)
    w = {k: torch.from_numpy(v).to(dev) for k, v in rib_synth.make_cla(C, seed=193).items()}
    g = rib.cla_gate(xm, w["w_dw"], w["b_dw"], w["w_pw"], w["b_pw"], wl.heads)
    plan = step.plan
    q, k, v, qp, kp = plan.inputs
    o_gated = torch.empty_like(plan.o)
    L = rib.lib()

    def gate():
        rib.cla_gate(xm, w["w_dw"], w["b_dw"], w["w_pw"], w["b_pw"], wl.heads, out=g)

    def gated():
        rib._check(L.rib_window_attn_fwd_gated(ctypes.byref(plan.shape), plan.dtype, plan.scale, rib._ptr(q),
                                               rib._ptr(k), rib._ptr(v), rib._ptr(qp), rib._ptr(kp), rib._ptr(g),
                                               rib._ptr(o_gated), rib._ptr(plan.lse), rib._ptr(plan.ws),
                                               plan.ws_bytes, rib._stream(dev)))

    def reset():
        for grp in rib.KERNEL_GROUPS:
            rib.kernel_timing_read(grp)

    rib.kernel_timing_enable(True)
    time_steps(gate, steps, 3, reset)
    gate_ms, _ = kernel_avg_ms(rib, "cla_gate")
    # gated and ungated launches alternate, so both see the same clock and cache state
    for _ in range(3):
        plan.run()
        gated()
    torch.cuda.synchronize()
    reset()
    t_plain = t_gated = 0.0
    for _ in range(steps):
        plan.run()
        t_plain += rib.kernel_timing_read("attn_fwd")[0]
        gated()
        t_gated += rib.kernel_timing_read("attn_fwd")[0]
    rib.kernel_timing_enable(False)
    gated_ms, rib_attn_ms = t_gated / steps, t_plain / steps
    tensor_bytes = wl.B * wl.H * wl.W * C * 2
    pixels = wl.B * wl.H * wl.W
    flops = pixels * (2 * 9 * C + 2 * C * C)
    return {"workload": f"gate of a [{wl.B}, {wl.H}, {wl.W}, {C}] bf16 map; gated forward on the headline inputs",
            "gate_kernel_ms": gate_ms and round(gate_ms, 5),
            "gate_GB/s": gate_ms and round(2 * tensor_bytes / gate_ms / 1e6, 1),
            "gate_frac_hbm": gate_ms and round(2 * tensor_bytes / gate_ms / 1e6 / PEAK_HBM_GBS, 3),
            "gate_tflops": gate_ms and round(flops / gate_ms / 1e9, 1),
            "gated_attn_kernel_ms": round(gated_ms, 5),
            "ungated_attn_kernel_ms_same_loop": round(rib_attn_ms, 5)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=40)
    ap.add_argument("--stack", action="store_true",
                    help="also time the window-size stack 16/32/64/96, forward + backward")
    ap.add_argument("--no-rpb", action="store_true",
                    help="skip the relative-position-bias comparison kernel")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other forward workloads (16x16 float32, 32x32, 64x64 windows)")
    ap.add_argument("--only-headline", action="store_true",
                    help="time the headline step only (no CLA, tiers, other workloads, RPB, stack or CPU "
                         "baseline): the command the profiler runs")
    ap.add_argument("--only-cla", action="store_true",
                    help="time the CLA gate on the headline map only and print its record (the command the "
                         "gate's counter runs use)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported - no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import torch
    import rib_synth
    import windowed_attention_implicit_amd as rib

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    wl = rib_synth.HEADLINE
    if args.only_cla:
        print(json.dumps({"cla": cla_gate_only(wl, dev, args.steps, args.warmup)}), flush=True)
        return
    x = rib_synth.make_inputs(wl)
    step = FwdStep(wl, x, dev)
    print(f"bench: {wl.name} units={wl.units} N={wl.N}", file=sys.stderr, flush=True)

    for _ in range(3):
        step.run()
    torch.cuda.synchronize()

    def reset():
        for g in rib.KERNEL_GROUPS:
            rib.kernel_timing_read(g)

    # Inside the timed steps only the attention kernel is bracketed by events (its launch time is
    # the roofline's); every event pair costs a few microseconds of idle GPU between launches.
    rib.kernel_timing_select("attn_fwd")
    ms, wall_ms = time_steps(step.run, args.steps, args.warmup, reset)
    attn_ms, attn_n = kernel_avg_ms(rib, "attn_fwd")
    dist = step_distribution(step.run, max(50, args.steps), rib)
    # the other groups' kernel times, from a loop of their own
    rib.kernel_timing_enable(True)
    time_steps(step.run, args.steps, 2, reset)
    part_ms, _ = kernel_avg_ms(rib, "partition")
    unp_ms, _ = kernel_avg_ms(rib, "unpartition")
    pg_ms, _ = kernel_avg_ms(rib, "posgen")
    cold = cold_kernel_ms(step.run, rib, ("posgen", "partition"), dev)
    rib.kernel_timing_enable(False)
    print(f"bench: step {ms:.4f} ms, attention kernel {attn_ms:.4f} ms over {attn_n} launches",
          file=sys.stderr, flush=True)

    flops = fwd_flops(wl.units, wl.N, wl.d_c, wl.r)
    tflops = flops / ms / 1e9
    attn_tflops = flops / attn_ms / 1e9
    tensor_bytes = wl.B * wl.H * wl.W * wl.heads * wl.d_c * 2
    # one pass gathers K and V (read + write each) and takes the key-norm maxima from the K_c it moves;
    # Q_c is read and O written in the map layout by the attention kernel itself, and Q_p, K_p are read
    # in place unless r needs padding to 16 or 32 (then they are packed: read + write each)
    part_bytes = 4 * tensor_bytes + (0 if wl.r in (16, 32) else 4 * wl.N * wl.r * 2)
    pg_bytes = 4 * (wl.hidden * 4 * wl.n_freq + 2 * wl.r * wl.hidden) + 2 * wl.N * wl.r * 2
    rec = counter_record()
    traffic = rec and rec.get("hbm_bytes_per_launch")
    sclk = rec and rec.get("sclk_ghz_under_counters")

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "RIB window attention forward, 96x96 windows: batch 4, 192x192 map, 6 heads, "
                               "d_c=32, r=16, bf16 (16 windows, 96 units of N=9216)",
                   "B": wl.B, "H": wl.H, "W": wl.W, "heads": wl.heads, "d_c": wl.d_c, "w": wl.w, "r": wl.r,
                   "windows": wl.windows, "units": wl.units, "parallelism": "single GPU"},
        "windows_per_s": round(wl.windows / (ms / 1e3), 1),
        "window_heads_per_s": round(wl.units / (ms / 1e3), 1),
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "attn_fwd_bf16_kernel", "flops_per_launch": flops,
                     "avg_launch_ms": round(attn_ms, 5),
                     # 4096 bf16 flop/clk/CU x 256 CUs at the shader clock the kernel ran at under counters
                     "sclk_ghz_under_counters": sclk,
                     "peak_at_that_clock": sclk and round(4.096 * 256 * sclk, 1),
                     "frac_at_that_clock": sclk and round(attn_tflops / (4.096 * 256 * sclk), 4),
                     "mfma_busy_under_counters": rec and rec.get("mfma_busy_frac")},
        "distribution": dist,
        "kernels": {
            "posgen": {"ms": pg_ms and round(pg_ms, 5), "GB/s": pg_ms and round(pg_bytes / pg_ms / 1e6, 1),
                       "cold_ms": round(cold["posgen"], 5)},
            "partition": ({"ms": None, "note": "none: the attention kernel reads K_c and V in their maps at this "
                                                "window size and rank (Q_p, K_p in place)"} if part_ms is None else
                          {"ms": round(part_ms, 5), "GB/s": round(part_bytes / part_ms / 1e6, 1),
                           "frac_hbm": round(part_bytes / part_ms / 1e6 / PEAK_HBM_GBS, 3),
                           "cold_ms": round(cold["partition"], 5),
                           "cold_GB/s": round(part_bytes / cold["partition"] / 1e6, 1),
                           "note": "GB/s over one read + one write of K_c and V (the key-norm maxima come from the "
                                   "same pass); cold_* with the 256 MB MALL flushed before each call"}),
            "attn_fwd": {"ms": round(attn_ms, 5), "TFLOP/s": round(attn_tflops, 1)},
            "unpartition": ({"ms": None, "note": "none: O rows are written in the map layout by the attention "
                                                 "kernel"} if unp_ms is None else
                            {"ms": round(unp_ms, 5),
                             "note": "the split-tail combine: the key-range pieces of each XCD's last partial round "
                                     "of work items summed into O and LSE (the attention kernel writes the other "
                                     "rows in the map layout itself)"}),
        },
        "host_ms_per_step": round(wall_ms, 4),
    }

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = 2 * n * 4

    if args.only_headline:
        args.no_configs = args.no_rpb = args.no_cpu_baseline = True
        args.stack = False
    else:
        print("bench: CLA gate", file=sys.stderr, flush=True)
        result["cla"] = cla_measure(wl, x, step, dev, max(10, args.steps // 2))
        print("bench: softmax tiers", file=sys.stderr, flush=True)
        result["softmax_tiers"] = tiers_measure(wl, x, dev, max(10, args.steps // 2))

    if not args.no_configs:
        print("bench: other workloads", file=sys.stderr, flush=True)
        result["configs"] = configs_measure(max(10, args.steps // 2), dev)

    if not args.no_rpb:
        print("bench: RPB comparison kernel", file=sys.stderr, flush=True)
        result["rpb_compare"] = rpb_compare(wl, x, dev, max(10, args.steps // 2), attn_ms)

    if args.stack:
        print("bench: window-size stack fwd+bwd", file=sys.stderr, flush=True)
        result["stack_fwd_bwd"] = stack_measure(max(5, args.steps // 3), 2, dev)

    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_units)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
