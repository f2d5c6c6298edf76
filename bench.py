#!/usr/bin/env python3
"""Benchmark of the quantized attention forward pass on one MI355X.

One step = the whole hot path on one batch already resident in HBM:
sage_quant_qkv (smooth K + INT8 Q/K + FP8 V, three launches) and sage_attn_fwd.
Default workload: the sequence-sweep configuration at N = 32768
(B=4, H=32, d=128, fp16, non-causal), the one the headline TOPS is quoted on.

Prints ONE JSON line.  ``value`` is whole-step TOPS, 4*B*H*N^2*d / t_step
(halved when causal), t_step from replays of the step captured as a HIP graph
(``--eager``: from eager launches; ``ms_per_step_eager`` is always reported);
``attn_tops`` is the attention kernel alone (the pages' convention:
quantization time excluded), from the mean of the per-step HIP-event times of
the eager steps; ``attn_tops_median`` takes their median (20 steps by default).
``roofline`` is the attention
kernel's algorithmic TOPS against the dense INT8/FP8 MFMA peak, with the
kernel time measured by HIP events on the launch stream.  ``cpu_baseline``
times the float64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TOPS = 5000.0          # MI355X dense INT8 (POPS) / FP8 (PFLOPS) peak, in T/s
HBM_GBS = 8000.0


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("attn_fwd.hip", "sage_device.hpp"):
        with open(os.path.join(ROOT, "quantized_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per attn_fwd launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel_source_hash:\s*(\w+)", txt)
    w = re.search(r"workload:\s*(\S+)", txt)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m and t and w) or m.group(1) != kernel_source_hash() or w.group(1) != workload:
        return None
    return float(t.group(1))


def cpu_baseline(w, budget_s: float = 15.0) -> dict:
    """Time the oracle on one (b, head) slice: its quantization plus the
    quantized attention of a block of query rows against all N keys."""
    import numpy as np
    import workloads as W
    from oracle import sage_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    t = W.generate(w, heads=[(0, 0)])
    q, k, v = t["q"][:, :1], t["k"][:, :1], t["v"][:, :1]
    t0 = time.perf_counter()
    qz = O.quantize_qk(q, k)
    vz = O.quantize_v(v)
    t_quant = time.perf_counter() - t0
    rows_done, t_attn, r0 = 0, 0.0, 0
    blk = 256
    while t_attn < budget_s and r0 < w.N:
        rows = np.arange(r0, min(r0 + blk, w.N))
        t1 = time.perf_counter()
        O.attn_quant(qz["q_i8"], qz["q_scale"], qz["k_i8"], qz["k_scale"], vz["v_f8"],
                     vz["v_scale"], causal=w.causal, sm_scale=w.sm_scale, rows=rows)
        t_attn += time.perf_counter() - t1
        rows_done += len(rows)
        r0 += blk
    # per-head time: quantization + attention scaled from the sampled rows
    # (causal rows differ in cost; the sample starts at row 0, so for causal
    # workloads this under-counts and is marked as such)
    t_head = t_quant + t_attn * (w.N / rows_done)
    ops_head = w.ops() / (w.B * w.H)
    return {"value": ops_head / t_head / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": f"1 of {w.B * w.H} heads: quantize Q/K/V of the head ({t_quant:.2f} s) + "
                      f"quantized attention of {rows_done} of {w.N} query rows x {w.N} keys "
                      f"({t_attn:.2f} s), scaled to the head"
                      + (" (causal: rows from 0, cost under-counted)" if w.causal else "")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="sweep@N32768",
                    help="workload name: tiny, llm_prefill, video_dit, sweep@N<n>, gqa_long")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--lse", action="store_true",
                    help="also time the log-sum-exp path (sage_lse_correction + "
                         "sage_attn_fwd_lse) and report its cost beside the plain step")
    ap.add_argument("--all", action="store_true",
                    help="time every configuration (tiny, llm_prefill, video_dit, sweep N=1K..32K, "
                         "gqa_long) and print one JSON line each instead of the single result line")
    ap.add_argument("--q-group", type=int, default=128, choices=(128, 32, 1),
                    help="Q tokens per INT8 scale: 128 per block (default), 32 per wave, "
                         "1 per query")
    ap.add_argument("--smooth-q", action="store_true",
                    help="smooth Q by its 128-block means and add the Delta S term back "
                         "(sage_attn_fwd_smooth_q: Delta S passes and attention in chunks of Q "
                         "blocks; the Delta S passes are also timed alone)")
    ap.add_argument("--pv", default="fp8", choices=("fp8", "mxfp4"),
                    help="P V format: FP8 E4M3 (the method's) or MXFP4 on the FP4 matrix cores")
    ap.add_argument("--eager", action="store_true",
                    help="time the whole step as eager launches (default: replays of the step "
                         "captured as a HIP graph; the kernel split is always timed eagerly)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MiB",
                    help="only run a plain device-to-device copy of this many MiB (3 times), "
                         "to calibrate the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    if args.calib_copy:
        import torch
        n = args.calib_copy << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_attention_amd as qa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    qa.load_library()
    if args.all:
        names = ["tiny", "llm_prefill", "video_dit"] + [f"sweep@N{n}" for n in
                                                        (1024, 2048, 4096, 8192, 16384, 32768)]
        names.append("gqa_long")
        for name in names:
            r = run_config(W.get(name), max(args.steps, 20), args.warmup, q_group=args.q_group,
                           smooth_q=args.smooth_q, pv=args.pv, graph=not args.eager)
            print(json.dumps(r), flush=True)
        return
    res = run_config(W.get(args.config), args.steps, args.warmup, full=True,
                     q_group=args.q_group, smooth_q=args.smooth_q, pv=args.pv,
                     graph=not args.eager)
    res["roofline"]["mfma_loop"] = mfma_loop(res["attn_tops"])
    if args.lse:
        res["lse"] = run_lse(W.get(args.config), args.steps, args.warmup)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(W.get(args.config), args.cpu_budget)
    print(json.dumps(res), flush=True)


def mfma_loop(attn_tops: float) -> dict:
    """The dense MFMA rate a register-only loop sustains (sage_mfma_peak: 256 workgroups of
    4 waves, one wave per SIMD when each CU takes one workgroup; INT8 32x32x32 and FP8
    32x32x64), the clocks each MFMA took in a wave, the shader clock during the INT8 loop,
    and the attention kernel's fraction of the INT8 loop's rate and of the published peak
    scaled to that clock.  (The clock under the attention kernel itself comes from the
    GRBM_GUI_ACTIVE counter of a profiled run; the loop's may differ.)"""
    import numpy as np
    import torch
    import quantized_attention_amd as qa
    stream = torch.cuda.current_stream()
    out = {}
    for kind, name, iters in ((0, "i8", 48000), (1, "f8", 24000)):
        qa.sage_mfma_peak(kind, 200)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ops, clocks, sink, khz = qa.sage_mfma_peak(kind, iters)
        e1.record(stream)
        torch.cuda.synchronize()
        if not torch.all(sink == 64 * (32 if kind == 0 else 64) * iters):
            raise RuntimeError("sage_mfma_peak: accumulator sums are not the expected ones")
        c = clocks.cpu().numpy().astype(np.float64)
        out[name + "_tops"] = round(ops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        # shader clocks per MFMA in a wave (32 and 64 at the full rate of a SIMD); waves
        # that shared a SIMD take longer, which the spread shows
        out[name + "_clocks_per_mfma"] = round(float(np.median(c[:, 0])) / (4 * iters), 2)
        out[name + "_wave_clock_spread"] = round(float(c[:, 0].max() / c[:, 0].min()), 3)
        if kind == 0:
            out["clock_ghz"] = round(float(np.median(c[:, 0] / c[:, 1])) * khz / 1e6, 3)
    out["attn_frac_of_i8_loop"] = round(attn_tops / out["i8_tops"], 4)
    out["peak_at_loop_clock"] = round(PEAK_TOPS * out["clock_ghz"] / 2.4, 1)
    out["attn_frac_at_loop_clock"] = round(attn_tops / out["peak_at_loop_clock"], 4)
    return out


def run_lse(w, steps: int, warmup: int) -> dict:
    """Time the log-sum-exp path: the correction kernel and the attention kernel
    that also writes the LSE (against the plain attention kernel)."""
    import torch
    import quantized_attention_amd as qa
    import workloads as W
    dev = torch.device("cuda:0")
    t = W.generate(w)
    q, k, v = (t[n].to(dev) for n in ("q", "k", "v"))
    del t
    plan = qa.SagePlan(w.B, w.H, w.H_kv, w.N, w.d, w.torch_dtype, w.causal, device=dev)
    plan.quant(q, k, v)
    corr = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    lse = torch.empty_like(corr)
    stream = torch.cuda.current_stream(dev)
    run = lambda: (qa.sage_lse_correction(q, plan.qk["k_mean"], plan.sm_scale, out=corr),
                   qa.sage_attn_fwd_lse(plan.qk, plan.vq, causal=w.causal, sm_scale=plan.sm_scale,
                                        out_dtype=w.torch_dtype, lse_corr=corr, out=plan.o,
                                        lse=lse))
    for _ in range(warmup):
        run()
        plan.attn()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        qa.sage_lse_correction(q, plan.qk["k_mean"], plan.sm_scale, out=corr)
        e[1].record(stream)
        qa.sage_attn_fwd_lse(plan.qk, plan.vq, causal=w.causal, sm_scale=plan.sm_scale,
                             out_dtype=w.torch_dtype, lse_corr=corr, out=plan.o, lse=lse)
        e[2].record(stream)
        plan.attn()
        e[3].record(stream)
    torch.cuda.synchronize()
    t_c = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    t_al = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    t_a = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    corr_bytes = w.B * w.H * w.N * (2 * w.d + 4)      # read Q, write one float per row
    return {"lse_correction_ms": round(t_c, 4),
            "lse_correction_gbs": round(corr_bytes / (t_c * 1e-3) / 1e9, 1),
            "attn_fwd_lse_ms": round(t_al, 4), "attn_fwd_ms": round(t_a, 4),
            "attn_fwd_lse_tops": round(w.ops() / (t_al * 1e-3) / 1e12, 2)}


def delta_s_alone(plan, k, steps: int) -> float:
    """Milliseconds of the Delta S work sage_attn_fwd_smooth_q does per call, without the
    attention between its passes: every head and Q block, in chunks of Q-block rows that
    fill the plan's workspace. The entry point may instead split the same work into groups
    of whole heads (its chunk rule); the launches then cover the same rows in another order."""
    import torch
    import quantized_attention_amd as qa
    B, H, _, N, _ = plan.shape
    nmb = -(-N // qa.BLKQ)
    rows = min(nmb, plan.ws_sq.numel() // (B * H * N * 4))
    if 16 < rows < nmb:
        rows -= rows % 16
    ws = plan.ws_sq[:B * H * rows * N * 4].view(torch.float32)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        for i0 in range(0, nmb, rows):
            n = min(rows, nmb - i0)
            qa.sage_delta_s(k, plan.qk, plan.sm_scale, i0=i0, nrows=n,
                            out=ws[:B * H * n * N].view(B, H, n, N))
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def run_config(w, steps: int, warmup: int, full: bool = False, q_group: int = 128,
               smooth_q: bool = False, pv: str = "fp8", graph: bool = True) -> dict:
    """Time `steps` whole steps of workload `w` (inputs resident on the GPU): first as
    eager launches with HIP events between the quantization and the attention (the
    kernel split), then, with `graph`, as replays of the step captured as a HIP graph
    (the whole-step rate; the same launches without the host's per-launch cost)."""
    import torch
    import quantized_attention_amd as qa
    import workloads as W
    dev = torch.device("cuda:0")
    t = W.generate(w)
    q, k, v = (t[n].to(dev) for n in ("q", "k", "v"))
    del t
    plan = qa.SagePlan(w.B, w.H, w.H_kv, w.N, w.d, w.torch_dtype, w.causal, device=dev,
                       q_group=q_group, smooth_q=smooth_q, pv=pv)
    stream = torch.cuda.current_stream(dev)

    for _ in range(warmup):
        plan(q, k, v)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        e = ev[s]
        e[0].record(stream)
        if pv == "mxfp4":
            qa.sage_quant_qk(q, k, True, q_group=q_group, smooth_q=smooth_q, out=plan.qk,
                             workspace=plan.ws_qk)
            plan.quant_v(v)
        else:
            qa.sage_quant_qkv(q, k, v, True, q_group=q_group, smooth_q=smooth_q, out_qk=plan.qk,
                              out_v=plan.vq, workspace=plan.ws_qk)
        e[1].record(stream)
        e[2].record(stream)
        plan.attn()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    wall = wall_eager
    launch = "eager"
    if graph:
        try:
            g = plan.capture(q, k, v)
        except RuntimeError as e:   # capture unsupported here: report the eager steps
            torch.cuda.synchronize()
            g, launch = None, f"eager (HIP graph capture failed: {str(e)[:120]})"
        if g is not None:
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            launch = "hip graph replay"
            del g
    # smooth Q: the attention phase includes the Delta S passes; time them alone too
    t_ds = delta_s_alone(plan, k, steps) if smooth_q else 0.0

    t_q = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    t_attn = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    t_attn_med = statistics.median(e[2].elapsed_time(e[3]) for e in ev)
    ms_step = wall * 1e3 / steps
    ops = w.ops()
    attn_tops = ops / (t_attn * 1e-3) / 1e12
    # algorithmic bytes of the quantizers: read 2 B + write 1 B per element of Q, K and V
    quant_bytes = 3 * (w.B * w.H * w.N * w.d + 2 * w.B * w.H_kv * w.N * w.d)
    # the committed counters were taken with the default 128-token Q groups
    traffic = (traffic_from_profile(w.name) if q_group == 128 and not smooth_q and pv == "fp8"
               else None)

    res = {
        "metric": "quantized attn fwd TOPS at N=32K hd128 (4BHN^2d/t); % of MFMA INT8/FP8 peak",
        "value": round(ops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "step_launch": launch,
        "ms_per_step_eager": round(wall_eager * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8(QK^T)+f8e4m3(PV), f32 accumulate",
        "data": "synthetic (seeded normals, shared K channel bias)",
        "config": {"workload": w.description, "name": w.name, "B": w.B, "H": w.H,
                   "H_kv": w.H_kv, "N": w.N, "d": w.d, "causal": w.causal,
                   "in_dtype": w.dtype, "q_group": q_group, "smooth_q": smooth_q, "pv": pv},
        "attn_tops": round(attn_tops, 2),
        "attn_ms": round(t_attn, 4),
        "attn_ms_median": round(t_attn_med, 4),
        "attn_tops_median": round(ops / (t_attn_med * 1e-3) / 1e12, 2),
        "quant_ms": round(t_q, 4),
        "quant_share": round(t_q / (t_q + t_attn), 4),
        "quant_gbs": round(quant_bytes / (t_q * 1e-3) / 1e9, 1),
        # smooth Q: the Delta S passes inside attn_ms, timed alone, and the workspace
        "delta_s_ms": round(t_ds, 4) if smooth_q else None,
        "delta_s_ws_bytes": plan.ws_sq.numel() if smooth_q else None,
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel",
            "achieved": round(attn_tops, 2),
            "peak": PEAK_TOPS,
            "unit": "TOPS",
            "frac": round(attn_tops / PEAK_TOPS, 4),
            "traffic": traffic,
        },
    }
    if not full:
        keep = ("value", "ms_per_step", "ms_per_step_eager", "config", "attn_tops", "attn_ms",
                "attn_ms_median",
                "attn_tops_median", "quant_ms", "quant_share", "quant_gbs", "delta_s_ms",
                "delta_s_ws_bytes")
        res = {k: res[k] for k in keep}
        res["attn_frac_of_peak"] = round(res["attn_tops"] / PEAK_TOPS, 4)
    return res


if __name__ == "__main__":
    main()
