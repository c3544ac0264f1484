"""Benchmark of the fused MoE experts forward on one MI355X.

One step = one full experts forward (route sort, activation quantization,
gate_up grouped GEMM + SwiGLU + h quantization, down grouped GEMM + routing
weight, deterministic combine) over one batch of synthetic inputs already
resident in HBM.  The headline workload is the Mixtral-8x7B-shaped layer (4096
tokens, hidden 4096, intermediate 14336, 8 experts, top-2, FP8 e4m3 with
128x128 weight scales and dynamic 1x128 activation scales).

Prints one JSON line.  `value` is active-expert TFLOP/s (6*H*I per valid slot)
of the headline workload; `roofline` covers its dominant kernel (the gate_up
grouped GEMM) timed with HIP events on the stream it runs on, against the
roofline its arithmetic intensity binds (MFMA at the FP8 peak, or HBM);
`cpu_baseline` is the CPU oracle on a bounded sample of the same tokens.
`per_config` repeats the measurement for the other workloads (the tiny layer,
the Qwen3-MoE-shaped decode batch, the DeepSeek-V3-shaped layer and the
Mega-MoE-style FP8 x FP4 layer), each with its own roofline and oracle sample;
the decode batch is also timed cold (a 1 GiB read between forwards evicts the
256 MB last-level cache) and warm, per forward.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks (dense)
PEAK_FP8_TFLOPS = 5000.0
PEAK_MXFP4_TFLOPS = 10100.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0

METRIC = "MoE-layer active-expert TFLOP/s + tokens/s at 1 GPU; % of FP8/MXFP4 MFMA peak"

# The gate_up GEMM kernel the library launches for a workload: the register-
# streaming FP8 kernel when there are at most 12 rows per expert on average (the
# library's own rule), else the LDS-tiled FP8 kernel, or the MX kernel.
SKINNY_ROWS_PER_EXPERT = 12
_CSRC = "block_scaled_fp8_sort_amd/csrc/"
_COMMON = [_CSRC + "gemm_common.h", _CSRC + "tile_layout.h", _CSRC + "device_common.h"]
GATE_UP_KERNELS = {
    "fp8_tiled": ("gemm_fp8_b128_kernel", [_CSRC + "gemm_tiled.hip"] + _COMMON),
    "fp8_skinny": ("gemm_fp8_skinny_kernel", [_CSRC + "gemm_fp8_skinny.hip"] + _COMMON),
    "mx": ("gemm_mx_kernel", [_CSRC + "gemm_mx.hip"] + _COMMON),
    "bf16": ("gemm_bf16_tiled_kernel", [_CSRC + "gemm_tiled.hip"] + _COMMON),
}


def gate_up_kernel(wl):
    """Key into GATE_UP_KERNELS; its sources define the dominant kernel, and its
    HBM byte counters (profiles/) are reported only while they are unchanged."""
    if wl.fmt == 2:
        return "bf16"
    if wl.fmt != 0:
        return "mx"
    return "fp8_skinny" if wl.T * wl.k <= SKINNY_ROWS_PER_EXPERT * wl.E else "fp8_tiled"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first ~30 ms of GPU work after an idle spell run 12-18% slower (the
    # clock ramping up); 30 untimed forwards put the timed steps past it
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="mixtral_8x7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--per-config-cpu-seconds", type=float, default=5.0,
                    help="target CPU time of the oracle sample of each per_config workload")
    ap.add_argument("--no-per-config", action="store_true",
                    help="measure the chosen workload only (no per_config block)")
    ap.add_argument("--only", choices=["gate_up", "down"], default=None,
                    help="time one grouped GEMM alone (for counter runs); prints its own JSON line")
    ap.add_argument("--router", action="store_true",
                    help="start each step from fp32 router logits: softmax top-k + route sort + the forward "
                         "(workloads with softmax routing only)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="time a plain device-to-device copy of this many bytes (counter calibration)")
    ap.add_argument("--mfma-probe", type=int, default=0, metavar="ITERS",
                    help="measure the matrix cores' issue rate for each MFMA form the GEMMs use (register "
                         "operands, ITERS rounds of 16 MFMAs per wave) and print one JSON line")
    return ap.parse_args()


PER_CONFIG = ["tiny", "qwen3_moe_decode", "deepseek_v3", "megamoe_fp8xfp4"]
DECODE = "qwen3_moe_decode"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path has no multi-GPU mode)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_bytes:
        return copy_calibration(args, dev)
    if args.mfma_probe:
        return mfma_probe(args, dev)
    if args.only:
        import block_scaled_fp8_sort_amd as moe
        import workloads as W

        wl = W.WORKLOADS[args.workload]
        inp = W.inputs(wl, dev)
        w = moe.prepare_weights(inp["w13"], inp["s13"], inp["w2"], inp["s2"], fmt=wl.fmt)
        return only_gemm(args, wl, inp, w, dev)

    result = measure(args.workload, args, dev, args.steps, args.warmup, args.cpu_seconds, router=args.router,
                     cold=args.workload == DECODE)
    line = {
        "metric": METRIC,
        "value": result.pop("tflops"),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": result.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": result.pop("dtype"),
        "data": "synthetic",
        "config": result.pop("config"),
        "roofline": result.pop("roofline"),
    }
    if "cpu_baseline" in result:
        line["cpu_baseline"] = result.pop("cpu_baseline")
    line.update(result)  # per-forward warm / cold timings of the decode batch
    if not args.no_per_config and args.workload == "mixtral_8x7b" and not args.router:
        # the other workloads, measured the same way after the headline (outside
        # its timed region); each drops its inputs before the next is generated
        torch.cuda.empty_cache()
        per = {}
        for name in PER_CONFIG:
            r = measure(name, args, dev, max(args.steps, 10), args.warmup, args.per_config_cpu_seconds,
                        cold=name == DECODE)
            per[name] = r
            torch.cuda.empty_cache()
        line["per_config"] = per
    print(json.dumps(line), flush=True)


def _percentiles(xs):
    import numpy as np

    a = np.asarray(xs)
    return {"median_us": round(float(np.median(a)) * 1e3, 2), "p90_us": round(float(np.percentile(a, 90)) * 1e3, 2),
            "min_us": round(float(a.min()) * 1e3, 2), "iterations": int(a.size)}


def measure(name, args, dev, steps, warmup, cpu_seconds, router=False, cold=False):
    """Time the forward of one workload (steps back to back, after warmup) and
    its gate_up GEMM alone; returns the numbers of one JSON record."""
    import numpy as np
    import torch

    import block_scaled_fp8_sort_amd as moe
    import workloads as W

    wl = W.WORKLOADS[name]
    log(f"[bench] workload {wl.name}: generating inputs on the GPU")
    inp = W.inputs(wl, dev)
    w = moe.prepare_weights(inp["w13"], inp["s13"], inp["w2"], inp["s2"], fmt=wl.fmt)
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    S = T * k
    logits = None
    if router:
        if wl.routing != "uniform":
            print(f"--router needs a workload routed by a softmax over logits; {wl.name} is {wl.routing}",
                  file=sys.stderr)
            sys.exit(2)
        # the router's own routing replaces the generated one everywhere below
        logits = W.router_logits(T, E, wl.seed, device=dev)
        inp["ids"], inp["w"], _, _, _, _ = moe.route_topk(logits, k, sort=False)
        torch.cuda.synchronize()
    x, ids, wts = inp["x"], inp["ids"], inp["w"]

    ids_h = ids.cpu().numpy()
    valid = (ids_h >= 0) & (ids_h < E)
    S_v = int(valid.sum())
    touched = np.unique(ids_h[valid])
    flop_l1 = 4.0 * H * I * S_v
    flop_total = 6.0 * H * I * S_v
    if wl.fmt == W.FMT_BF16:
        w13_bytes = 2 * I * H * 2
        w2_bytes = H * I * 2
    elif wl.fmt == W.FMT_FP8_B128:
        w13_bytes = 2 * I * H + 4 * (2 * I // 128) * (H // 128)
        w2_bytes = H * I + 4 * (H // 128) * (I // 128)
    else:
        w13_bytes = 2 * I * H // 2 + 2 * I * H // 32
        w2_bytes = H * I // 2 + H * I // 32
    alg_bytes = len(touched) * (w13_bytes + w2_bytes) + 2 * T * H * 2 + T * k * 8

    ws = torch.empty(moe.forward_workspace_bytes(T, k, w), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    if logits is None:
        def step():
            moe.experts_forward(x, ids, wts, w, swiglu_limit=wl.swiglu_limit, out=out, workspace=ws)
    else:
        r_ids, r_w = torch.empty_like(ids), torch.empty_like(wts)

        def step():
            moe.experts_forward_from_logits(x, logits, k, w, swiglu_limit=wl.swiglu_limit, out=out,
                                            top_k_index=r_ids, top_k_weights=r_w, workspace=ws)

    log(f"[bench] warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {steps} steps")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    # clock stamps just outside the timed region: the mean shader clock over it
    clk0 = moe.clock_stamp(1024, dev)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    clk1 = moe.clock_stamp(1024, dev)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / steps
    fwd_sclk = _sclk_summary(moe.shader_clock_ghz(clk0, clk1))
    log(f"[bench] {ms:.3f} ms/step (wall {1e3 * t_wall / steps:.3f} ms/step)")
    extra = {}
    if cold:
        # one forward at a time, each bracketed by its own events: warm (back to
        # back) and cold (a 1 GiB read between forwards evicts the 256 MB
        # last-level cache, so weights and inputs come from HBM; a read, not a
        # fill, so that the cache holds clean lines, as after a layer that
        # streamed its own weights, and no write-back lands on the forward)
        n_it = 200
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_it)]
        for a, b in evs:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        warm = [a.elapsed_time(b) for a, b in evs]
        scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        total = torch.empty((), dtype=torch.float32, device=dev)
        for i, (a, b) in enumerate(evs):
            torch.sum(scratch, dim=0, out=total)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        cold_t = [a.elapsed_time(b) for a, b in evs]
        del scratch
        extra["warm"] = _percentiles(warm)
        extra["cold"] = dict(_percentiles(cold_t), evict_read_bytes_between=1 << 30)
        extra["cold"]["hbm_gbs_algorithmic_median"] = round(alg_bytes / (np.median(cold_t) * 1e-3) / 1e9, 1)
        extra["cold"]["hbm_frac_median"] = round(alg_bytes / (np.median(cold_t) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        log(f"[bench] per forward: warm median {np.median(warm) * 1e3:.1f} us, cold median {np.median(cold_t) * 1e3:.1f} us")
    router_us = None
    if logits is not None:
        # the router + route sort launch(es) alone, as moe_route_topk enqueues them
        rt = [torch.empty_like(ids), torch.empty_like(wts)]
        ss_b = torch.empty(S, dtype=torch.int32, device=dev)
        off_b = torch.empty(E + 1, dtype=torch.int32, device=dev)
        r_ws = torch.empty(max(1, moe.load_library().moe_route_topk_workspace(T, k, E)), dtype=torch.uint8,
                           device=dev)

        def route():
            moe.load_library().moe_route_topk(logits.data_ptr(), T, E, k, 1, rt[0].data_ptr(), rt[1].data_ptr(), E,
                                              0, ss_b.data_ptr(), off_b.data_ptr(), None, None, r_ws.data_ptr(),
                                              r_ws.numel(), stream.cuda_stream)

        for _ in range(max(3, warmup)):
            route()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(steps):
            route()
        ev1.record(stream)
        torch.cuda.synchronize()
        router_us = ev0.elapsed_time(ev1) / steps * 1e3
        log(f"[bench] router + route sort {router_us:.1f} us")

    # ---- dominant kernel: gate_up grouped GEMM with the SwiGLU + h-quant epilogue,
    # enqueued through the C ABI in the same configuration as in the forward
    ss, off, a_codes, a_scales, h_codes, h_scales, a_sorted = _gemm_inputs(wl, inp, dev)

    # zeroed tile counters, reused: each launch leaves them zero (as in the forward)
    counters = torch.zeros(moe.TILE_COUNTERS_INTS, dtype=torch.int32, device=dev)

    def l1():
        moe.grouped_gemm(w, 0, a_codes, a_scales, T, off, moe.EPI_SWIGLU_QUANT, S, a_row_index=ss, a_row_divisor=k,
                         h_codes=h_codes, h_scales=h_scales, swiglu_limit=wl.swiglu_limit, tile_counters=counters,
                         a_scales_sorted=a_sorted)

    for _ in range(max(2, warmup)):  # past the clock ramp after the host-side preparation above
        l1()
    torch.cuda.synchronize()
    clk0 = moe.clock_stamp(1024, dev)
    ev0.record(stream)
    for _ in range(steps):
        l1()
    ev1.record(stream)
    clk1 = moe.clock_stamp(1024, dev)
    torch.cuda.synchronize()
    l1_ms = ev0.elapsed_time(ev1) / steps
    l1_sclk = _sclk_summary(moe.shader_clock_ghz(clk0, clk1))
    l1_tflops = flop_l1 / (l1_ms * 1e-3) / 1e12
    act_b = 2 if wl.fmt == W.FMT_BF16 else 1  # bytes per activation / h element
    l1_bytes = int(len(touched) * w13_bytes + (T * H + S_v * I) * act_b)  # weights + A in + h out
    l1_gbs = l1_bytes / (l1_ms * 1e-3) / 1e9
    log(f"[bench] gate_up GEMM {l1_ms:.3f} ms = {l1_tflops:.1f} TFLOP/s, {l1_gbs:.0f} GB/s algorithmic")
    # e4m3 x e2m1 MFMAs issue at the FP8 rate on gfx950 (measured), so the MX
    # contraction is priced against the FP8 peak; its MXFP4 fraction is given too
    peak_flops = PEAK_BF16_TFLOPS if wl.fmt == W.FMT_BF16 else PEAK_FP8_TFLOPS
    # binding roofline from the kernel's arithmetic intensity (flop per HBM byte)
    mfma_bound = flop_l1 / l1_bytes >= peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    kname, _ = GATE_UP_KERNELS[gate_up_kernel(wl)]
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(l1_tflops, 2), "peak": peak_flops, "unit": "TFLOP/s",
                "frac": round(l1_tflops / peak_flops, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(l1_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(l1_gbs / PEAK_HBM_GBS, 4)}

    tflops = flop_total / (ms * 1e-3) / 1e12
    config = {
        "workload": wl.name, "tokens": T, "hidden": H, "intermediate": I, "experts": E, "top_k": k,
        "format": {W.FMT_FP8_B128: "fp8 e4m3, fp32 scales 1x128 act / 128x128 weight",
                   W.FMT_MX: "e4m3 act x e2m1 weight, UE8M0 per 1x32",
                   W.FMT_BF16: "bf16 act x bf16 weight, no quantization"}[wl.fmt],
        "routing": wl.routing, "skipped_slot_prob": wl.skip, "swiglu_limit": wl.swiglu_limit,
        "valid_slots": S_v, "active_tflop": round(flop_total / 1e12, 4),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "pct_fp8_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2),
        "pct_mxfp4_peak": round(100.0 * tflops / PEAK_MXFP4_TFLOPS, 2),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "hbm_gbs_algorithmic": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac_algorithmic": round(alg_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "algorithmic_bytes": int(alg_bytes),
    }
    if logits is not None:
        config["router"] = "fp32 logits N(0,1): softmax, top-k (lower id on ties), renormalised"
        config["router_sort_us"] = round(router_us, 2)
    result = {
        "ms_per_step": round(ms, 4),
        "tflops": round(tflops, 2),
        "sclk_ghz": fwd_sclk,
        "dtype": {W.FMT_FP8_B128: "fp8e4m3", W.FMT_MX: "fp8e4m3 x fp4e2m1", W.FMT_BF16: "bf16"}[wl.fmt],
        "config": config,
        "roofline": dict(roof, **{
            "traffic": traffic_record(wl),
            "kernel": f"gate_up grouped GEMM + SwiGLU + h quantization ({kname}, MOE_EPI_SWIGLU_QUANT)",
            "ms_per_launch": round(l1_ms, 4), "algorithmic_bytes_per_launch": l1_bytes,
            "algorithmic_flop_per_launch": flop_l1, "tflops": round(l1_tflops, 2), "gbs": round(l1_gbs, 1),
            "pct_fp8_peak": round(100.0 * l1_tflops / PEAK_FP8_TFLOPS, 2),
            "pct_mxfp4_peak": round(100.0 * l1_tflops / PEAK_MXFP4_TFLOPS, 2),
            # the shader clock over the timed launches (published peaks assume
            # 2.4 GHz), and the fraction of the peak scaled to that clock
            "sclk_ghz": l1_sclk,
            "frac_at_sclk": (round(roof["frac"] * 2.4 / l1_sclk["mean"], 4)
                             if roof["bound"] == "mfma" and l1_sclk["mean"] else None),
        }),
    }
    result.update(extra)
    del w, ws, out, h_codes, h_scales, a_codes
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inp, cpu_seconds)
    del inp
    return result


def _sclk_summary(per_xcd):
    """Mean, lowest and highest per-XCD shader clock (GHz) of a bracketed span."""
    v = list(per_xcd.values())
    if not v:
        return {"mean": None, "min": None, "max": None, "xcds": 0}
    return {"mean": round(sum(v) / len(v), 3), "min": round(min(v), 3), "max": round(max(v), 3), "xcds": len(v)}


def traffic_record(wl):
    """Calibrated HBM bytes per launch of the gate_up GEMM from the committed
    rocprofv3 counter summary, or None when the kernel changed since."""
    import hashlib

    key = gate_up_kernel(wl)
    path = os.path.join(ROOT, "profiles", f"gate_up_gemm_{key}_{wl.name}_hbm_bytes.md")
    srcs = GATE_UP_KERNELS[key][1]
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("traffic-record: "):
            rec = json.loads(line[len("traffic-record: "):])
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec.get("kernel_sources_sha256"):
        return None
    return rec["traffic_bytes_per_launch"]


def _gemm_inputs(wl, inp, dev):
    import torch

    import block_scaled_fp8_sort_amd as moe
    import workloads as W

    S, I, H = wl.T * wl.k, wl.I, wl.H
    ss, off, _, _ = moe.route_sort(inp["ids"], wl.E, with_slot_pos=False)
    if wl.fmt == W.FMT_BF16:  # the bf16 GEMMs read bf16 rows as they are
        return ss, off, inp["x"], None, torch.zeros((S, I), dtype=torch.bfloat16, device=dev), None, None
    a_codes, a_scales = moe.quant_act(inp["x"], wl.fmt)
    if moe.forward_sorts_scales(wl.T, wl.k, wl.fmt):
        # as the forward launches it: the scales by sorted row ([H/128][S] or
        # [H/128][S][4]), prepared here outside the timed region
        a_scales_sorted = a_scales[:, (ss.long() // wl.k)].contiguous()
    else:
        a_scales_sorted = None
    sdt = torch.float32 if wl.fmt == W.FMT_FP8_B128 else torch.uint8
    h_codes = torch.zeros((I // 128, S, 128), dtype=torch.uint8, device=dev)
    if wl.fmt == W.FMT_FP8_B128:
        h_scales = torch.ones((I // 128, S), dtype=sdt, device=dev)
    else:
        h_scales = torch.full((I // 128, S, 4), 127, dtype=sdt, device=dev)
    return ss, off, a_codes, a_scales, h_codes, h_scales, a_scales_sorted


def only_gemm(args, wl, inp, w, dev):
    """Time one grouped GEMM alone, as the forward launches it (for counter runs)."""
    import torch

    import block_scaled_fp8_sort_amd as moe

    S, I, H, k = wl.T * wl.k, wl.I, wl.H, wl.k
    ss, off, a_codes, a_scales, h_codes, h_scales, a_sorted = _gemm_inputs(wl, inp, dev)
    slot_out = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
    counters = torch.zeros(moe.TILE_COUNTERS_INTS, dtype=torch.int32, device=dev)
    if args.only == "gate_up":
        def run():
            moe.grouped_gemm(w, 0, a_codes, a_scales, wl.T, off, moe.EPI_SWIGLU_QUANT, S, a_row_index=ss,
                             a_row_divisor=k, h_codes=h_codes, h_scales=h_scales, swiglu_limit=wl.swiglu_limit,
                             tile_counters=counters, a_scales_sorted=a_sorted)
    else:
        def run():
            moe.grouped_gemm(w, 1, h_codes, h_scales, S, off, moe.EPI_WEIGHTED_SCATTER, S, slot_out=slot_out,
                             top_k_weights=inp["w"], slot_of_row=ss, tile_counters=counters)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"mode": f"only {args.only}", "workload": wl.name, "ms_per_launch": round(ms, 4)}), flush=True)


def copy_calibration(args, dev):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    import torch

    n = args.copy_bytes
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"mode": "copy", "bytes": n, "ms_per_copy": round(ms, 4),
                      "GB/s (read+write)": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def mfma_probe(args, dev):
    """The MFMA issue rate of each form the grouped GEMMs use (moe_probe_mfma_rate),
    against the published dense peak of its operand type and against that peak
    scaled to the shader clock the probe ran at (published peaks assume 2.4 GHz)."""
    import block_scaled_fp8_sort_amd as moe

    peaks = {0: PEAK_FP8_TFLOPS, 1: PEAK_FP8_TFLOPS, 2: PEAK_MXFP4_TFLOPS, 3: PEAK_BF16_TFLOPS, 4: PEAK_FP8_TFLOPS}
    peak_names = {0: "fp8", 1: "fp8 (also reported against mxfp4)", 2: "mxfp4", 3: "bf16", 4: "fp8"}
    rows = {}
    for kind in sorted(moe.PROBE_KINDS):
        tf, ghz = moe.probe_mfma_rate(kind, args.mfma_probe, dev)
        peak = peaks[kind]
        row = {"form": moe.PROBE_KINDS[kind], "tflops": round(tf, 1), "sclk_ghz": round(ghz, 3),
               "peak": peak, "peak_of": peak_names[kind], "frac_of_peak": round(tf / peak, 4),
               "frac_of_peak_at_this_clock": round(tf / (peak * ghz / 2.4), 4) if ghz > 0 else None}
        if kind == 1:
            row["frac_of_mxfp4_peak"] = round(tf / PEAK_MXFP4_TFLOPS, 4)
        rows[str(kind)] = row
        log(f"[bench] mfma probe kind {kind} ({moe.PROBE_KINDS[kind]}): {tf:.0f} TFLOP/s at {ghz:.2f} GHz")
    print(json.dumps({"mode": "mfma probe", "iters_per_wave": args.mfma_probe, "kinds": rows}), flush=True)


def cpu_baseline(wl, inp, seconds):
    """The CPU oracle, as it stands, on a seeded sample of the workload's tokens."""
    import numpy as np

    import oracle
    import workloads as W

    n = {k: W.to_numpy(v) for k, v in inp.items()}
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    # calibrate on a few tokens, then size the sample for about `seconds`
    probe = W.sample_tokens(wl.T, 2 * threads, wl.seed + 100)
    t0 = time.perf_counter()
    oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], n["ids"], n["w"],
                   swiglu_limit=wl.swiglu_limit, tokens=probe)
    dt = time.perf_counter() - t0
    per_tok = dt / probe.size
    count = int(max(threads, min(wl.T, seconds / max(per_tok, 1e-9))))
    sample = W.sample_tokens(wl.T, count, wl.seed + 200)
    t0 = time.perf_counter()
    oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], n["ids"], n["w"],
                   swiglu_limit=wl.swiglu_limit, tokens=sample)
    dt = time.perf_counter() - t0
    ids = n["ids"][sample]
    s_v = int(((ids >= 0) & (ids < wl.E)).sum())
    flop = 6.0 * wl.H * wl.I * s_v
    log(f"[bench] oracle: {sample.size} tokens in {dt:.1f} s on {threads} threads")
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{sample.size} of {wl.T} tokens (seeded), {s_v} valid slots, {dt:.1f} s",
            "tokens_per_s": round(sample.size / dt, 2), "cpu_model": _cpu_model(),
            "host_logical_cpus": os.cpu_count()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
