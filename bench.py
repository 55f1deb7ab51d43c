"""Benchmark of the MXFP8 attention-forward hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input already resident in
HBM: MXFP8-quantize Q and K (RCEIL), cast V to E4M3 (fp8 PV mode), and the fused attention
forward. The three preparation passes share one launch (prepare_qkv; --separate-prep launches
them one by one). The per-tensor workload casts Q, K (with K's group maxima, the precision
guard's bound on |k|) and V instead. With BF16 V (--pv-mode bf16) the K quantizer also writes K's
quantized values as BF16 (2 B per element more), which the attention's tiles that fail the
precision guard load instead of converting K themselves (--no-k-deq: without). The packed-sequence
metadata is built once, before timing.

Prints ONE JSON line:
* value = attention FLOPs (4 * Lq * Lk * H * D summed over sequences) per second of whole step,
  over exactly --steps steps after --warmup untimed ones (nothing is stamped inside them);
* roofline = the attention kernel's own rate: its FLOPs over its average launch duration, the
  mean per-launch time of the protocol pass below (HIP events on the launching stream around
  batches of back-to-back forwards), against the dense FP8 matrix peak (published, and measured:
  measured_peaks); beside it, a labelled pass after the timed steps in which every attention
  dispatch stamps a HIP event pair at its start and end (hipExtLaunchKernel, --stamped samples);
* protocol = the LP-FA4 README's benchmark protocol ("Benchmark reproduction"): operands quantized
  once, the forward alone back to back, 1 s of warmup, then a 5 s window of event-timed batches
  (each >= 1 ms); raw per-launch samples, the padded scale offsets, the workload and the
  environment go into the line;
* quantizer_gbps / cast_e4m3_gbps / prepare_qkv_gbps / cast_current_gbps = the preparation
  kernels replayed from a HIP graph of many back-to-back launches (eager launches of these short
  kernels are bound by the host); attention_pv_bf16_tflops / attention_pv_mx_tflops = the forward
  with BF16 V and with V MXFP8 along tokens; attention_bf16_fa_tflops = the BF16 FlashAttention
  forward on the same shapes, and mxfp8_speedup_vs_bf16_fa; attention_bwd_* = the MXFP8 backward
  with MXFP8 dK/dV (2.5 x the forward's FLOPs, BF16 matrix products);
* measured_peaks = FP8 and BF16 matrix-instruction loops and an HBM copy on this GPU (libpeak.so);
* cpu_baseline = the float64 CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense] [--pv-mode fp8]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 matrix peak (AMD spec, no sparsity)
BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBPS = 8000.0

# The PV mode each workload is specified with (the dense shape is run in both; fp8 is its headline)
DEFAULT_PV_MODE = {"tiny": "bf16", "dense": "fp8", "varlen": "bf16", "pertensor": "fp8", "cross": "fp8", "batch8": "fp8"}

WORKLOAD_TEXT = {
    "tiny": "tiny: 1 sequence x 256 tokens, 2 heads, head_dim 128, noncausal MHA",
    "dense": "dense: 1 sequence x 2048 tokens, 16 heads, head_dim 128, noncausal MHA",
    "varlen": "varlen: 8 sequences, lengths uniform in [128, 4096] (seed 0), 16 heads, head_dim 128, 0.1% x20 outliers",
    "pertensor": "pertensor: 2 x 16384 tokens, 24 heads, head_dim 128, per-tensor FP8 e4m3 (no descale)",
    "cross": "cross: queries 4096 tokens, keys/values 32768 tokens, 16 heads, head_dim 128, keys N(0, 0.25)",
    "batch8": "batch8: 8 sequences x 2048 tokens, 16 heads, head_dim 128, noncausal MHA (the README's bundled shape)",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="dense", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--pv-mode", default=None, choices=["bf16", "fp8"],
                    help="P V mode (default: the workload's own: bf16 for tiny and varlen, fp8 otherwise)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows per (sequence, head) in the oracle sample (default: all of the dense workload)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (reference dispatch "
                         "for scaling HBM byte counters)")
    ap.add_argument("--stamped", type=int, default=64,
                    help="steps of the labelled pass after the timed ones whose attention dispatch stamps an event pair")
    ap.add_argument("--protocol-warmup-s", type=float, default=1.0,
                    help="warmup of the README protocol pass (seconds of back-to-back forwards)")
    ap.add_argument("--protocol-window-s", type=float, default=5.0,
                    help="measurement window of the README protocol pass (seconds)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other PV modes, the BF16 forward, the backward and the peak loops")
    ap.add_argument("--no-k-deq", action="store_true",
                    help="bf16 PV: quantize K without its BF16 values (guard-failing tiles then convert K themselves)")
    ap.add_argument("--separate-prep", action="store_true",
                    help="launch the Q, K quantizers and the V cast separately instead of as one kernel")
    ap.add_argument("--b2b-iters", type=int, default=0,
                    help="launches in the back-to-back and quantizer-only loops (0: about half a second)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "attn_traffic.json"),
                    help="measured HBM bytes per attention launch (from rocprofv3 counters), if present")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import precision_attention_mxfp8_amd as lp
    from synth import make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = lp.load_library()   # fails loudly if the HIP library is missing

    wl = make_workload(args.workload, seed=args.seed)
    pv_mode = args.pv_mode or DEFAULT_PV_MODE[args.workload]
    mq = lp.VarlenMeta.from_lengths(wl.lengths_q, dev)
    mk = lp.VarlenMeta.from_lengths(wl.lengths_k, dev)
    up = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = up(wl.q_bits), up(wl.k_bits), up(wl.v_bits)
    flops = wl.flops()
    per_tensor = args.workload == "pertensor"
    if per_tensor:
        pv_mode = "fp8"
    order = lp.longest_first_tile_order(mq, mk, wl.num_heads) if args.workload == "varlen" else None

    # every output (quantized operands, O, LSE) is allocated once; each step writes into it
    h = wl.num_heads
    kgm = None
    kdeq = None
    if per_tensor:
        qx = torch.empty((mq.total_tokens, h, 128), dtype=torch.uint8, device=dev)
        kx = torch.empty((mk.total_tokens, h, 128), dtype=torch.uint8, device=dev)
        kgm = torch.empty(lp.e4m3_group_max_shape(mk.total_tokens, h), dtype=torch.uint8, device=dev)
    else:
        qx = lp.Mxfp8Tensor(torch.empty((mq.total_tokens, h, 128), dtype=torch.uint8, device=dev),
                            torch.empty((mq.total_scale_rows, h, 4), dtype=torch.uint8, device=dev), mq)
        # with BF16 V the K quantizer also writes K's quantized values as BF16, which the kernel's
        # guard-failing tiles load instead of converting every K block themselves
        kdeq = (torch.empty((mk.total_tokens, h, 128), dtype=torch.bfloat16, device=dev)
                if pv_mode == "bf16" and not args.no_k_deq else None)
        kx = lp.Mxfp8Tensor(torch.empty((mk.total_tokens, h, 128), dtype=torch.uint8, device=dev),
                            torch.empty((mk.total_scale_rows, h, 4), dtype=torch.uint8, device=dev), mk,
                            torch.empty((mk.total_scale_rows // 16, h), dtype=torch.uint8, device=dev), kdeq)
    vx = torch.empty((mk.total_tokens, h, 128), dtype=torch.uint8, device=dev) if pv_mode == "fp8" else v
    plan = lp.AttnPlan(mq, mk, h, pv_mode=pv_mode, mx=not per_tensor, tile_order=order)
    out, lse = plan.out, plan.lse
    state = {"fence": torch.cuda.Event(), "ev": None}

    fused_prep = not per_tensor and pv_mode == "fp8" and not args.separate_prep

    def attend(timing=None):
        plan(qx, kx, vx, timing=timing, k_group_max=kgm)

    def step():
        if fused_prep:  # quantize Q, K and cast V in one launch (byte-identical to the three calls)
            lp.prepare_qkv(q, k, v, mq, mk, out=(qx, kx, vx))
        else:
            if per_tensor:
                lp.cast_e4m3(q, out=qx)
                lp.cast_e4m3(k, out=kx, group_max_out=kgm)
            else:
                lp.quantize_mxfp8_varlen(q, mq, out=qx)
                lp.quantize_mxfp8_varlen(k, mk, out=kx)
            if pv_mode == "fp8":
                lp.cast_e4m3(v, out=vx)
        # in the stamped pass the kernel's own dispatch stamps a (start, stop) event pair; a plain
        # event recorded first makes the queue finish the preparation before it picks up the
        # stamped dispatch, so the start stamp is not taken while the preparation still drains
        if state["ev"] is not None:
            state["fence"].record()
        attend(state["ev"])

    log(f"workload {args.workload} pv_mode {pv_mode}: {flops / 1e9:.2f} GFLOP per forward")
    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb * (1 << 20)
        src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)   # one elementwise dispatch: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        log(f"copy calibration: one neg dispatch reads {n} bytes and writes {n} bytes")
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, nothing stamped ----
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = start.elapsed_time(stop) / args.steps

    # ---- labelled stamped pass: every attention dispatch stamps its own start and end ----
    n_st = max(1, args.stamped)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_st)]
    for e0, e1 in evs:   # create the HIP events (torch creates them on first record)
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    for i in range(n_st):
        state["ev"] = evs[i]
        step()
    state["ev"] = None
    torch.cuda.synchronize()
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    attn_avg_ms = float(np.mean(attn_ms))
    attn_med_ms = float(np.median(attn_ms))
    log(f"step {step_ms * 1e3:.2f} us (wall {wall / args.steps * 1e6:.2f} us); stamped pass: attention avg "
        f"{attn_avg_ms * 1e3:.2f} us median {attn_med_ms * 1e3:.2f} us over {n_st} dispatches")

    # ---- the README's protocol: quantize once, forward back to back, 1 s warmup, 5 s window ----
    proto = protocol_pass(torch, attend, args.protocol_warmup_s, args.protocol_window_s)
    b2b_ms = proto["median_us"] * 1e-3
    log(f"protocol: {len(proto['samples_us'])} batches of {proto['batch']} forwards, median {proto['median_us']:.2f} us")

    # ---- quantizer and V cast alone: graphs of back-to-back launches, replayed ----
    extra = {}
    quant_gbps = cast_gbps = None
    if per_tensor:
        cms = graph_ms_per_call(torch, lambda: lp.cast_e4m3(k, out=kx, group_max_out=kgm))
        cast_gbps = k.numel() * 3 / (cms * 1e-3) / 1e9
    else:
        qbytes = sum(t.numel() * 2 + t.numel() + m.total_scale_rows * wl.num_heads * 4
                     for t, m in ((q, mq), (k, mk)))
        qms = graph_ms_per_call(torch, lambda: (lp.quantize_mxfp8_varlen(q, mq, out=qx),
                                                lp.quantize_mxfp8_varlen(k, mk, out=kx)))
        quant_gbps = qbytes / (qms * 1e-3) / 1e9
        if pv_mode == "fp8":
            cms = graph_ms_per_call(torch, lambda: lp.cast_e4m3(v, out=vx))
            cast_gbps = v.numel() * 3 / (cms * 1e-3) / 1e9
            # per-tensor current scaling of the same V (amax pass, then the scaled cast): the
            # algorithmic bytes are those of one cast (3 B per element); the amax pass reads V again
            cur_ms = graph_ms_per_call(torch, lambda: lp.cast_e4m3_current(v, out=vx))
            extra["cast_current_gbps"] = round(v.numel() * 3 / (cur_ms * 1e-3) / 1e9, 1)
            # the one-launch preparation (Q and K quantized, V cast), graph-replayed: algorithmic
            # bytes of both quantizers plus the cast, and K's group maxima
            pms = graph_ms_per_call(torch, lambda: lp.prepare_qkv(q, k, v, mq, mk, out=(qx, kx, vx)))
            pbytes = qbytes + v.numel() * 3 + (mk.total_scale_rows // 16) * h
            extra["prepare_qkv_gbps"] = round(pbytes / (pms * 1e-3) / 1e9, 1)

    n_b2b = args.b2b_iters or max(10, min(2000, int(0.5 / max(b2b_ms * 1e-3, 1e-6))))
    if not per_tensor and pv_mode == "fp8" and not args.no_extras:
        extra.update(other_modes(torch, lp, wl, q, k, v, qx, kx, mq, mk, order, out, lse, n_b2b, b2b_ms, flops, up))
    elif not per_tensor and not args.no_extras:
        # bf16 PV: the BF16 FlashAttention forward on the same data, back to back (its ceiling)
        plan_b = lp.AttnPlan(mq, mk, h, pv_mode="bf16", mx=False, qk_bf16=True, tile_order=order)
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        plan_b(q, k, v)
        a_ev.record()
        for _ in range(n_b2b):
            plan_b(q, k, v)
        b_ev.record()
        torch.cuda.synchronize()
        bfa_ms = a_ev.elapsed_time(b_ev) / n_b2b
        extra["attention_bf16_fa_tflops"] = round(flops / (bfa_ms * 1e-3) / 1e12, 2)
        extra["mxfp8_speedup_vs_bf16_fa"] = round(bfa_ms / b2b_ms, 3)

    peaks = None if args.no_extras else measured_peaks(torch, dev)

    # the kernel's average launch duration: the README protocol's event-timed batches of
    # back-to-back forwards on the launching stream (thousands of launches in the 5 s window), the
    # same launches that dominate a kernel trace of this command; the stamped pass, whose fence
    # before each dispatch adds the queue's start-up to every sample, is reported beside it
    proto_mean_us = float(np.mean(proto["samples_us"]))
    achieved = flops / (proto_mean_us * 1e-6) / 1e12
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            key = f"{args.workload}/{pv_mode}"
            if key in tj and tj[key].get("kernel_source_hash") == kernel_source_hash():
                traffic = tj[key]["bytes_per_launch"]
        except Exception as e:  # pragma: no cover
            log(f"traffic file unreadable: {e}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, pv_mode, args.cpu_rows, per_tensor)

    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel_us_avg": round(proto_mean_us, 3), "kernel_us_median": round(proto["median_us"], 3),
                "samples": len(proto["samples_us"]) * proto["batch"],
                "source": "README protocol: mean per-launch time of event-timed batches of back-to-back forwards",
                "stamped_us_avg": round(attn_avg_ms * 1e3, 3), "stamped_us_median": round(attn_med_ms * 1e3, 3),
                "stamped_samples": n_st}
    if peaks is not None:
        roofline["peak_measured"] = peaks["fp8_tflops"]
        roofline["frac_of_measured"] = round(achieved / peaks["fp8_tflops"], 4)
    line = {
        "metric": "MXFP8 attention fwd TFLOP/s (1 GPU) + % of FP8 MFMA peak; quantizer GB/s",
        "value": round(flops / (step_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3" if pv_mode == "fp8" else "fp8e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "pv_mode": pv_mode,
                   "scaling_mode": "rceil" if not per_tensor else "per-tensor",
                   "seq_lens_q": list(wl.lengths_q), "seq_lens_k": list(wl.lengths_k),
                   "cu_scale_q": list(mq.cu_scale_host) if not per_tensor else None,
                   "cu_scale_k": list(mk.cu_scale_host) if not per_tensor else None,
                   "heads": wl.num_heads, "head_dim": 128, "seed": args.seed,
                   "step": ("quantize Q,K + cast V (one launch) + attention forward" if fused_prep else
                            "quantize Q,K + cast V + attention forward" if pv_mode == "fp8" else
                            "quantize Q, K (with K's BF16 values) + attention forward" if kdeq is not None else
                            "quantize Q, K + attention forward") if not per_tensor
                   else "cast Q, K (with group maxima), V + attention forward"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "protocol": proto,
        "attention_kernel_tflops_b2b": round(flops / (b2b_ms * 1e-3) / 1e12, 2),
        "attention_kernel_us_avg": round(proto_mean_us, 3),
        "attention_kernel_us_median": round(proto["median_us"], 3),
        "attention_stamped_us_avg": round(attn_avg_ms * 1e3, 3),
        "attention_stamped_us_median": round(attn_med_ms * 1e3, 3),
        "quantizer_gbps": None if quant_gbps is None else round(quant_gbps, 1),
        "cast_e4m3_gbps": None if cast_gbps is None else round(cast_gbps, 1),
        "pct_fp8_peak": round(100 * achieved / FP8_PEAK_TFLOPS, 2),
        "measured_peaks": peaks,
        "env": environment(torch),
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


def protocol_pass(torch, attend, warmup_s, window_s, min_batch_ms=1.0):
    """The LP-FA4 README's benchmark protocol on already quantized operands: back-to-back forwards for
    warmup_s seconds, then event-timed batches (each at least min_batch_ms long) until window_s
    seconds have passed. Returns the raw per-launch samples (microseconds, one per batch)."""
    t_end = time.perf_counter() + warmup_s
    n = 0
    while time.perf_counter() < t_end or n < 3:
        attend()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(4):
        attend()
    b.record()
    torch.cuda.synchronize()
    est_ms = max(a.elapsed_time(b) / 4, 1e-4)
    batch = max(1, int(math.ceil(min_batch_ms / est_ms)))
    samples = []
    t_end = time.perf_counter() + window_s
    while time.perf_counter() < t_end or len(samples) < 3:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(batch):
            attend()
        b.record()
        b.synchronize()
        samples.append(round(a.elapsed_time(b) / batch * 1e3, 3))
    return {"warmup_s": warmup_s, "window_s": window_s, "batch": batch, "samples_us": samples,
            "median_us": float(np.median(samples)), "source": "LP-FA4 README, Benchmark reproduction"}


def other_modes(torch, lp, wl, q, k, v, qx, kx, mq, mk, order, out, lse, n_b2b, b2b_ms, flops, up):
    """The same workload's other forward variants and the backward, back to back."""
    h = wl.num_heads
    extra = {}
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def b2b(fn, n):
        fn()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    plan_bf16 = lp.AttnPlan(mq, mk, h, pv_mode="bf16", tile_order=order, out=out, lse=lse)
    bf_ms = b2b(lambda: plan_bf16(qx, kx, v), n_b2b)
    extra["attention_pv_bf16_tflops"] = round(flops / (bf_ms * 1e-3) / 1e12, 2)
    # MX-scaled V (V MXFP8 along tokens, one scale per 32 tokens per column), and its quantizer
    vt = lp.quantize_mxfp8_varlen_tokens(v, mk)
    plan_mx = lp.AttnPlan(mq, mk, h, pv_mode="mx", tile_order=order, out=out, lse=lse)
    mx_ms = b2b(lambda: plan_mx(qx, kx, vt), n_b2b)
    extra["attention_pv_mx_tflops"] = round(flops / (mx_ms * 1e-3) / 1e12, 2)
    tms = graph_ms_per_call(torch, lambda: lp.quantize_mxfp8_varlen_tokens(v, mk, out=vt))
    tbytes = v.numel() * 2 + v.numel() + (mk.total_scale_rows // 32) * h * 128
    extra["quantizer_tokens_gbps"] = round(tbytes / (tms * 1e-3) / 1e9, 1)
    # the BF16 FlashAttention forward on the same shapes (BF16 Q, K, V): the baseline that the
    # MXFP8 forward's speedup is taken against (both back-to-back, inputs resident)
    plan_b = lp.AttnPlan(mq, mk, h, pv_mode="bf16", mx=False, qk_bf16=True, tile_order=order, out=out, lse=lse)
    bfa_ms = b2b(lambda: plan_b(q, k, v), n_b2b)
    extra["attention_bf16_fa_tflops"] = round(flops / (bfa_ms * 1e-3) / 1e12, 2)
    extra["attention_bf16_fa_pct_bf16_peak"] = round(100 * flops / (bfa_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2)
    extra["mxfp8_speedup_vs_bf16_fa"] = round(bfa_ms / b2b_ms, 3)
    # the MXFP8 backward with fused MXFP8 dK/dV output (the README times the backward on that
    # path): D, dK/dV and dQ kernels back-to-back, on the MX-V forward's own output and LSE;
    # FLOPs = 2.5 x the forward's (five matrix products of the forward's size each)
    from synth import make_output_grad
    qt_b = lp.quantize_mxfp8_varlen_tokens(q, mq)
    kt_b = lp.quantize_mxfp8_varlen_tokens(k, mk)
    vd_b = lp.quantize_mxfp8_varlen(v, mk)
    plan_mx(qx, kx, vt)
    dout = up(make_output_grad(mq.total_tokens, h, seed=1))
    bplan = lp.BwdPlan(qx, kx, vd_b, qt_b, kt_b, out, dout, lse, output_mxfp8_dkv=True)
    bwd_ms = b2b(bplan, max(10, n_b2b // 4))
    extra["attention_bwd_us"] = round(bwd_ms * 1e3, 2)
    extra["attention_bwd_tflops"] = round(2.5 * flops / (bwd_ms * 1e-3) / 1e12, 2)
    extra["attention_bwd_pct_bf16_peak"] = round(100 * 2.5 * flops / (bwd_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2)
    return extra


def measured_peaks(torch, dev):
    """Ceilings measured on this GPU: FP8 and BF16 matrix-instruction loops (two waves per SIMD, eight
    independent accumulators each) and an HBM copy of 2 GiB (read + write)."""
    import ctypes
    path = os.path.join(ROOT, "precision_attention_mxfp8_amd", "libpeak.so")
    if not os.path.exists(path):
        log("libpeak.so missing: no measured peaks")
        return None
    lib = ctypes.CDLL(path)
    for fn in (lib.peak_mfma_fp8, lib.peak_mfma_bf16):
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.peak_copy.restype = ctypes.c_int
    stream = torch.cuda.current_stream().cuda_stream
    wps = 2
    out = torch.empty((256 * wps * 4,), dtype=torch.float32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn, flop in (("fp8_tflops", lib.peak_mfma_fp8, 65536), ("bf16_tflops", lib.peak_mfma_bf16, 16384)):
        iters = 2000
        assert fn(wps, iters, out.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        a.record()
        assert fn(wps, iters, out.data_ptr(), stream) == 0
        b.record()
        torch.cuda.synchronize()
        total = 256 * wps * 4 * iters * 8 * flop
        res[name] = round(total / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    assert lib.peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream) == 0
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        assert lib.peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream) == 0
    b.record()
    torch.cuda.synchronize()
    res["hbm_copy_gbps"] = round(5 * 2 * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del src, dst
    res["published"] = {"fp8_tflops": FP8_PEAK_TFLOPS, "bf16_tflops": BF16_PEAK_TFLOPS, "hbm_gbps": HBM_PEAK_GBPS}
    return res


def environment(torch):
    """Device, software versions and host cores of this run."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    for f in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(f):
            rocm = open(f).read().strip()
            break
    return {"device": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "memory_gib": round(props.total_memory / 2 ** 30, 1),
            "rocm": rocm, "torch": torch.__version__, "hip": torch.version.hip,
            "host_cores": len(os.sched_getaffinity(0)), "python": sys.version.split()[0]}


def graph_ms_per_call(torch, call, per_graph=25, replays=20):
    """Milliseconds per `call` when `per_graph` calls captured in one HIP graph are replayed
    `replays` times back to back (the calls record no memset and allocate nothing)."""
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(per_graph):
            call()
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (replays * per_graph)


def kernel_source_hash() -> str:
    """sha256[:16] over the attention kernel's source and the headers it is compiled with."""
    import hashlib
    h = hashlib.sha256()
    for name in ("attn_fwd.hip", "device_common.h", "kernels.h"):
        h.update(open(os.path.join(ROOT, "precision_attention_mxfp8_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(wl, pv_mode, rows_per_head, per_tensor):
    """The float64 oracle on a bounded sample: quantize Q and K in full, then attention for
    `rows_per_head` evenly spaced query rows of each sequence and head against all keys."""
    import oracle
    from synth import bf16_bits_to_f32
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    xq = bf16_bits_to_f32(wl.q_bits).astype(np.float64)
    xk = bf16_bits_to_f32(wl.k_bits).astype(np.float64)
    xv = bf16_bits_to_f32(wl.v_bits).astype(np.float64)
    if per_tensor:
        qh, kh = oracle.e4m3_decode(oracle.e4m3_encode(xq)), oracle.e4m3_decode(oracle.e4m3_encode(xk))
    else:
        pq, sq, cq = oracle.mx_quantize_varlen(xq, wl.cu_q)
        pk, sk, ck = oracle.mx_quantize_varlen(xk, wl.cu_k)
        qh = oracle.mx_dequantize_varlen(pq, sq, wl.cu_q, cq)
        kh = oracle.mx_dequantize_varlen(pk, sk, wl.cu_k, ck)
    vp = oracle.e4m3_decode(oracle.e4m3_cast(xv)) if pv_mode == "fp8" else xv
    rows = {r: np.linspace(0, lq - 1, min(rows_per_head, lq)).astype(np.int64)
            for r, lq in enumerate(wl.lengths_q) if lq > 0}
    oracle.attention_varlen(qh, kh, vp, wl.cu_q, wl.cu_k, pv_mode=pv_mode, rows=rows)
    dt = time.perf_counter() - t0
    sample_flops = sum(4 * len(rows[r]) * wl.lengths_k[r] * wl.num_heads * 128 for r in rows)
    return {"value": round(sample_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(min(threads, cores)),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle: full MXFP8 quantize of Q and K, then attention for "
                      f"{sum(len(v) for v in rows.values())} query rows of every head against all keys ({sample_flops / 1e9:.2f} GFLOP); "
                      f"{dt:.1f} s wall; host affinity {cores} cores"}


if __name__ == "__main__":
    main()
