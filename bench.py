"""Benchmark of the MXFP8 attention-forward hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input already resident in
HBM: MXFP8-quantize Q and K (RCEIL), cast V to E4M3 (fp8 PV mode), and the fused attention
forward. The three preparation passes share one launch (prepare_qkv; --separate-prep launches
them one by one). The packed-sequence metadata is built once, before timing (the LP-FA4 README's
benchmark quantizes once and builds metadata up front; here quantization is inside the step
and is also reported on its own).

Prints ONE JSON line: value = attention FLOPs (4 * Lq * Lk * H * D summed over sequences)
per second of whole step; roofline = the attention kernel's own rate from HIP events that its
dispatch stamps at its start and end (hipExtLaunchKernel) in every --stamp-every'th step of the
timed region, against the dense FP8 matrix peak (stamping a dispatch makes the runtime do about
20 us of extra work for that step, so stamping all of them would slow the step being measured);
quantizer_gbps / cast_e4m3_gbps = the quantizer and the V cast replayed from a HIP graph of many
back-to-back launches (eager launches of these short kernels are bound by the host);
attention_pv_bf16_tflops / attention_pv_mx_tflops = back-to-back forwards with BF16 V and with V
MXFP8 along tokens, and quantizer_tokens_gbps that V quantizer, graph-replayed;
attention_bf16_fa_tflops = the BF16 FlashAttention forward (BF16 Q, K, V) on the same shapes,
back-to-back, and mxfp8_speedup_vs_bf16_fa = its time over the MXFP8 forward's back-to-back time;
cast_current_gbps = per-tensor current scaling of V (amax, then the scaled cast), graph-replayed;
prepare_qkv_gbps = the one-launch preparation (Q, K quantized and V cast), graph-replayed;
attention_bwd_tflops / _us / _pct_bf16_peak = the MXFP8 backward with MXFP8 dK/dV output,
back-to-back (2.5 x the forward's FLOPs; its matrix products run in BF16);
cpu_baseline = the float64 CPU oracle on a bounded sample of the same workload.

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
    ap.add_argument("--pv-mode", default="fp8", choices=["bf16", "fp8"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows per (sequence, head) in the oracle sample (default: all of the dense workload)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (reference dispatch "
                         "for scaling HBM byte counters)")
    ap.add_argument("--stamp-every", type=int, default=8,
                    help="the attention dispatch of every n-th timed step stamps a HIP event pair")
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
    pv_mode = args.pv_mode
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
    if per_tensor:
        qx = torch.empty((mq.total_tokens, h, 128), dtype=torch.uint8, device=dev)
        kx = torch.empty((mk.total_tokens, h, 128), dtype=torch.uint8, device=dev)
    else:
        qx = lp.Mxfp8Tensor(torch.empty((mq.total_tokens, h, 128), dtype=torch.uint8, device=dev),
                            torch.empty((mq.total_scale_rows, h, 4), dtype=torch.uint8, device=dev), mq)
        kx = lp.Mxfp8Tensor(torch.empty((mk.total_tokens, h, 128), dtype=torch.uint8, device=dev),
                            torch.empty((mk.total_scale_rows, h, 4), dtype=torch.uint8, device=dev), mk,
                            torch.empty((mk.total_scale_rows // 16, h), dtype=torch.uint8, device=dev))
    vx = torch.empty((mk.total_tokens, h, 128), dtype=torch.uint8, device=dev) if pv_mode == "fp8" else v
    plan = lp.AttnPlan(mq, mk, h, pv_mode=pv_mode, mx=not per_tensor, tile_order=order)
    out, lse = plan.out, plan.lse
    state = {"fence": torch.cuda.Event()}

    fused_prep = not per_tensor and pv_mode == "fp8" and not args.separate_prep

    def step():
        if fused_prep:  # quantize Q, K and cast V in one launch (byte-identical to the three calls)
            lp.prepare_qkv(q, k, v, mq, mk, out=(qx, kx, vx))
        else:
            if per_tensor:
                lp.cast_e4m3(q, out=qx)
                lp.cast_e4m3(k, out=kx)
            else:
                lp.quantize_mxfp8_varlen(q, mq, out=qx)
                lp.quantize_mxfp8_varlen(k, mk, out=kx)
            if pv_mode == "fp8":
                lp.cast_e4m3(v, out=vx)
        # in the timed region the kernel's own dispatch stamps a (start, stop) event pair; a plain
        # event recorded first makes the queue finish the preparation before it picks up the
        # stamped dispatch, so the start stamp is not taken while the preparation still drains
        if state.get("ev") is not None:
            state["fence"].record()
        plan(qx, kx, vx, timing=state.get("ev"))

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

    # ---- timed region: exactly K steps; every n-th attention dispatch stamps an event pair ----
    every = max(1, args.stamp_every)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range((args.steps + every - 1) // every)]
    for e0, e1 in evs:   # create the HIP events (torch creates them on first record)
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        state["ev"] = evs[i // every] if i % every == 0 else None
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    state["ev"] = None
    step_ms = start.elapsed_time(stop) / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    attn_avg_ms = float(np.mean(attn_ms))
    attn_med_ms = float(np.median(attn_ms))
    log(f"step {step_ms * 1e3:.2f} us (wall {wall / args.steps * 1e6:.2f} us), attention avg {attn_avg_ms * 1e3:.2f} us "
        f"median {attn_med_ms * 1e3:.2f} us over {len(evs)} stamped dispatches")

    # ---- attention back-to-back (the pages' protocol: quantize once, time the forward) ----
    n_b2b = args.b2b_iters or max(10, min(2000, int(0.5 / max(attn_avg_ms * 1e-3, 1e-6))))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n_b2b):
        plan(qx, kx, vx)
    b.record()
    torch.cuda.synchronize()
    b2b_ms = a.elapsed_time(b) / n_b2b

    # ---- quantizer and V cast alone: graphs of back-to-back launches, replayed ----
    quant_gbps = cast_gbps = None
    if not per_tensor:
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
            state["cast_current_gbps"] = round(v.numel() * 3 / (cur_ms * 1e-3) / 1e9, 1)
            # the one-launch preparation (Q and K quantized, V cast), graph-replayed: algorithmic
            # bytes of both quantizers plus the cast, and K's group maxima
            pms = graph_ms_per_call(torch, lambda: lp.prepare_qkv(q, k, v, mq, mk, out=(qx, kx, vx)))
            pbytes = qbytes + v.numel() * 3 + (mk.total_scale_rows // 16) * h
            state["prepare_qkv_gbps"] = round(pbytes / (pms * 1e-3) / 1e9, 1)

    # ---- pv bf16 variant of the same workload, for the record ----
    extra = {}
    if not per_tensor and pv_mode == "fp8":
        plan_bf16 = lp.AttnPlan(mq, mk, h, pv_mode="bf16", tile_order=order, out=out, lse=lse)
        a.record()
        for _ in range(n_b2b):
            plan_bf16(qx, kx, v)
        b.record()
        torch.cuda.synchronize()
        bf_ms = a.elapsed_time(b) / n_b2b
        extra["attention_pv_bf16_tflops"] = round(flops / (bf_ms * 1e-3) / 1e12, 2)
        # MX-scaled V (V MXFP8 along tokens, one scale per 32 tokens per column), and its quantizer
        vt = lp.quantize_mxfp8_varlen_tokens(v, mk)
        plan_mx = lp.AttnPlan(mq, mk, h, pv_mode="mx", tile_order=order, out=out, lse=lse)
        a.record()
        for _ in range(n_b2b):
            plan_mx(qx, kx, vt)
        b.record()
        torch.cuda.synchronize()
        mx_ms = a.elapsed_time(b) / n_b2b
        extra["attention_pv_mx_tflops"] = round(flops / (mx_ms * 1e-3) / 1e12, 2)
        tms = graph_ms_per_call(torch, lambda: lp.quantize_mxfp8_varlen_tokens(v, mk, out=vt))
        tbytes = v.numel() * 2 + v.numel() + (mk.total_scale_rows // 32) * h * 128
        extra["quantizer_tokens_gbps"] = round(tbytes / (tms * 1e-3) / 1e9, 1)
        # the BF16 FlashAttention forward on the same shapes (BF16 Q, K, V): the baseline that the
        # MXFP8 forward's speedup is taken against (both back-to-back, inputs resident)
        plan_b = lp.AttnPlan(mq, mk, h, pv_mode="bf16", mx=False, qk_bf16=True, tile_order=order, out=out, lse=lse)
        a.record()
        for _ in range(n_b2b):
            plan_b(q, k, v)
        b.record()
        torch.cuda.synchronize()
        bfa_ms = a.elapsed_time(b) / n_b2b
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
        bplan()
        torch.cuda.synchronize()
        n_bwd = max(10, n_b2b // 4)
        a.record()
        for _ in range(n_bwd):
            bplan()
        b.record()
        torch.cuda.synchronize()
        bwd_ms = a.elapsed_time(b) / n_bwd
        extra["attention_bwd_us"] = round(bwd_ms * 1e3, 2)
        extra["attention_bwd_tflops"] = round(2.5 * flops / (bwd_ms * 1e-3) / 1e12, 2)
        extra["attention_bwd_pct_bf16_peak"] = round(100 * 2.5 * flops / (bwd_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2)

    achieved = flops / (attn_avg_ms * 1e-3) / 1e12
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
                   "seq_lens_q": list(wl.lengths_q)[:16], "seq_lens_k": list(wl.lengths_k)[:16],
                   "heads": wl.num_heads, "head_dim": 128, "seed": args.seed,
                   "step": ("quantize Q,K + cast V (one launch) + attention forward" if fused_prep else
                            "quantize Q,K + cast V + attention forward") if not per_tensor
                   else "cast Q,K,V + attention forward"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "attention_kernel_tflops_b2b": round(flops / (b2b_ms * 1e-3) / 1e12, 2),
        "attention_kernel_us_avg": round(attn_avg_ms * 1e3, 3),
        "attention_kernel_us_median": round(attn_med_ms * 1e3, 3),
        "quantizer_gbps": None if quant_gbps is None else round(quant_gbps, 1),
        "cast_e4m3_gbps": None if cast_gbps is None else round(cast_gbps, 1),
        "pct_fp8_peak": round(100 * achieved / FP8_PEAK_TFLOPS, 2),
    }
    for key in ("cast_current_gbps", "prepare_qkv_gbps"):
        if key in state:
            extra[key] = state[key]
    line.update(extra)
    print(json.dumps(line), flush=True)


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
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "precision_attention_mxfp8_amd", "csrc", "attn_fwd.hip")
    h.update(open(src, "rb").read())
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
