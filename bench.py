#!/usr/bin/env python3
"""Benchmark of the GPTQ layer quantizer on one MI355X.

One step = the whole hot path on one Llama-shaped layer with synthetic,
seeded inputs already resident in HBM: H.zero_(), H += 2 X^T X over all
calibration tokens (gptq_hessian_accumulate), then gptq_quantize_layer
(damping, activation order, blocked Cholesky + inverse, the in-block
quantize-and-compensate loop, the lazy trailing updates, bit packing).

Metric: layer-quantize throughput in TFLOP/s of algorithmic work
(F_H + F_upd) / t_step with F_H = n d_in (d_in + 1) (symmetric half of the
Hessian) and F_upd = d_out d_in (d_in - 1) (all compensation FMAs x 2);
ms_per_step is the layer time.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload q_proj]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0
STAGE_HESSIAN_PRODUCT = 0      # gptq_profile stage index of the Hessian product kernel
COUNTERS = os.path.join(ROOT, "profiles", "hessian_product_q_proj_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_flops(wl):
    f_h = wl.n * wl.d_in * (wl.d_in + 1)
    f_upd = wl.d_out * wl.d_in * (wl.d_in - 1)
    return f_h, f_upd


def describe(wl):
    return (f"{wl.name} {wl.d_out}x{wl.d_in} {wl.dtype}, n={wl.n} tokens, {wl.bits}-bit, group {wl.group_size}, "
            f"block {wl.block_size}, act_order {'on' if wl.act_order else 'off'}")


def kernel_source_hash():
    """sha256 of the Hessian kernels' source: hessian.hip and the part of
    common.h they use (the shared types and the Hessian declarations, up to
    the next section)."""
    csrc = os.path.join(ROOT, "post_weight_quantization_04_amd", "csrc")
    common = open(os.path.join(csrc, "common.h"), "rb").read()
    cut = common.find(b"// Preparation (prep.hip)")
    h = hashlib.sha256()
    h.update(open(os.path.join(csrc, "hessian.hip"), "rb").read())
    h.update(common[:cut] if cut >= 0 else common)
    return h.hexdigest()


def measured_traffic(wl):
    """Bytes per launch the Hessian product kernel moves beyond L2, from
    committed rocprofv3 counter runs on this workload, or None when absent,
    taken on another workload or on other kernel source."""
    try:
        c = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != kernel_source_hash() or not c.get("workload", "").startswith(wl.name + " "):
        return None
    return c.get("hbm_bytes_per_launch")


def batch_ends(wl):
    """Column where each batch of blocks ends (a far update follows every one
    but the last): batches of eight blocks up to 128 columns wide, of 1024
    columns for wider ones, cut after a block that ends a group wider than a
    block; blocks wider than 256 columns run as the widest width <= 256 that
    keeps every group start on a block start."""
    d, B = wl.d_in, min(wl.block_size, wl.d_in)
    g = wl.d_in if (wl.group_size == -1 or wl.group_size >= d) else wl.group_size
    if B > 256:
        B = 256 if g >= d else ((256 // g) * g if g <= 256 else next(c for c in range(256, 0, -16) if g % c == 0))
    far = 8 if B <= 128 else max(1, 1024 // B)
    ends, e = [], 0
    while e < d:
        nblk = 0
        while nblk < far and e < d:
            e = min(e + B, d)
            nblk += 1
            if g > B and e % g == 0:
                break
        ends.append(e)
    return B, ends


def layer_roofline(wl, stages, ms_layer):
    """Every stage at its own roofline (max of flops at the MFMA peak of its
    type and bytes at HBM bandwidth), summed, against the measured layer."""
    d, do, n = wl.d_in, wl.d_out, wl.n
    xb = 2 if wl.dtype == "bf16" else 4
    f_h, f_upd = workload_flops(wl)
    groups = -(-d // (d if (wl.group_size == -1 or wl.group_size >= d) else wl.group_size))
    words = -(-wl.bits * d // 32)
    peak_h = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    _, ends = batch_ends(wl)
    starts = [0] + ends[:-1]
    f_far = sum(2 * do * (e - p) * (d - e) for p, e in zip(starts, ends) if e < d)
    work = {   # stage: (flops, flop peak TFLOP/s, bytes)
        "hessian": (f_h, peak_h, xb * n * d + 8 * d * d),
        "prep": (0, PEAK_FP32_TFLOPS, 8 * d * d + (xb + 4) * do * d),
        "factor": (2 * d ** 3 / 3, PEAK_FP32_TFLOPS, 8 * d * d),
        "update": (f_upd, PEAK_FP32_TFLOPS, 9 * do * d),
        "pack": (0, PEAK_FP32_TFLOPS, do * d + 4 * words * do + 8 * groups * do),
    }
    at_peak = {k: max(f / (p * 1e12), b / (PEAK_HBM_GBS * 1e9)) * 1e3 for k, (f, p, b) in work.items()}
    ms = lambda k: stages.get(k, {}).get("ms_per_step", 0.0)
    t_upd = ms("quant_block") + ms("trail_update")
    rates = {
        "hessian_product_tflops": f_h / (ms("hessian_product") * 1e9) if ms("hessian_product") else None,
        "factor_tflops": (2 * d ** 3 / 3) / (ms("factor") * 1e9) if ms("factor") else None,
        "update_tflops": f_upd / (t_upd * 1e9) if t_upd else None,
        "trail_update_tflops": f_far / (ms("trail_update") * 1e9) if ms("trail_update") else None,
        "quant_block_gbs": 9 * do * d / (ms("quant_block") * 1e6) if ms("quant_block") else None,
        "pack_gbs": (do * d + 4 * words * do) / (ms("pack") * 1e6) if ms("pack") else None,
    }
    total = sum(at_peak.values())
    return {"sum_at_peak_ms": total, "t_layer_ms": ms_layer, "frac": total / ms_layer,
            "at_peak_ms": at_peak, "trailing_flops": f_far, "stage_rates": rates}


def gemv_bench(P, torch, wl, q, Xd, calls=200):
    """The product with the packed layer just quantized (gptq_dequant_matmul),
    m = 1 and m = 8 activation rows taken from the calibration set.  The
    packed weights, scales and zero points are cycled through enough copies
    (> 256 MB) that the memory-side cache cannot hold them, so every call
    reads them from HBM; bytes per call = packed words + scales + zero points
    + activations + outputs."""
    nbytes_w = q.qpacked.numel() * 4 + (q.scales.numel() + q.zeros.numel()) * 4
    ncopy = max(2, -(-320 * 2 ** 20 // nbytes_w))
    copies = [P.QuantizedLayer(q.qpacked.clone(), q.scales.clone(), q.zeros.clone(), q.perm, q.bits, q.group_size,
                               q.d_in, q.act_order) for _ in range(ncopy)]
    out = {}
    stream = torch.cuda.current_stream()
    for m in (1, 8):
        A = Xd[:m].contiguous()
        ws = torch.zeros(max(P.dequant_matmul_workspace_size(m, wl.d_out, wl.d_in, q.bits, q.group_size), 1),
                         dtype=torch.uint8, device=A.device)
        Y = [P.dequant_matmul(A, c, workspace=ws) for c in copies[:2]]   # warm
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(calls):
            P.dequant_matmul(A, copies[i % ncopy], workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / calls
        nbytes = nbytes_w + A.numel() * A.element_size() + m * wl.d_out * 4
        gbs = nbytes / (us * 1e-6) / 1e9
        out[f"m{m}"] = {"us_per_call": us, "bytes_per_call": nbytes, "achieved_GBs": gbs, "peak_GBs": PEAK_HBM_GBS,
                        "frac": gbs / PEAK_HBM_GBS, "weight_copies": ncopy}
        log(f"bench: dequant product m={m}: {us:.2f} us/call, {gbs:.0f} GB/s")
    out["bound"] = "hbm"
    out["layer"] = f"{wl.d_out}x{wl.d_in} {q.bits}-bit group {q.group_size}, the layer just quantized"
    # prefill shape: the wide path (bf16 matrix cores), bound by them
    m = min(4096, Xd.shape[0])
    if Xd.dtype == torch.bfloat16 and wl.d_in % 8 == 0:
        A = Xd[:m].contiguous()
        ws = torch.zeros(max(P.dequant_matmul_workspace_size(m, wl.d_out, wl.d_in, q.bits, q.group_size), 1),
                         dtype=torch.uint8, device=A.device)
        P.dequant_matmul(A, q, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(20):
            P.dequant_matmul(A, q, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 20
        tf = 2.0 * m * wl.d_out * wl.d_in / (us * 1e-6) / 1e12
        out[f"m{m}"] = {"us_per_call": us, "tflops": tf, "peak_tflops": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS,
                        "bound": "mfma"}
        log(f"bench: dequant product m={m}: {us:.1f} us/call, {tf:.0f} TFLOP/s")
    return out


def other_workloads(P, torch, np, synth, skip):
    """Every other configuration of the layer, timed in the same run: inputs
    from the same seeded generator, resident in HBM; one untimed step, then a
    few timed ones (two for the 70B layer).  Per workload: ms per layer,
    TFLOP/s (Hessian + update flops), the Hessian product's average launch
    time (library hipEvents) and fraction of its peak, and the layer's
    roofline fraction (from one more step with every stage timed)."""
    out = {}
    dev = "cuda:0"
    for name, wl in synth.WORKLOADS.items():
        if name == skip:
            continue
        steps = 2 if wl.d_in > 16384 else 3
        t0 = time.perf_counter()
        W, X = synth.make_w(wl), synth.make_x(wl)

        def to_dev(a):
            if wl.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        Xd, Wd = to_dev(X), to_dev(W)
        del W, X
        H = torch.zeros(wl.d_in, wl.d_in, dtype=torch.float32, device=dev)
        code = P.BF16 if wl.dtype == "bf16" else P.F32
        ws_h = torch.empty(max(P.hessian_workspace_size(wl.n, wl.d_in, code), 1), dtype=torch.uint8, device=dev)
        ws_q = torch.empty(P.quantize_layer_workspace_size(wl.d_out, wl.d_in, wl.bits, wl.group_size,
                                                           wl.block_size, wl.act_order), dtype=torch.uint8, device=dev)

        def step():
            H.zero_()
            P.hessian_accumulate(Xd, H, workspace=ws_h)
            return P.quantize_layer(Wd, H, wl.bits, wl.group_size, wl.block_size, wl.damp, wl.act_order,
                                    workspace=ws_q)

        step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        P.profile_enable(1 << STAGE_HESSIAN_PRODUCT)
        P.profile_read(reset=True)
        ev0.record(stream)
        for _ in range(steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        ms_h, n_h = P.profile_read(reset=True)["hessian_product"]
        P.profile_enable(True)
        step()
        torch.cuda.synchronize()
        prof = P.profile_read(reset=True)
        P.profile_enable(False)
        stages = {k: {"ms_per_step": v[0], "launches_per_step": v[1]} for k, v in prof.items()}
        f_h, f_upd = workload_flops(wl)
        avg_h = ms_h / max(n_h, 1)
        peak_h = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
        out[name] = {"workload": describe(wl), "steps": steps, "ms_per_step": ms,
                     "tflops": (f_h + f_upd) / (ms * 1e-3) / 1e12,
                     "hessian_product": {"avg_launch_ms": avg_h, "achieved_tflops": f_h / (avg_h * 1e9),
                                         "peak_tflops": peak_h, "frac": f_h / (avg_h * 1e9) / peak_h},
                     "layer_roofline_frac": layer_roofline(wl, stages, ms)["frac"],
                     "stages_ms": {k: v["ms_per_step"] for k, v in stages.items()}}
        log(f"bench: {name}: {ms:.2f} ms per layer ({time.perf_counter() - t0:.1f} s with generation)")
        del Xd, Wd, H, ws_h, ws_q
        torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, W, X):
    """The float64 oracle on a bounded sample of the same workload, scaled to
    the whole layer: Hessian over n_s tokens (scaled by n / n_s), the inverse
    factor at d_s channels (scaled by (d/d_s)^3) and the quantization loop on
    r_s rows of a d_s-channel slice (scaled by (d_out/r_s) (d/d_s)^2)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O

    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores, user_api="blas"):
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
        d_s = min(wl.d_in, 4096)
        n_s = int(min(wl.n, max(512, 1e13 // (2 * d_s * d_s))))
        r_s = min(wl.d_out, 512)
        t0 = time.perf_counter()
        H = O.hessian([X[:n_s, :d_s]], wl.dtype, d_s)
        t_h = time.perf_counter() - t0
        t0 = time.perf_counter()
        perm = O.act_order_perm(H) if wl.act_order else np.arange(d_s)
        Hd = H[np.ix_(perm, perm)] + O.damping(H, wl.damp) * np.eye(d_s)
        U = O.inverse_cholesky_upper(Hd)
        t_f = time.perf_counter() - t0
        W0 = O.widen(W[:r_s, :d_s], wl.dtype)
        t0 = time.perf_counter()
        O.gptq(W0, H, wl.bits, wl.group_size, wl.block_size, wl.damp, wl.act_order, perm=perm, U=U)
        t_loop = time.perf_counter() - t0
    sc = wl.d_in / d_s
    t_full = t_h * (wl.n / n_s) * sc * sc + t_f * sc ** 3 + t_loop * (wl.d_out / r_s) * sc * sc
    f_h, f_upd = workload_flops(wl)
    return {
        "value": (f_h + f_upd) / t_full / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "ms_per_layer_est": t_full * 1e3,
        "sample": (f"float64 oracle: Hessian over {n_s} tokens x {d_s} channels ({t_h:.2f} s), inverse factor at "
                   f"d={d_s} ({t_f:.2f} s), quantization loop on {r_s} rows x {d_s} channels ({t_loop:.2f} s); "
                   f"scaled to the full layer ({wl.n} tokens, {wl.d_out}x{wl.d_in})"),
    }


def run_block(args, P, synth, torch, np):
    """One step = every linear layer of one transformer block: per input, H
    over the calibration tokens, then gptq_quantize_layers on the layers that
    read that input (one factorization per input instead of per layer)."""
    groups = synth.block_workloads(args.workload)
    b = synth.BLOCKS[args.workload]
    dev = "cuda:0"
    log(f"bench: generating the {args.workload} inputs ({len(groups)} inputs, "
        f"{sum(len(l) for _, l in groups)} layers, n={b['n']} tokens)")
    t0 = time.perf_counter()
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    data = []
    for xw, lws in groups:
        Xd = bf(synth.make_x(xw))
        Wds = [bf(synth.make_w(lw)) for lw in lws]
        data.append((xw, lws, Xd, Wds))
    log(f"bench: inputs ready in {time.perf_counter() - t0:.1f} s")
    dmax = max(xw.d_in for xw, *_ in data)
    H = torch.zeros(dmax * dmax, dtype=torch.float32, device=dev)
    ws_h = torch.empty(max(max(P.hessian_workspace_size(b["n"], xw.d_in, P.BF16) for xw, *_ in data), 1),
                       dtype=torch.uint8, device=dev)
    import ctypes
    need = 0
    for xw, lws, _, _ in data:
        d_outs = (ctypes.c_int64 * len(lws))(*[lw.d_out for lw in lws])
        need = max(need, P.lib.gptq_quantize_layers_workspace_size(len(lws), d_outs, xw.d_in, b["bits"],
                                                                   b["group_size"], b["block_size"],
                                                                   int(b["act_order"])))
    ws_q = torch.empty(need, dtype=torch.uint8, device=dev)

    def step():
        out = []
        for xw, lws, Xd, Wds in data:
            Hg = H[:xw.d_in * xw.d_in].view(xw.d_in, xw.d_in)
            Hg.zero_()
            P.hessian_accumulate(Xd, Hg, workspace=ws_h)
            out += P.quantize_layers(Wds, Hg, b["bits"], b["group_size"], b["block_size"], 0.01, b["act_order"],
                                     workspace=ws_q)
        return out

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"bench: warmup step {i + 1}/{args.warmup} done")
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    P.profile_enable(True)
    P.profile_read(reset=True)
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = P.profile_read(reset=True)
    P.profile_enable(False)
    f_h = sum(b["n"] * xw.d_in * (xw.d_in + 1) for xw, *_ in data)
    f_upd = sum(lw.d_out * lw.d_in * (lw.d_in - 1) for _, lws, *_ in data for lw in lws)
    f_factor = sum(2 * xw.d_in ** 3 / 3 for xw, *_ in data)
    n_layers = sum(len(lws) for _, lws, *_ in data)
    line = {
        "metric": f"GPTQ transformer-block sweep ms + TFLOP/s (Hessian+update), {args.workload}",
        "value": (f_h + f_upd) / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16+fp32", "data": "synthetic",
        "config": {"workload": f"{args.workload}: " + "; ".join(
            f"{xw.name} d_in={xw.d_in} -> " + ", ".join(f"{lw.name} {lw.d_out}x{lw.d_in}" for lw in lws)
            for xw, lws, *_ in data) + f"; n={b['n']} tokens, {b['bits']}-bit, group {b['group_size']}, "
            f"block {b['block_size']}, act_order {'on' if b['act_order'] else 'off'}",
            "layers": n_layers, "inputs": len(data), "parallelism": "single GPU"},
        "factorizations": {"per_step": len(data), "without_sharing": n_layers,
                           "factor_ms_per_step": prof["factor"][0] / args.steps,
                           "flops_per_step": f_factor},
        "stages": {k: {"ms_per_step": v[0] / args.steps, "launches_per_step": v[1] / args.steps}
                   for k, v in prof.items()},
        "flops": {"hessian": f_h, "update": f_upd},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="q_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemv", action="store_true", help="skip the product with the packed layer")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip timing the other layer configurations after the headline one")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run a plain device-to-device copy of MIB MiB three times (the known-size kernel "
                         "that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings) and exit")
    ap.add_argument("--unprofiled-check", action="store_true",
                    help="accepted for compatibility (the timed steps always run without per-stage events)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the quantizer runs on a single MI355X and has no "
              "multi-GPU path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}), flush=True)
        return

    import post_weight_quantization_04_amd as P
    from post_weight_quantization_04_amd import synth

    if args.workload in synth.BLOCKS:
        return run_block(args, P, synth, torch, np)
    wl = synth.WORKLOADS[args.workload]
    dev = "cuda:0"
    log(f"bench: generating {describe(wl)}")
    t0 = time.perf_counter()
    W = synth.make_w(wl)
    X = synth.make_x(wl)
    log(f"bench: inputs ready in {time.perf_counter() - t0:.1f} s; copying to HBM")

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    Xd, Wd = to_dev(X), to_dev(W)
    H = torch.zeros(wl.d_in, wl.d_in, dtype=torch.float32, device=dev)
    code = P.BF16 if wl.dtype == "bf16" else P.F32
    ws_h = torch.empty(max(P.hessian_workspace_size(wl.n, wl.d_in, code), 1), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(P.quantize_layer_workspace_size(wl.d_out, wl.d_in, wl.bits, wl.group_size, wl.block_size,
                                                       wl.act_order), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        H.zero_()
        P.hessian_accumulate(Xd, H, workspace=ws_h)
        return P.quantize_layer(Wd, H, wl.bits, wl.group_size, wl.block_size, wl.damp, wl.act_order, workspace=ws_q)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"bench: warmup step {i + 1}/{args.warmup} done")
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Timed region: only the Hessian product's launches carry an event pair
    # (its average duration feeds the roofline); every other stage runs bare.
    P.profile_enable(1 << STAGE_HESSIAN_PRODUCT)
    P.profile_read(reset=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    prof_h = P.profile_read(reset=True)
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"bench: {args.steps} timed steps, {ms_step:.3f} ms/step (wall {wall / args.steps * 1e3:.3f} ms/step)")
    # Stage breakdown: the same steps again with every stage timed (outside
    # the timed region; the events add a little to each stage)
    P.profile_enable(True)
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = P.profile_read(reset=True)
    P.profile_enable(False)

    f_h, f_upd = workload_flops(wl)
    value = (f_h + f_upd) / (ms_step * 1e-3) / 1e12
    stages = {k: {"ms_per_step": v[0] / args.steps, "launches_per_step": v[1] / args.steps} for k, v in prof.items()}
    ms_h, n_h = prof_h["hessian_product"]
    avg_h = ms_h / max(n_h, 1)
    achieved = f_h / (avg_h * 1e-3) / 1e12 if n_h else None
    traffic = measured_traffic(wl)
    roofline = {"kernel": "hess_bf16_kernel" if wl.dtype == "bf16" else "hess_f32_kernel",
                "bound": "mfma", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                "frac": (achieved / (PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS)) if achieved else None,
                "traffic": traffic, "avg_launch_ms": avg_h, "algorithmic_flops_per_launch": f_h}

    gemv = None
    if not args.no_gemv:
        gemv = gemv_bench(P, torch, wl, step(), Xd)

    others = None
    if not args.no_other_workloads:
        others = other_workloads(P, torch, np, synth, wl.name)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on a bounded sample")
        cpu = cpu_baseline(wl, W, X)
        log(f"bench: oracle {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")

    line = {
        "metric": f"GPTQ layer-quantize ms + TFLOP/s (Hessian+update), {wl.d_out}\u00d7{wl.d_in}, n={wl.n} tok",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16+fp32", "data": "synthetic",
        "config": {"workload": describe(wl), "d_out": wl.d_out, "d_in": wl.d_in, "tokens": wl.n,
                   "bits": wl.bits, "group_size": wl.group_size, "block_size": wl.block_size,
                   "act_order": wl.act_order, "damp": wl.damp, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layer_roofline": layer_roofline(wl, stages, ms_step),
        "dequant_gemv": gemv,
        "stages": stages,
        "other_workloads": others,
        "flops": {"hessian": f_h, "update": f_upd},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
