#!/usr/bin/env python3
"""Benchmark of the fused mixed-precision MoE layer on one MI355X.

    python bench.py [--workload dsv3_decode_mxfp4_bf16] [--steps K] [--warmup W]

One step = one pass of the whole layer (routing, token quantisation, GEMM1 +
SwiGLU, FC2 input, GEMM2, finalize) over one batch of synthetic tokens with
inputs and packed weights already resident in HBM.  Prints ONE JSON line.

The default workload is the DeepSeek-V3-shaped decode batch (64 tokens, 256
experts, top-8, hidden 7168, intermediate 2048, MXFP4 weights x BF16
activations), which is bound by HBM bandwidth: the roofline entry reports the
GEMM1 kernel's achieved bytes (packed W1 codes + E8M0 scales of every expert
that receives a token) per launch over its average launch duration, measured
with HIP events recorded by the library on the kernel's stream.  Prefill
workloads report GEMM1 FLOP/s against the FP8 (or BF16) MFMA peak instead.

cpu_baseline: the CPU oracle (float64 NumPy), timed on this host on a bounded
sample of tokens of the same workload, with expert weights drawn by the host
generator and quantised before the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_inputs as MI  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "mxfp8": 5000.0, "mxfp4": 10100.0, "bf16": 2500.0}
COPY_CALIB_BYTES = 256 << 20
METRIC = "fused-MoE tokens/s + % MFMA peak (prefill) / % HBM GB/s (decode), 1 GPU"
ORACLE_SAMPLE_TOKENS = {"tiny_mxfp4_fp8": 16, "dsv3_decode_mxfp4_bf16": 12,
                        "dsv3_prefill_mxfp4_fp8": 12, "dsv4pro_prefill_mxfp4_fp8": 24,
                        "dsv3_int4_fp8": 9, "dsv3_prefill_mxfp4_mxfp8": 12,
                        "dsv3_prefill_mxfp4_mxfp4": 12}
CSRC = "mixed_precision_moe_topk_amd/csrc/"


def gemm_source_sha256(afmt, cfg):
    """SHA-256 of the sources of the GEMM kernel that runs for this activation
    format and tile configuration (16-row tiles and BF16 activations use the
    register-direct kernel, the rest the LDS-staged kernels)."""
    import hashlib

    kfile = "moe_gemm_direct.hip" if (cfg == 0 or afmt == "bf16") else "moe_gemm_lds.hip"
    h = hashlib.sha256()
    for f in (kfile, "moe_gemm_common.h", "moe_common.h"):
        h.update(open(os.path.join(ROOT, CSRC + f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload, source_sha):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a calibration copy), or None when no
    summary exists or the kernel's source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"gemm1_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("gemm_source_sha256") != source_sha:
        return None
    return float(rec["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_decode_mxfp4_bf16", choices=sorted(MI.WORKLOADS))
    ap.add_argument("--weights", default="device", choices=["device", "host"],
                    help="draw float32 masters on the device (torch Philox, fast) or with the "
                         "host generator shared with the oracle (slow for 256+ experts)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--autotune", action="store_true",
                    help="validate and time every GEMM tile configuration on the workload's "
                         "inputs before the timed region, and run the fastest")
    return ap.parse_args()


def device_weights(d, wl, torch, chunk=8):
    """Packed weights from float32 N(0, 0.02) masters drawn on the device."""
    import mixed_precision_moe_topk_amd as M

    wb, sb = M.weights_query(d)
    weights = torch.empty(wb, dtype=torch.uint8, device="cuda")
    scales = torch.empty(sb, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    for e0 in range(0, wl.experts, chunk):
        n = min(chunk, wl.experts - e0)
        w1 = torch.randn((n, 2 * wl.inter, wl.hidden), generator=g, device="cuda") * 0.02
        w2 = torch.randn((n, wl.hidden, wl.inter), generator=g, device="cuda") * 0.02
        M.prepare_weights(d, w1, w2, e0, weights, scales)
        del w1, w2
    torch.cuda.synchronize()
    return weights, scales


def cpu_baseline(wl):
    import oracle as O

    s = min(ORACLE_SAMPLE_TOKENS.get(wl.key, 4), wl.tokens)
    hb = MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)[:s]
    lg = MI.router_logits(wl.seed, wl.tokens, wl.experts, wl.bias_sigma)[:s]
    ids, _ = O.route(lg, wl.top_k)
    need = sorted(set(ids.reshape(-1).tolist()))
    cache = {}
    for e, w1, w2 in MI.expert_weights_many(wl.seed, need, wl.hidden, wl.inter):
        cache[e] = O.quantize_expert(w1, w2, wl.wfmt)  # quantised before the timed region
    t0 = time.perf_counter()
    O.forward(hb, lg, wl.top_k, lambda e: cache[e], wl.wfmt, wl.afmt)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": round(s / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {s} tokens of the workload ({len(need)} experts), float64 oracle "
                      f"routing->output, {dt:.2f} s; weights quantised beforehand"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU only (expert-parallel sharding "
                                   "across GPUs is not implemented); --gpus must be 1"}))
        return 2
    import torch

    import mixed_precision_moe_topk_amd as M

    wl = MI.WORKLOADS[args.workload]
    d = M.LayerDims(wl.experts, wl.hidden, wl.inter, wl.wfmt, wl.afmt)
    print(f"# workload {wl.key}: preparing weights ({args.weights})", file=sys.stderr, flush=True)
    if args.weights == "device":
        weights, scales = device_weights(d, wl, torch)
    else:
        from mixed_precision_moe_topk_amd.staging import prepare_from_host
        weights, scales = prepare_from_host(
            d, MI.expert_weights_many(wl.seed, range(wl.experts), wl.hidden, wl.inter))
    hidden = torch.from_numpy(MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden).view(np.int16)).cuda()
    logits = torch.from_numpy(MI.router_logits(wl.seed, wl.tokens, wl.experts, wl.bias_sigma)).cuda()
    out = torch.empty((wl.tokens, wl.hidden), dtype=torch.int16, device="cuda")
    default_cfg = M.workspace_layout(d, wl.tokens, wl.top_k).gemm_cfg
    tuning = None
    if args.autotune:
        print("# autotune", file=sys.stderr, flush=True)
        chosen, cfg_ms = M.autotune(d, hidden, logits, weights, scales, wl.top_k, iters=5)
        tuning = {"default_cfg": default_cfg, "chosen_cfg": chosen,
                  "layer_ms_per_cfg": [round(m, 4) for m in cfg_ms]}
    lay = M.workspace_layout(d, wl.tokens, wl.top_k)
    ws = torch.empty(lay.total, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    # A plain device copy of known size (256 MiB read + 256 MiB written), run
    # before the timed region: rocprofv3 FETCH_SIZE / WRITE_SIZE counters read
    # for it calibrate the counters read for the layer's kernels.
    calib_src = torch.ones(COPY_CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    print(f"# warmup {args.warmup}, timed {args.steps}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        M.run_ws(d, hidden, logits, weights, scales, wl.top_k, out, ws, stream=stream)
    torch.cuda.synchronize()
    # timed region: HIP events around GEMM1 only (two per step; a full stage
    # trace would add seven event records to every step)
    M.trace_enable(M.TRACE_GEMM1)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        M.run_ws(d, hidden, logits, weights, scales, wl.top_k, out, ws, stream=stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    M.trace_enable(M.TRACE_OFF)
    calls, stage_ms = M.trace_read()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gemm1_ms = stage_ms["gemm1"] / max(calls, 1)
    # per-stage breakdown from a separate, untimed traced pass
    M.trace_enable(M.TRACE_ALL)
    for _ in range(min(args.steps, 10)):
        M.run_ws(d, hidden, logits, weights, scales, wl.top_k, out, ws, stream=stream)
    torch.cuda.synchronize()
    M.trace_enable(M.TRACE_OFF)
    bcalls, bstage_ms = M.trace_read()
    stage_avg = {k: v / max(bcalls, 1) for k, v in bstage_ms.items()}

    offsets = ws[lay.offsets:lay.offsets + 4 * (wl.experts + 1)].cpu().numpy().view(np.int32)
    active = int(np.count_nonzero(np.diff(offsets)))
    rows = wl.tokens * wl.top_k
    wbytes, sbytes = M.weights_query(d)
    per_expert = (wbytes + sbytes) / wl.experts
    # packed W1 of one expert: 2I x H E2M1/INT4 codes plus its scales
    w1_codes = wl.inter * wl.hidden
    if wl.wfmt == "mxfp4":
        w1_scales = 2 * wl.inter * (-(-wl.hidden // 512)) * 16
    else:
        w1_scales = 2 * wl.inter * (wl.hidden // 128) * 4
    gemm1_bytes = active * (w1_codes + w1_scales)
    gemm1_flops = 2.0 * rows * 2 * wl.inter * wl.hidden
    g1_s = gemm1_ms / 1e3
    src_sha = gemm_source_sha256(wl.afmt, lay.gemm_cfg)
    if wl.regime in ("hbm", "latency"):
        achieved = gemm1_bytes / g1_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(wl.key, src_sha)}
    else:
        achieved = gemm1_flops / g1_s / 1e12
        peak = MFMA_PEAK_TFLOPS[wl.afmt]
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(wl.key, src_sha)}
    roof["kernel"] = "gemm1"
    roof["kernel_ms"] = round(gemm1_ms, 4)
    roof["kernel_source_sha256"] = src_sha
    roof["algorithmic_bytes"] = gemm1_bytes if wl.regime in ("hbm", "latency") else None
    roof["algorithmic_flops"] = gemm1_flops

    layer_bytes = active * per_expert
    layer_flops = 6.0 * rows * wl.inter * wl.hidden
    rec = {
        "metric": METRIC,
        "value": round(wl.tokens / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # operand type of the matrix products: bf16, E4M3 (FP8, MXFP8) or E2M1 (W4A4)
        "dtype": {"bf16": "bf16", "mxfp4": "fp4"}.get(wl.afmt, "fp8"),
        "data": "synthetic",
        "config": {"workload": wl.key, "tokens": wl.tokens, "experts": wl.experts,
                   "top_k": wl.top_k, "hidden": wl.hidden, "inter": wl.inter,
                   "weights": wl.wfmt, "activations": wl.afmt, "active_experts": active,
                   "gemm_cfg": lay.gemm_cfg, "tile_m": lay.tile_m,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer": {"weight_GBps": round(layer_bytes / (ms_per_step / 1e3) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                  "gemm_TFLOPs": round(layer_flops / (ms_per_step / 1e3) / 1e12, 1),
                  "stage_ms": {k: round(v, 4) for k, v in stage_avg.items()}},
    }
    if tuning is not None:
        rec["autotune"] = tuning
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
