#!/usr/bin/env python3
"""Benchmark of the fused mixed-precision MoE layer on one MI355X.

    python bench.py [--workload dsv4pro_prefill_mxfp4_fp8] [--steps K] [--warmup W]

One step = one pass of the whole layer (routing, token quantisation, GEMM1 +
SwiGLU, FC2 input, GEMM2, finalize) over one batch of synthetic tokens with
inputs and packed weights already resident in HBM.  Prints ONE JSON line.

The default workload is the largest one, the DeepSeek-V4-Pro-shaped prefill
batch (16384 tokens, 384 experts, top-6, hidden 7168, intermediate 3072,
MXFP4 weights x per-token E4M3 activations, router logits with a per-expert
bias for skewed loads), which is bound by the matrix cores: the roofline
entry reports the GEMM1 kernel's algorithmic FLOP/s (2 * rows * 2I * H per
launch over its average launch duration, measured with HIP events the
library records on the kernel's stream) against the FP8 MFMA peak, and
`layer` the whole layer's GEMM FLOP/s against the same peak.  The
HBM-bound workloads (decode, INT4) report GEMM1's active-expert weight bytes
per second against the HBM peak instead.

cpu_baseline: the CPU oracle (float64 NumPy) timed on this host.  Its cost
is dominated by the expert passes (weight decode plus the rows' GEMMs), so
it is timed on all tokens with the expert passes of a random sample of whole
active experts, and once with no expert pass (routing, token quantisation,
finalize); the layer time is the latter plus the sampled passes scaled by
active / sampled experts.  Weights are quantised before the timed region.
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
# active experts whose whole expert pass the CPU baseline times
ORACLE_SAMPLE_EXPERTS = {"tiny_mxfp4_fp8": 8, "dsv3_decode_mxfp4_bf16": 16,
                         "dsv3_prefill_mxfp4_fp8": 8, "dsv4pro_prefill_mxfp4_fp8": 6,
                         "dsv3_int4_fp8": 10, "dsv3_prefill_mxfp4_mxfp8": 8,
                         "dsv3_prefill_mxfp4_mxfp4": 8}
DEFAULT_WORKLOAD = "dsv4pro_prefill_mxfp4_fp8"
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
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(MI.WORKLOADS))
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


def cpu_model():
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl):
    """Oracle layer time on this host, estimated from timed parts of the
    oracle on the full workload (see the module docstring)."""
    import oracle as O

    hb = MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)
    lg = MI.router_logits(wl.seed, wl.tokens, wl.experts, wl.bias_sigma)
    ids, _ = O.route(lg, wl.top_k)
    counts = np.bincount(ids.reshape(-1), minlength=wl.experts)
    active = np.flatnonzero(counts)
    by_rows = active[np.argsort(counts[active], kind="stable")]
    m = min(ORACLE_SAMPLE_EXPERTS.get(wl.key, 8), len(active))
    # systematic sample over the experts sorted by rows, plus the hottest one
    pick = ((np.arange(max(m - 1, 1)) + 0.5) * len(by_rows) / max(m - 1, 1)).astype(int)
    sample = sorted(set(by_rows[pick].tolist()) | {int(by_rows[-1])})
    cache = {}
    for e, w1, w2 in MI.expert_weights_many(wl.seed, sample, wl.hidden, wl.inter):
        cache[e] = O.quantize_expert(w1, w2, wl.wfmt)  # quantised before the timed region
    t0 = time.perf_counter()
    O.forward(hb, lg, wl.top_k, lambda e: cache[e], wl.wfmt, wl.afmt, only_experts=set())
    t1 = time.perf_counter()
    O.forward(hb, lg, wl.top_k, lambda e: cache[e], wl.wfmt, wl.afmt, only_experts=set(sample))
    t2 = time.perf_counter()
    ex = cache[sample[0]]
    O.layer.decode_weight(ex.w1q, ex.w1s, wl.wfmt)
    O.layer.decode_weight(ex.w2q, ex.w2s, wl.wfmt)
    t3 = time.perf_counter()
    t_tok = t1 - t0                      # routing, token quantisation, finalize
    t_pass = max(t2 - t1 - t_tok, 0.0)   # the sampled expert passes
    t_dec = t3 - t2                      # decoding one expert's weights
    rows_s = int(counts[sample].sum())
    per_row = max(t_pass - len(sample) * t_dec, 0.0) / max(rows_s, 1)
    rows = wl.tokens * wl.top_k
    est = t_tok + len(active) * t_dec + rows * per_row
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": round(wl.tokens / est, 2), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"float64 oracle on all {wl.tokens} tokens: routing + token quant + "
                      f"finalize {t_tok:.2f} s; expert passes of {len(sample)} of the "
                      f"{len(active)} active experts (the hottest plus a systematic sample by "
                      f"rows; {rows_s} of {rows} rows) {t_pass:.2f} s; one expert's weight "
                      f"decode {t_dec:.3f} s; layer estimate {est:.1f} s = token steps + "
                      f"{len(active)} x decode + {rows} rows x {per_row * 1e3:.3f} ms/row; "
                      f"weights quantised beforehand"}


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
                  "mfma_frac": round(layer_flops / (ms_per_step / 1e3) / 1e12
                                     / MFMA_PEAK_TFLOPS[wl.afmt], 4),
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
