"""Seeded synthetic inputs for the fused MoE layer.

This module is shared by the CPU oracle, the tests and the benchmark.  It holds
only workload shapes and random number draws: no routing, quantisation or GEMM
arithmetic of the layer lives here.

Workloads (shapes of the DeepSeek-V3 and DeepSeek-V4-Pro MoE layers named in the
"Performance" section of flashinfer PR #3738, "perf: optimize MXFP4xBF16 &
INT4xFP8 and add MXFP4xFP8 CUTLASS MoE backend for SM90"; the pages use no
dataset, so every tensor is drawn here):

* hidden states: bf16 rounding (round-to-nearest-even) of float32 N(0, 1);
* router logits: float32 N(0, 1); the skewed-load workload adds a per-expert
  bias drawn as float32 N(0, 1) times 2 (standard deviation 2), shared by all
  tokens, added in float32;
* expert weights: float32 N(0, 1) times float32(0.02), drawn expert by expert
  so that the float32 masters of a 256-expert layer (45 GB) are never resident.

Every draw uses numpy's PCG64 seeded with SeedSequence([seed, tensor_id,
expert]); tensor ids: 0 hidden, 1 logits, 2 bias, 3 W1, 4 W2.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os as _os
from dataclasses import dataclass

import numpy as np

TENSOR_HIDDEN, TENSOR_LOGITS, TENSOR_BIAS, TENSOR_W1, TENSOR_W2 = 0, 1, 2, 3, 4
WEIGHT_STD = np.float32(0.02)


@dataclass(frozen=True)
class Workload:
    """One MoE layer shape plus its weight/activation formats."""

    key: str
    seed: int
    tokens: int
    experts: int
    top_k: int
    hidden: int
    inter: int
    wfmt: str  # "mxfp4" or "int4"
    afmt: str  # "fp8" (per-token E4M3), "mxfp8" (E4M3 + E8M0 per 32) or "bf16"
    bias_sigma: float = 0.0
    regime: str = ""

    def with_tokens(self, tokens: int) -> "Workload":
        return Workload(self.key, self.seed, tokens, self.experts, self.top_k,
                        self.hidden, self.inter, self.wfmt, self.afmt,
                        self.bias_sigma, self.regime)


WORKLOADS = {
    "tiny_mxfp4_fp8": Workload("tiny_mxfp4_fp8", 1, 16, 8, 2, 256, 512,
                               "mxfp4", "fp8", 0.0, "latency"),
    "dsv3_decode_mxfp4_bf16": Workload("dsv3_decode_mxfp4_bf16", 2, 64, 256, 8,
                                       7168, 2048, "mxfp4", "bf16", 0.0, "hbm"),
    "dsv3_prefill_mxfp4_fp8": Workload("dsv3_prefill_mxfp4_fp8", 3, 4096, 256, 8,
                                       7168, 2048, "mxfp4", "fp8", 0.0, "mfma"),
    "dsv4pro_prefill_mxfp4_fp8": Workload("dsv4pro_prefill_mxfp4_fp8", 4, 16384,
                                          384, 6, 7168, 3072, "mxfp4", "fp8",
                                          2.0, "mfma"),
    "dsv3_int4_fp8": Workload("dsv3_int4_fp8", 5, 1024, 256, 8, 7168, 2048,
                              "int4", "fp8", 0.0, "hbm"),
    # the DeepSeek-V3 prefill shape with MXFP8 activations (E8M0 per 32)
    "dsv3_prefill_mxfp4_mxfp8": Workload("dsv3_prefill_mxfp4_mxfp8", 6, 4096, 256, 8,
                                         7168, 2048, "mxfp4", "mxfp8", 0.0, "mfma"),
    # the same shape with W4A4: MXFP4 activations (E2M1, E8M0 per 32)
    "dsv3_prefill_mxfp4_mxfp4": Workload("dsv3_prefill_mxfp4_mxfp4", 7, 4096, 256, 8,
                                         7168, 2048, "mxfp4", "mxfp4", 0.0, "mfma"),
}


def _rng(seed: int, tensor_id: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, tensor_id, expert])))


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    # torch's float32 -> bfloat16 cast rounds to nearest even; used here as a
    # plain data-type conversion of the drawn values.
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def hidden_bf16(seed: int, tokens: int, hidden: int) -> np.ndarray:
    """bf16 bit patterns (uint16) of shape [tokens, hidden]."""
    x = _rng(seed, TENSOR_HIDDEN).standard_normal((tokens, hidden), dtype=np.float32)
    return _to_bf16_bits(x)


def router_logits(seed: int, tokens: int, experts: int,
                  bias_sigma: float = 0.0) -> np.ndarray:
    """float32 logits [tokens, experts]; optional shared per-expert bias."""
    z = _rng(seed, TENSOR_LOGITS).standard_normal((tokens, experts), dtype=np.float32)
    if bias_sigma:
        b = _rng(seed, TENSOR_BIAS).standard_normal(experts, dtype=np.float32)
        b = (np.float32(bias_sigma) * b).astype(np.float32)
        z = (z + b[None, :]).astype(np.float32)
    return z


def expert_weights(seed: int, expert: int, hidden: int, inter: int):
    """float32 masters of one expert: W1 [2*inter, hidden] (rows [0, inter) are
    the gate projection, rows [inter, 2*inter) the up projection) and
    W2 [hidden, inter]."""
    w1 = _rng(seed, TENSOR_W1, expert).standard_normal((2 * inter, hidden), dtype=np.float32)
    w1 *= WEIGHT_STD
    w2 = _rng(seed, TENSOR_W2, expert).standard_normal((hidden, inter), dtype=np.float32)
    w2 *= WEIGHT_STD
    return w1, w2


def expert_weights_many(seed: int, experts, hidden: int, inter: int, threads: int | None = None):
    """Yields (expert, W1, W2) for the given experts, drawn on a thread pool
    (numpy releases the GIL while filling), in the order given."""
    experts = list(experts)
    threads = threads or min(16, _os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=threads) as pool:
        futs = {}
        ahead = threads
        for i, e in enumerate(experts[:ahead]):
            futs[i] = pool.submit(expert_weights, seed, e, hidden, inter)
        for i, e in enumerate(experts):
            w1, w2 = futs.pop(i).result()
            j = i + ahead
            if j < len(experts):
                futs[j] = pool.submit(expert_weights, seed, experts[j], hidden, inter)
            yield e, w1, w2


def small_workload(tokens=24, experts=6, top_k=3, hidden=384, inter=256,
                   wfmt="mxfp4", afmt="fp8", seed=101, bias_sigma=0.0) -> Workload:
    """A custom small shape (parity tests at sizes the oracle finishes in seconds)."""
    return Workload(f"custom_{seed}", seed, tokens, experts, top_k, hidden, inter,
                    wfmt, afmt, bias_sigma, "test")
