"""Python binding of the MI355X fused mixed-precision MoE library (libmoe_amd.so).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library; PyTorch provides device memory and the current stream.  The C
ABI is declared in include/moe.h.  If the library is missing every call raises
(there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_amd.so")

W_MXFP4, W_INT4_G128 = 0, 1
A_FP8_TOKEN, A_BF16, A_MXFP8, A_MXFP4 = 0, 1, 2, 3
WFMT = {"mxfp4": W_MXFP4, "int4": W_INT4_G128}
AFMT = {"fp8": A_FP8_TOKEN, "bf16": A_BF16, "mxfp8": A_MXFP8, "mxfp4": A_MXFP4}

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP", 5: "MOE_ERR_INTERNAL"}

EXPORTS = ("moe_abi_version", "moe_last_error", "moe_weights_query", "moe_prepare_weights",
           "moe_unpack_weights", "moe_workspace_query", "moe_workspace_layout", "moe_run_ws",
           "moe_run", "moe_route", "moe_quantize_tokens", "moe_tune_set", "moe_tune_clear",
           "moe_autotune", "moe_trace_enable", "moe_trace_read", "moe_release_arenas",
           "moe_set_fc2_fused", "moe_run_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES
STAGES = ("route", "quant", "gemm1", "requant", "gemm2", "finalize")


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("wfmt", ctypes.c_int32), ("afmt", ctypes.c_int32)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "total", "ids", "topk_w", "chunk_counts", "offsets", "row_token", "slot_row", "tiles",
        "num_tiles", "tok_codes", "tok_scales", "h", "fc2_codes", "fc2_scales", "y2")] + [
        ("tile_m", ctypes.c_int32), ("gemm_cfg", ctypes.c_int32), ("max_tiles", ctypes.c_int64),
        ("tok_bscales", ctypes.c_size_t), ("fc2_bscales", ctypes.c_size_t),
        ("fc2_fused", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixed_precision_moe_topk_amd.build`")
        # torch ships its own HIP runtime (soname libamdhip64.so.7, loaded by
        # torch under the file name libamdhip64.so).  Loaded first, it also
        # satisfies the library's libamdhip64.so.7 dependency, so the process
        # has one runtime; the library loaded first would bring the system
        # runtime and torch a second one, and one of the two would find no
        # device.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        DP = ctypes.POINTER(Dims)
        L.moe_abi_version.restype = I32
        L.moe_last_error.restype = ctypes.c_char_p
        sig = {
            "moe_weights_query": [DP, ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
            "moe_prepare_weights": [DP, P, P, I32, I32, P, P, P],
            "moe_unpack_weights": [DP, P, P, I32, I32, P, P, P, P, P],
            "moe_workspace_query": [DP, I64, I32, ctypes.POINTER(SZ)],
            "moe_workspace_layout": [DP, I64, I32, ctypes.POINTER(WsLayout)],
            "moe_run_ws": [DP, P, I64, P, P, P, I32, P, P, SZ, P],
            "moe_run": [DP, P, I64, P, P, P, I32, P, P],
            "moe_run_noalloc": [DP, P, I64, P, P, P, I32, P, P],
            "moe_route": [DP, P, I64, I32, P, P, P, P, P, P, SZ, P],
            "moe_quantize_tokens": [DP, P, I64, P, P, P, P],
            "moe_tune_set": [DP, I64, I32, I32],
            "moe_tune_clear": [],
            "moe_autotune": [DP, P, I64, P, P, P, I32, I32, ctypes.POINTER(I32),
                             ctypes.POINTER(ctypes.c_float), P],
            "moe_trace_enable": [I32],
            "moe_release_arenas": [],
            "moe_set_fc2_fused": [I32],
            "moe_trace_read": [ctypes.POINTER(ctypes.c_float), I32, ctypes.POINTER(I32)],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclass(frozen=True)
class LayerDims:
    num_experts: int
    hidden: int
    inter: int
    wfmt: str = "mxfp4"
    afmt: str = "fp8"

    def c(self) -> Dims:
        return Dims(self.num_experts, self.hidden, self.inter, WFMT[self.wfmt], AFMT[self.afmt])


def abi_version() -> int:
    return lib().moe_abi_version()


def weights_query(d: LayerDims):
    w, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().moe_weights_query(ctypes.byref(d.c()), ctypes.byref(w), ctypes.byref(s)))
    return w.value, s.value


def prepare_weights(d: LayerDims, w1, w2, expert_begin: int, weights, scales, stream=None):
    """w1: float32 cuda [n, 2I, H]; w2: float32 cuda [n, H, I] for experts
    [expert_begin, expert_begin + n); weights/scales: uint8 cuda buffers."""
    n = 0 if w1 is None else int(w1.shape[0])
    _check(lib().moe_prepare_weights(ctypes.byref(d.c()), _ptr(w1), _ptr(w2), expert_begin, n,
                                     _ptr(weights), _ptr(scales), _stream(stream)))


def unpack_weights(d: LayerDims, weights, scales, expert_begin: int, w1q, w1s, w2q, w2s,
                   stream=None):
    n = int(w1q.shape[0])
    _check(lib().moe_unpack_weights(ctypes.byref(d.c()), _ptr(weights), _ptr(scales),
                                    expert_begin, n, _ptr(w1q), _ptr(w1s), _ptr(w2q), _ptr(w2s),
                                    _stream(stream)))


def workspace_query(d: LayerDims, num_tokens: int, top_k: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().moe_workspace_query(ctypes.byref(d.c()), num_tokens, top_k, ctypes.byref(b)))
    return b.value


def workspace_layout(d: LayerDims, num_tokens: int, top_k: int) -> WsLayout:
    L = WsLayout()
    _check(lib().moe_workspace_layout(ctypes.byref(d.c()), num_tokens, top_k, ctypes.byref(L)))
    return L


def run_ws(d: LayerDims, hidden, logits, weights, scales, top_k: int, out, workspace,
           stream=None):
    """hidden: bf16 (or int16 bits) cuda [T, H]; logits: float32 cuda [T, E];
    out: bf16 cuda [T, H]; workspace: uint8 cuda of workspace_query bytes."""
    T = int(hidden.shape[0])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_run_ws(ctypes.byref(d.c()), _ptr(hidden), T, _ptr(logits), _ptr(weights),
                            _ptr(scales), top_k, _ptr(out), _ptr(workspace), nbytes,
                            _stream(stream)))


def run(d: LayerDims, hidden, logits, weights, scales, top_k: int, out, stream=None):
    T = int(hidden.shape[0])
    _check(lib().moe_run(ctypes.byref(d.c()), _ptr(hidden), T, _ptr(logits), _ptr(weights),
                         _ptr(scales), top_k, _ptr(out), _stream(stream)))


def run_noalloc(d: LayerDims, hidden, logits, weights, scales, top_k: int, out, stream=None):
    """The layer with the library's static device workspace (allocates
    nothing; workspaces above NOALLOC_SCRATCH_BYTES are refused)."""
    T = int(hidden.shape[0])
    _check(lib().moe_run_noalloc(ctypes.byref(d.c()), _ptr(hidden), T, _ptr(logits),
                                 _ptr(weights), _ptr(scales), top_k, _ptr(out), _stream(stream)))


def route(d: LayerDims, logits, top_k: int, ids, weights, expert_offsets, row_token,
          slot_row, workspace, stream=None):
    """The routing step alone.  logits: float32 cuda [T, E]; outputs int32/
    float32 cuda: ids [T, k], weights [T, k], expert_offsets [E + 1],
    row_token [T*k], slot_row [T, k]; workspace: uint8 cuda of
    workspace_query bytes."""
    T = int(logits.shape[0])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_route(ctypes.byref(d.c()), _ptr(logits), T, top_k, _ptr(ids), _ptr(weights),
                           _ptr(expert_offsets), _ptr(row_token), _ptr(slot_row),
                           _ptr(workspace), nbytes, _stream(stream)))


def quantize_tokens(d: LayerDims, hidden, codes, scales, block_scales=None, stream=None):
    """The token quantisation step alone.  hidden: bf16 bits cuda [T, H];
    codes: uint8 cuda [T, H] (E4M3) or [T, H/2] (E2M1); scales: float32 cuda
    [T]; block_scales: uint8 cuda [T, 16*ceil(H/512)] for the MX formats."""
    T = int(hidden.shape[0])
    _check(lib().moe_quantize_tokens(ctypes.byref(d.c()), _ptr(hidden), T, _ptr(codes),
                                     _ptr(scales), _ptr(block_scales), _stream(stream)))


NUM_GEMM_CFG = 3


def tune_set(d: LayerDims, num_tokens: int, top_k: int, gemm_cfg: int):
    """Tile configuration for this shape and token bucket (-1 removes it)."""
    _check(lib().moe_tune_set(ctypes.byref(d.c()), num_tokens, top_k, gemm_cfg))


def tune_clear():
    _check(lib().moe_tune_clear())


def autotune(d: LayerDims, hidden, logits, weights, scales, top_k: int, iters: int = 5,
             stream=None):
    """Validates and times every tile configuration on these inputs, keeps the
    fastest for the shape and token bucket; -> (chosen, [ms per call or -1])."""
    T = int(hidden.shape[0])
    chosen = ctypes.c_int32()
    ms = (ctypes.c_float * NUM_GEMM_CFG)()
    _check(lib().moe_autotune(ctypes.byref(d.c()), _ptr(hidden), T, _ptr(logits), _ptr(weights),
                              _ptr(scales), top_k, iters, ctypes.byref(chosen), ms,
                              _stream(stream)))
    return chosen.value, [float(v) for v in ms]


TRACE_OFF, TRACE_ALL, TRACE_GEMM1 = 0, 1, 2


def trace_enable(mode=TRACE_ALL):
    """Stage timing: TRACE_ALL (every stage), TRACE_GEMM1 (GEMM1 only, two
    events per call) or TRACE_OFF; True / False mean TRACE_ALL / TRACE_OFF."""
    if mode is True:
        mode = TRACE_ALL
    elif mode is False:
        mode = TRACE_OFF
    _check(lib().moe_trace_enable(int(mode)))


def trace_read():
    """-> (calls, {stage: summed ms}) of the calls recorded since the last read."""
    n = len(STAGES)
    arr = (ctypes.c_float * n)()
    calls = ctypes.c_int32()
    _check(lib().moe_trace_read(arr, n, ctypes.byref(calls)))
    return calls.value, {s: float(arr[i]) for i, s in enumerate(STAGES)}


def release_arenas():
    """Frees the workspaces moe_run keeps per device and stream."""
    _check(lib().moe_release_arenas())


def set_fc2_fused(enable: bool):
    """Test hook: False makes GEMM1 store float32 h and the separate FC2
    quantiser run for every format (process-wide; changes the workspace
    layout)."""
    _check(lib().moe_set_fc2_fused(1 if enable else 0))
