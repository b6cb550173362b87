"""The C-ABI library loads, exports every symbol include/moe.h declares, and
rejects bad arguments on the host before touching a device (CPU only)."""
import ctypes
import os
import re

import pytest

import mixed_precision_moe_topk_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|int32_t|const char\*)\s+(moe_\w+)\(", src, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(M.LIB_PATH):
        pytest.skip("library not built")
    return M.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(M.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert L.moe_abi_version() == 7


def _d(**kw):
    base = dict(num_experts=256, hidden=7168, inter=2048, wfmt="mxfp4", afmt="fp8")
    base.update(kw)
    return M.LayerDims(**base)


def test_weight_sizes(L):
    w, s = M.weights_query(_d())
    assert w == 256 * (2 * 2048 * 7168 + 7168 * 2048) // 2
    assert s == 256 * (2 * 2048 * 7168 + 7168 * 2048) // 32
    w, s = M.weights_query(_d(wfmt="int4"))
    assert s == 256 * (2 * 2048 * 7168 + 7168 * 2048) // 128 * 4
    # K/128 not a multiple of 4: scale rows are padded to 512-element chunks
    w, s = M.weights_query(_d(num_experts=8, hidden=256, inter=512))
    assert s == 8 * (1024 * 1 * 16 + 256 * 1 * 16)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=100), 1), (dict(inter=0), 1), (dict(num_experts=0), 1),
    (dict(num_experts=2000), 1), (dict(wfmt="int4", afmt="bf16"), 2),
    (dict(wfmt="int4", afmt="mxfp8"), 2), (dict(wfmt="int4", afmt="mxfp4"), 2)])
def test_bad_dims(L, kw, status):
    with pytest.raises(M.MoeError) as ei:
        M.weights_query(_d(**kw))
    assert ei.value.status == status


def test_bad_topk_and_tokens(L):
    with pytest.raises(M.MoeError) as ei:
        M.workspace_query(_d(num_experts=8), 16, 9)
    assert ei.value.status == 1
    with pytest.raises(M.MoeError):
        M.workspace_query(_d(), 16, 17)
    with pytest.raises(M.MoeError):
        M.workspace_query(_d(), -1, 8)
    assert M.workspace_query(_d(), 0, 8) > 0


def test_run_rejects_before_launch(L):
    d = _d(num_experts=8, hidden=256, inter=512).c()
    P = ctypes.c_void_p
    # T = 0 is a no-op success even with null pointers
    assert L.moe_run_ws(ctypes.byref(d), None, 0, None, None, None, 2, None, None, 0, None) == 0
    # null pointers
    assert L.moe_run_ws(ctypes.byref(d), None, 4, None, None, None, 2, None, None, 0, None) == 1
    # misaligned pointer
    fake = P(0x1000 + 8)
    ok = P(0x1000)
    assert L.moe_run_ws(ctypes.byref(d), fake, 4, ok, ok, ok, 2, ok, ok, 1 << 30, None) == 1
    # workspace too small
    assert L.moe_run_ws(ctypes.byref(d), ok, 4, ok, ok, ok, 2, ok, ok, 16, None) == 3
    assert b"workspace" in L.moe_last_error()
    # expert slice out of range
    assert L.moe_prepare_weights(ctypes.byref(d), ok, ok, 6, 3, ok, ok, None) == 1
    assert L.moe_prepare_weights(ctypes.byref(d), ok, ok, 0, 0, ok, ok, None) == 0


def test_workspace_layout_regions(L):
    lay = M.workspace_layout(_d(), 4096, 8)
    offs = [lay.ids, lay.topk_w, lay.chunk_counts, lay.offsets, lay.row_token, lay.slot_row,
            lay.tiles, lay.num_tiles, lay.tok_codes, lay.tok_scales, lay.h, lay.fc2_codes,
            lay.fc2_scales, lay.y2]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.y2 + 4096 * 8 * 7168 * 4 <= lay.total
    assert lay.tile_m == 160 and lay.gemm_cfg == 2
    assert M.workspace_layout(_d(), 64, 8).tile_m == 16


def test_workspace_layout_mxfp8(L):
    # MXFP8: E4M3 codes for tokens and FC2 inputs plus E8M0 block scales in
    # 16-byte groups per 512 columns (hidden 7168 -> 224 B, inter 2048 -> 64 B)
    lay = M.workspace_layout(_d(afmt="mxfp8"), 4096, 8)
    assert lay.tok_bscales % 256 == 0 and lay.fc2_bscales % 256 == 0
    assert lay.fc2_bscales >= lay.tok_bscales + 4096 * 224
    assert lay.fc2_bscales + 4096 * 8 * 64 <= lay.total
    assert lay.fc2_codes + 4096 * 8 * 2048 <= lay.fc2_scales  # one byte per code
    assert lay.tile_m == 160 and lay.gemm_cfg == 2
    # 384 columns: one partial group of 16 bytes per row
    lay = M.workspace_layout(_d(num_experts=8, hidden=384, inter=256, afmt="mxfp8"), 100, 2)
    assert lay.fc2_bscales - lay.tok_bscales >= 100 * 16
    assert M.workspace_layout(_d(), 4096, 8).tok_bscales == M.workspace_layout(_d(), 4096, 8).fc2_bscales


def test_tune_table(L):
    """Tuned tile configurations: per shape, top-k and token bucket
    ceil(log2 T); the workspace size never changes."""
    d = _d()
    M.tune_clear()
    base = M.workspace_layout(d, 4096, 8)
    assert base.gemm_cfg == 2
    try:
        M.tune_set(d, 4096, 8, 1)
        lay = M.workspace_layout(d, 4096, 8)
        assert lay.gemm_cfg == 1 and lay.tile_m == 64 and lay.total == base.total
        assert M.workspace_layout(d, 2049, 8).gemm_cfg == 1      # same bucket (2^12)
        assert M.workspace_layout(d, 2048, 8).gemm_cfg == 2      # bucket 2^11: default
        assert M.workspace_layout(d, 4096, 6).gemm_cfg == 2      # other top-k
        assert M.workspace_layout(_d(afmt="bf16"), 4096, 8).gemm_cfg == 2  # other format
        M.tune_set(d, 4096, 8, 0)
        lay = M.workspace_layout(d, 4096, 8)
        assert lay.tile_m == 16 and lay.total == base.total
        assert lay.max_tiles == 4096 * 8 // 16 + 256
        M.tune_set(d, 4096, 8, -1)                                # removal
        assert M.workspace_layout(d, 4096, 8).gemm_cfg == 2
        for bad in (3, -2):
            with pytest.raises(M.MoeError) as ei:
                M.tune_set(d, 4096, 8, bad)
            assert ei.value.status == 1
        with pytest.raises(M.MoeError):
            M.tune_set(d, 0, 8, 1)
        M.tune_set(d, 4096, 8, 1)
        M.tune_clear()
        assert M.workspace_layout(d, 4096, 8).gemm_cfg == 2
    finally:
        M.tune_clear()


def test_autotune_rejects_bad_args(L):
    d = _d(num_experts=8, hidden=256, inter=512).c()
    ok = ctypes.c_void_p(0x1000)
    chosen = ctypes.c_int32()
    # iters out of range and null result pointer fail before touching the device
    assert L.moe_autotune(ctypes.byref(d), ok, 4, ok, ok, ok, 2, 0, ctypes.byref(chosen), None,
                          None) == 1
    assert L.moe_autotune(ctypes.byref(d), ok, 4, ok, ok, ok, 2, 5, None, None, None) == 1
    assert L.moe_autotune(ctypes.byref(d), ok, 0, ok, ok, ok, 2, 5, ctypes.byref(chosen), None,
                          None) == 1


def test_workspace_layout_w4a4(L):
    # MXFP4 activations: packed E2M1 codes (half a byte each) plus the same
    # block-scale regions as MXFP8
    a = M.workspace_layout(_d(afmt="mxfp4"), 4096, 8)
    b = M.workspace_layout(_d(afmt="mxfp8"), 4096, 8)
    assert a.tok_scales - a.tok_codes >= 4096 * 7168 // 2
    assert a.fc2_scales - a.fc2_codes >= 4096 * 8 * 2048 // 2
    assert a.total < b.total
    assert a.fc2_bscales - a.tok_bscales == b.fc2_bscales - b.tok_bscales
    assert a.tile_m == 160 and a.gemm_cfg == 2
    # GEMM1 writes the FC2 input itself for the MX formats and BF16, not for per-token FP8
    assert a.fc2_fused == 1 and b.fc2_fused == 1
    assert M.workspace_layout(_d(afmt="mxfp4"), 64, 8).fc2_fused == 1
    assert M.workspace_layout(_d(), 4096, 8).fc2_fused == 0
    assert M.workspace_layout(_d(afmt="bf16"), 64, 8).fc2_fused == 1  # bf16(h) from GEMM1


def test_trace_modes(L):
    # off / all stages / GEMM1 only are accepted, anything else is an argument error
    for mode in (M.TRACE_ALL, M.TRACE_GEMM1, M.TRACE_OFF):
        assert L.moe_trace_enable(mode) == 0
    assert L.moe_trace_enable(7) == 1
    assert L.moe_trace_enable(M.TRACE_OFF) == 0


def test_stage_calls_reject_before_launch(L):
    """moe_route and moe_quantize_tokens check their arguments on the host:
    no device is touched for any of these cases."""
    d = _d(num_experts=8, hidden=256, inter=512).c()
    ok, bad = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1000 + 4)
    big = 1 << 30
    # T = 0: success without a launch, null pointers included
    assert L.moe_route(ctypes.byref(d), None, 0, 2, None, None, None, None, None, None, 0,
                       None) == 0
    assert L.moe_quantize_tokens(ctypes.byref(d), None, 0, None, None, None, None) == 0
    # null, misaligned, top_k out of range, workspace too small
    assert L.moe_route(ctypes.byref(d), ok, 4, 2, ok, ok, None, ok, ok, ok, big, None) == 1
    assert L.moe_route(ctypes.byref(d), ok, 4, 2, ok, bad, ok, ok, ok, ok, big, None) == 1
    assert L.moe_route(ctypes.byref(d), ok, 4, 9, ok, ok, ok, ok, ok, ok, big, None) == 1
    assert L.moe_route(ctypes.byref(d), ok, 4, 2, ok, ok, ok, ok, ok, ok, 64, None) == 3
    assert b"workspace" in L.moe_last_error()
    # FP8 per-token activations take no block scales; BF16 has no quantiser
    assert L.moe_quantize_tokens(ctypes.byref(d), ok, 4, ok, ok, ok, None) == 1
    assert L.moe_quantize_tokens(ctypes.byref(d), ok, 4, None, ok, None, None) == 1
    assert L.moe_quantize_tokens(ctypes.byref(d), bad, 4, ok, ok, None, None) == 1
    assert L.moe_quantize_tokens(ctypes.byref(d), ok, -1, ok, ok, None, None) == 1
    bf = _d(num_experts=8, hidden=256, inter=512, afmt="bf16").c()
    assert L.moe_quantize_tokens(ctypes.byref(bf), ok, 4, ok, ok, None, None) == 2
    mx = _d(num_experts=8, hidden=256, inter=512, afmt="mxfp8").c()
    assert L.moe_quantize_tokens(ctypes.byref(mx), ok, 4, ok, ok, None, None) == 1  # needs block scales
    assert L.moe_quantize_tokens(ctypes.byref(mx), ok, 4, ok, ok, bad, None) == 1


@pytest.mark.parametrize("afmt", ["bf16", "mxfp8", "mxfp4", "fp8"])
def test_fc2_fusion_switch_changes_the_layout(L, afmt):
    """moe_set_fc2_fused(0) makes every format store h (reserved in the
    workspace) and run the separate FC2 quantiser; with fusion (the default)
    the MX formats and BF16 reserve no h."""
    d = _d(afmt=afmt)
    T, k = 300, 8
    fused = M.workspace_layout(d, T, k)
    try:
        M.set_fc2_fused(False)
        plain = M.workspace_layout(d, T, k)
    finally:
        M.set_fc2_fused(True)
    assert plain.fc2_fused == 0
    assert plain.fc2_codes - plain.h >= T * k * 2048 * 4
    if afmt == "fp8":
        assert fused.fc2_fused == 0 and fused.total == plain.total
    else:
        assert fused.fc2_fused == 1 and fused.fc2_codes == fused.h
        assert plain.total - fused.total >= T * k * 2048 * 4
    assert M.workspace_layout(d, T, k).total == fused.total
    with pytest.raises(M.MoeError) as ei:
        _ = L.moe_set_fc2_fused(2) and M._check(L.moe_set_fc2_fused(2))
    assert ei.value.status == 1
