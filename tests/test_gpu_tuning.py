"""Tile-configuration selection on the GPU: every configuration of every format
combination matches the oracle (forced through the tuning table, on skewed
routing), the configurations give identical bits (each K step is accumulated
in the same order by the same matrix instruction whatever the tile shape),
and the autotuner validates, times and stores its choice.

The FC2 input that GEMM1 writes itself (MX formats, BF16) is checked bit for
bit: with the fusion switched off GEMM1 stores h and the separate quantiser
runs, whose bytes must equal the oracle's quantiser applied to that h
(compare_all), and the fused run's bytes must equal the separate ones."""
import numpy as np
import pytest

import moe_inputs as MI
from tests.harness import Problem, compare_all

pytestmark = pytest.mark.gpu

FORMATS = [("mxfp4", "fp8"), ("mxfp4", "bf16"), ("int4", "fp8"), ("mxfp4", "mxfp8"),
           ("mxfp4", "mxfp4")]


@pytest.mark.parametrize("wf,af", FORMATS, ids=[f"{w}x{a}" for w, a in FORMATS])
def test_every_tile_config_matches_oracle(wf, af):
    import mixed_precision_moe_topk_amd as M

    # 120 rows per expert on average, skewed by a router bias: full, ragged
    # and (for 16-row tiles) many tiles per expert; N tails in both GEMMs
    wl = MI.small_workload(300, 5, 2, 256, 640, wf, af, 41, 2.0)
    p = Problem(wl)
    r = p.run_oracle()
    runs = {}
    M.tune_clear()
    try:
        for c in range(M.NUM_GEMM_CFG):
            M.tune_set(p.dims, wl.tokens, wl.top_k, c)
            g = p.run_gpu()
            assert g["gemm_cfg"] == c
            rel, mx = compare_all(g, r, wl)
            print(f"{wf}x{af} cfg {c} tile_m={g['tile_m']} tiles={g['num_tiles']} rel-L2={rel:.2e}")
            runs[c] = g
            if af in ("mxfp8", "mxfp4", "bf16"):
                M.set_fc2_fused(False)
                try:
                    gu = p.run_gpu()
                finally:
                    M.set_fc2_fused(True)
                assert not gu["fc2_fused"] and gu["h"] is not None
                compare_all(gu, r, wl)  # separate quantiser == oracle's quantiser of this h
                fkeys = ["fc2_codes", "y2", "out"] + (["fc2_block_scales"] if af != "bf16" else [])
                for key in fkeys:
                    assert np.array_equal(g[key].view(np.uint8), gu[key].view(np.uint8)), (c, key)
    finally:
        M.tune_clear()
        M.set_fc2_fused(True)
    keys = ["fc2_codes", "y2", "out"]
    if af in ("mxfp8", "mxfp4", "bf16"):
        # every configuration writes the FC2 input from GEMM1 (no h)
        assert all(runs[c]["fc2_fused"] for c in range(M.NUM_GEMM_CFG))
        if af != "bf16":
            keys.append("fc2_block_scales")
    else:
        keys.append("h")
    for c in range(1, M.NUM_GEMM_CFG):
        for key in keys:
            assert np.array_equal(runs[c][key].view(np.uint8), runs[0][key].view(np.uint8)), (c, key)


def test_autotune_validates_times_and_stores():
    import mixed_precision_moe_topk_amd as M

    wl = MI.small_workload(300, 5, 2, 256, 384, "mxfp4", "fp8", 42, 2.0)
    p = Problem(wl, experts_for_oracle=[])
    M.tune_clear()
    try:
        default = p.run_gpu()
        chosen, ms = M.autotune(p.dims, p.h_dev, p.l_dev, p.weights, p.scales, wl.top_k, iters=3)
        print(f"autotune: chosen {chosen}, ms per call {ms}")
        assert all(m > 0 for m in ms), ms  # every configuration matched the reference
        assert chosen == int(np.argmin(ms))
        assert M.workspace_layout(p.dims, wl.tokens, wl.top_k).gemm_cfg == chosen
        tuned = p.run_gpu()
        assert tuned["gemm_cfg"] == chosen
        assert np.array_equal(tuned["out"], default["out"])
    finally:
        M.tune_clear()
