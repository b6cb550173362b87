"""CPU oracle of the fused mixed-precision MoE layer.

TEST INFRASTRUCTURE ONLY.  A plain, slow, float64 NumPy implementation of what
the GPU path computes, written from the layer's definition.  Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it; the GPU
library and its Python binding never do, and this package imports nothing from
them.  It shares no code with the GPU path: the only common module is the
seeded input generator (moe_inputs), which holds no arithmetic of the layer.

Pins (tests marked "not gpu"): OCP code tables and exhaustive/brute-force
encoder checks, quantiser invariants, a brute-force router, exact rational
GEMMs on tiny shapes, dense-equivalence and single-expert reductions.  The
pages print no worked example, vector or result for this layer, so no value
of the pages pins the whole-layer output ("parity unpinned" against the
pages themselves; pinned against definitions and invariants).
"""
from . import formats, quant, layer  # noqa: F401
from .layer import route, expand, forward, finalize, quantize_expert, ExpertWeights  # noqa: F401
