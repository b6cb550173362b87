"""Host -> device weight preparation in expert chunks.

The float32 masters of a 256-expert DeepSeek-V3-shaped layer take 45 GB, so
they are streamed: each chunk of experts is copied to a pinned host buffer,
uploaded, and quantised on the device by moe_prepare_weights into the packed
layout; only the packed codes and scales stay resident.
"""
from __future__ import annotations

import numpy as np

from . import LayerDims, prepare_weights, weights_query


def prepare_from_host(d: LayerDims, experts_iter, chunk: int = 8, device="cuda", stream=None):
    """experts_iter yields (expert, W1 float32 [2I, H], W2 float32 [H, I]) for
    experts 0, 1, ..., E-1 in order.  Returns (weights, scales) uint8 device
    tensors holding every expert."""
    import torch

    wb, sb = weights_query(d)
    weights = torch.empty(wb, dtype=torch.uint8, device=device)
    scales = torch.empty(sb, dtype=torch.uint8, device=device)
    n1 = (2 * d.inter, d.hidden)
    n2 = (d.hidden, d.inter)
    h1 = torch.empty((chunk, *n1), dtype=torch.float32, pin_memory=True)
    h2 = torch.empty((chunk, *n2), dtype=torch.float32, pin_memory=True)
    g1 = torch.empty((chunk, *n1), dtype=torch.float32, device=device)
    g2 = torch.empty((chunk, *n2), dtype=torch.float32, device=device)
    st = stream if stream is not None else torch.cuda.current_stream()
    pending = []
    expect = 0

    def flush():
        nonlocal pending
        if not pending:
            return
        n = len(pending)
        first = pending[0][0]
        st.synchronize()  # staging buffers are free again
        for i, (_, w1, w2) in enumerate(pending):
            h1[i].numpy()[...] = w1
            h2[i].numpy()[...] = w2
        with torch.cuda.stream(st):
            g1[:n].copy_(h1[:n], non_blocking=True)
            g2[:n].copy_(h2[:n], non_blocking=True)
            prepare_weights(d, g1[:n], g2[:n], first, weights, scales, stream=st)
        pending = []

    for e, w1, w2 in experts_iter:
        if e != expect:
            raise ValueError(f"experts must come in order: got {e}, expected {expect}")
        expect += 1
        pending.append((e, np.asarray(w1, dtype=np.float32), np.asarray(w2, dtype=np.float32)))
        if len(pending) == chunk:
            flush()
    flush()
    if expect != d.num_experts:
        raise ValueError(f"got {expect} experts, layer has {d.num_experts}")
    st.synchronize()
    return weights, scales
