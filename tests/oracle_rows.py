"""Oracle rows for the full-size GPU tests, one expert per worker process.

A worker draws one expert's seeded float32 master weights (the same draw
the GPU's weights were packed from), quantises them with the oracle and
runs the oracle's pass of that one expert over the given tokens.  Only the
oracle and the seeded input generators are imported here: nothing touches
the GPU, so the workers can be spawned next to a process that holds it."""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

import moe_inputs as MI
import oracle as O


def expert_rows(job):
    """job = (workload name, expert, bf16 hidden rows [n, H], float32 logits
    [n, E]) -> (expert, h rows, y2 rows) of the n tokens' rows for that
    expert, in token order (each token must route to the expert)."""
    name, e, hidden, logits = job
    wl = MI.WORKLOADS[name]
    w1, w2 = MI.expert_weights(wl.seed, e, wl.hidden, wl.inter)
    ow = O.quantize_expert(w1, w2, wl.wfmt)
    del w1, w2
    sub = O.forward(hidden, logits, wl.top_k, lambda x: ow, wl.wfmt, wl.afmt,
                    only_experts={e})
    ti, tj = np.nonzero(sub["ids"] == e)
    assert np.array_equal(ti, np.arange(len(hidden))), "each token must pick the expert once"
    rows = sub["slot_row"][ti, tj]
    return e, sub["h"][rows], sub["y2"][rows]


def expert_rows_many(jobs, workers=None):
    """Runs `expert_rows` over the jobs in spawned worker processes (at most
    16, the host share of one GPU) and yields the results in job order."""
    workers = workers or max(1, min(16, os.cpu_count() or 1, len(jobs)))
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as pool:
        yield from pool.map(expert_rows, jobs, chunksize=1)
