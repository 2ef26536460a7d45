"""The CPU oracle fanned out over worker processes, for the full-size parity tests.

Each worker imports only the oracle and the seeded generators (no torch, no GPU)
and evaluates whole layers or single experts exactly as the oracle defines them;
the parent assembles the results. Workers are spawned (not forked) so that they
inherit nothing from a process that has initialised the GPU.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

from oracle import moe_ref as R
from synth import gen


def _init_worker(threads: int) -> None:
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(threads)
    except ImportError:
        pass


def pool(workers: int | None = None) -> cf.ProcessPoolExecutor:
    n = workers or max(1, min(8, len(os.sched_getaffinity(0)) // 2))
    return cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=_init_worker,
                                  initargs=(2,))


def _expert(w: gen.Workload, layer: int, e: int) -> R.Expert:
    return R.Expert(gen.expert_tensors(w.seed, layer, e, w.H, w.I), w.H, w.I)


def layer_ref(w: gen.Workload, layer: int, x_bits: np.ndarray, logits=None):
    """Oracle of one layer (router GEMV when logits is None): (y, ids, w, l)."""
    wr = gen.router_weight(w.seed, layer, w.E, w.H) if logits is None else None
    cache = {}

    def experts(e):
        if e not in cache:
            cache[e] = _expert(w, layer, e)
        return cache[e]

    shared = _expert(w, layer, gen.SHARED_EXPERT) if w.shared else None
    return R.moe_layer(x_bits, experts, w.K, logits=logits, w_router=wr, shared=shared)


def expert_rows(w: gen.Workload, layer: int, e: int, x_bits_rows: np.ndarray) -> np.ndarray:
    """The oracle's FFN of expert e (gen.SHARED_EXPERT for the shared one) on the given rows."""
    return _expert(w, layer, e)(R.bf16_bits_to_f64(x_bits_rows))


def expert_major_layer(ex: cf.Executor, w: gen.Workload, layer: int, x_bits: np.ndarray, logits: np.ndarray):
    """moe_layer_expert_major with the per-expert products spread over the pool:
    (y, ids, w) from the oracle's routing, per-pair FFN outputs and rank-ordered combine."""
    ids, wts = R.route(logits, w.K)
    T = ids.shape[0]
    o = np.empty((T, w.K, w.H), dtype=np.float64)
    futs = {}
    for e in np.unique(ids):
        t_idx, k_idx = np.nonzero(ids == e)
        futs[ex.submit(expert_rows, w, layer, int(e), x_bits[t_idx])] = (t_idx, k_idx)
    shared_fut = ex.submit(expert_rows, w, layer, gen.SHARED_EXPERT, x_bits) if w.shared else None
    for f in cf.as_completed(futs):
        t_idx, k_idx = futs[f]
        o[t_idx, k_idx] = f.result()
    y = R.combine(o, wts, shared_fut.result() if shared_fut is not None else None)
    return y, ids, wts
