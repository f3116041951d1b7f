"""Runs the oracle over a generated workload (test infrastructure only).

Feeds each operator call of a ``workloads.Workload`` to ``oracle.run_call``
with the exact float64 values of the stored inputs, keeps the oracle's own KV
record between chunked calls, and for a workload with a second,
sliding-window layer runs that layer on the compacted tokens at their
original positions (the review's propagation step: dropped tokens skip all
later sublayers, sliding-window attention included).
"""
from __future__ import annotations

import numpy as np

from workloads import to_f64

from .prefill import KVCacheModel, run_call


def segments_of(call):
    return [(s.prompt, s.ctx, s.n, bool(s.flagged)) for s in call.segments]


def row_tensors(call):
    rows = {"hidden": call.hidden, "positions": call.positions, "slot_mapping": call.slot_mapping}
    rows.update(call.extra)
    return rows


def initial_cache(wl) -> KVCacheModel:
    cache = KVCacheModel()
    for pid, (K, V) in wl.given_cache.items():
        cache.put(pid, to_f64(K, wl.dtype), to_f64(V, wl.dtype))
    return cache


def run_workload(wl, threads=None, cache=None, layer2=True):
    """Oracle results for every call of ``wl`` (a list of dicts)."""
    cache = cache if cache is not None else initial_cache(wl)
    results = []
    for call in wl.calls:
        res = run_call(segments=segments_of(call), q=to_f64(call.q, wl.dtype),
                       k=to_f64(call.k, wl.dtype), v=to_f64(call.v, wl.dtype),
                       positions=call.positions, cu_seqlens=call.cu_seqlens, Hq=wl.Hq, Hkv=wl.Hkv,
                       D=wl.D, theta=wl.theta, window=wl.window, block_size=wl.block_size, p=wl.p,
                       cache=cache, rows=row_tensors(call), threads=threads)
        if layer2 and wl.layer2 is not None:
            res["layer2"] = run_layer2(wl, call, res, threads=threads)
        results.append(res)
    return results


def run_layer2(wl, call, res, threads=None):
    """Sliding-window layer over the compacted tokens (no scoring)."""
    ro = res["rows_out"]
    cu = res["cu_seqlens_out"]
    segs = [(s.prompt, 0, int(cu[i + 1] - cu[i]), False) for i, s in enumerate(call.segments)]
    return run_call(segments=segs, q=to_f64(ro["q2"], wl.dtype), k=to_f64(ro["k2"], wl.dtype),
                    v=to_f64(ro["v2"], wl.dtype), positions=ro["positions"], cu_seqlens=cu,
                    Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, theta=wl.layer2["theta"],
                    window=wl.layer2["window"], block_size=wl.block_size, p=wl.p,
                    cache=KVCacheModel(), score=False, select=False, threads=threads)
