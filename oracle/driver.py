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


def run_workload(wl, threads=None, cache=None, layer2=True, scope="segment"):
    """Oracle results for every call of ``wl`` (a list of dicts); ``scope``
    "prompt" scores the flagged segments over their whole prompt."""
    cache = cache if cache is not None else initial_cache(wl)
    results = []
    for call in wl.calls:
        res = run_call(segments=segments_of(call), q=to_f64(call.q, wl.dtype),
                       k=to_f64(call.k, wl.dtype), v=to_f64(call.v, wl.dtype),
                       positions=call.positions, cu_seqlens=call.cu_seqlens, Hq=wl.Hq, Hkv=wl.Hkv,
                       D=wl.D, theta=wl.theta, window=wl.window, block_size=wl.block_size, p=wl.p,
                       cache=cache, rows=row_tensors(call), threads=threads, scope=scope)
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


# --------------------------------------------------------------------------
# sampled evaluation for full-size workloads
# --------------------------------------------------------------------------
def prompt_kv_before(wl, call_index, pid):
    """Raw k, v and positions of prompt ``pid`` from the calls before
    ``call_index`` (the tokens its cache holds), float64."""
    ks, vs, ps = [], [], []
    for call in wl.calls[:call_index]:
        for i, s in enumerate(call.segments):
            if s.prompt == pid:
                a, b = int(call.cu_seqlens[i]), int(call.cu_seqlens[i + 1])
                ks.append(to_f64(call.k[a:b], wl.dtype))
                vs.append(to_f64(call.v[a:b], wl.dtype))
                ps.append(np.asarray(call.positions[a:b], np.int64))
    if not ks:
        return None
    return np.concatenate(ks), np.concatenate(vs), np.concatenate(ps)


def sampled_segment(wl, call, si, rows, *, cached=None, theta=None, window=None,
                    score=False, q=None, k=None, v=None, positions=None, cu=None, threads=None,
                    scope="segment"):
    """Oracle outputs of segment ``si`` for local query rows ``rows`` and,
    with ``score``, the segment's float32 block scores.

    ``cached``: (K, V) float64 already rotated for positions 0..c-1, or None.
    q/k/v/positions/cu default to the call's own arrays (layer 2 passes the
    compacted ones)."""
    from .prefill import apply_rope, attention, block_mass, normalise_scores

    theta = wl.theta if theta is None else theta
    window = wl.window if window is None else window
    cu = call.cu_seqlens if cu is None else cu
    a, b = int(cu[si]), int(cu[si + 1])
    n = b - a
    qa = to_f64((call.q if q is None else q)[a:b], wl.dtype)
    ka = to_f64((call.k if k is None else k)[a:b], wl.dtype)
    va = to_f64((call.v if v is None else v)[a:b], wl.dtype)
    pos = np.asarray((call.positions if positions is None else positions)[a:b], np.int64)
    k_rot = apply_rope(ka, pos, theta)
    c = 0 if cached is None else cached[0].shape[0]
    if c:
        keys = np.concatenate([cached[0], k_rot])
        vals = np.concatenate([cached[1], va])
    else:
        keys, vals = k_rot, va
    k_pos = np.concatenate([np.arange(c, dtype=np.int64), pos])
    rows = np.asarray(rows, np.int64)
    q_rot = apply_rope(qa[rows], pos[rows], theta)
    out, lse = attention(q_rot, keys, vals, pos[rows], k_pos, window, threads=threads)
    res = {"rows": rows, "out": out, "lse": lse}
    if score:
        q_all = apply_rope(qa, pos, theta)
        m = block_mass(q_all, keys, pos, k_pos, c, n, wl.block_size, window, scope=scope)
        res["scores"] = normalise_scores(m).astype(np.float32)
    return res
