"""Pins of the oracle's sampled-evaluation glue (``oracle/driver.py``).

The full-size GPU tests take their expected values from
``driver.sampled_segment`` (one segment, selected rows), fed with the cached
keys that ``driver.prompt_kv_before`` rebuilds from earlier calls, and the
second layer's arguments.  These tests check that glue against facts the
pages fix and against the whole-call oracle:

* chunked prefill equals one pass (glossary "Chunked Prefill", "How chunked
  prefill works"): a chunk's rows, evaluated with the rebuilt cache, equal
  the same rows of a one-pass run over the whole prompt;
* packed equals unpacked (Prepacking summary, "Technical framework" and
  "Key design"): a packed segment's rows equal that prompt run alone;
* row for row agreement with ``run_workload`` (outputs within 1e-12,
  float32 scores bit-equal) on small workloads of each shape: the fp32
  chunked one (with and without rotary), a chunked long prompt with segment
  and whole-prompt scoring, a continuous-batching step with decodes over a
  given cache, and the sliding-window second layer on the kept tokens;
* the second layer's window reaches the evaluation: a window narrower than
  the segments changes the result, and both the glue and ``run_layer2``
  agree with torch's scaled_dot_product_attention in float64 under the
  windowed mask on the compacted tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import driver

TOL = 1e-12


def _cached(wl, ci, seg):
    if seg.ctx == 0:
        return None
    if seg.prompt in wl.given_cache:
        K, V = wl.given_cache[seg.prompt]
        return W.to_f64(K, wl.dtype)[: seg.ctx], W.to_f64(V, wl.dtype)[: seg.ctx]
    kk, vv, pp = driver.prompt_kv_before(wl, ci, seg.prompt)
    return oracle.apply_rope(kk, pp, wl.theta), vv


def _agree_with_run_workload(wl, scope="segment", rows_of=None):
    res = driver.run_workload(wl, threads=4, scope=scope, layer2=False)
    n_checked = 0
    for ci, call in enumerate(wl.calls):
        cu = call.cu_seqlens
        for si, s in enumerate(call.segments):
            rows = rows_of(s.n) if rows_of else list(range(s.n))
            r = driver.sampled_segment(wl, call, si, rows, cached=_cached(wl, ci, s),
                                       score=s.flagged, threads=4, scope=scope)
            want = res[ci]["out"][cu[si] + np.asarray(rows)]
            assert np.abs(r["out"] - want).max() <= TOL, (ci, si)
            assert np.abs(r["lse"] - res[ci]["lse"][cu[si] + np.asarray(rows)]).max() <= TOL
            if s.flagged:
                assert r["scores"].dtype == np.float32
                assert np.array_equal(r["scores"], res[ci]["scores"][si]), (ci, si)
            n_checked += 1
    return res, n_checked


@pytest.mark.parametrize("theta", [0.0, 500000.0])
def test_sampled_segment_equals_run_workload_small_chunked_fp32(theta):
    wl = W.make("small_chunked_fp32")
    wl.theta = theta
    _, n = _agree_with_run_workload(wl)
    assert n == sum(len(c.segments) for c in wl.calls) == 8


def _small_long_prompt():
    # the chunked 128K workload's shape at 1/128 of its length: 32/8 heads,
    # block 128, chunks of 256 over a paged cache
    return W.config_chunked_128k(total=1024, chunk=256)


@pytest.mark.parametrize("scope", ["segment", "prompt"])
def test_sampled_segment_equals_run_workload_chunked_long_prompt(scope):
    wl = _small_long_prompt()
    assert len(wl.calls) == 4 and wl.calls[3].segments[0].ctx == 768
    _agree_with_run_workload(wl, scope=scope, rows_of=lambda n: sorted({0, 1, 100, n - 2, n - 1}))


def test_sampled_segment_chunk_equals_one_pass():
    """A chunk evaluated over the rebuilt cache equals the same rows of the
    whole prompt computed in one pass (the glossary's chunked-prefill
    fact), for every chunk."""
    wl = _small_long_prompt()
    q = np.concatenate([W.to_f64(c.q, wl.dtype) for c in wl.calls])
    k = np.concatenate([W.to_f64(c.k, wl.dtype) for c in wl.calls])
    v = np.concatenate([W.to_f64(c.v, wl.dtype) for c in wl.calls])
    pos = np.concatenate([c.positions for c in wl.calls]).astype(np.int64)
    one = oracle.run_call(segments=[(0, 0, 1024, True)], q=q, k=k, v=v, positions=pos,
                          cu_seqlens=np.array([0, 1024]), Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                          theta=wl.theta, window=0, block_size=wl.block_size, p=wl.p,
                          cache=oracle.KVCacheModel(), threads=4, select=False)
    for ci, call in enumerate(wl.calls):
        s = call.segments[0]
        rows = [0, 17, 128, s.n - 1]
        r = driver.sampled_segment(wl, call, 0, rows, cached=_cached(wl, ci, s), threads=4)
        want = one["out"][s.ctx + np.asarray(rows)]
        assert np.abs(r["out"] - want).max() <= 1e-12, ci
    # whole-prompt scores of the final chunk equal the one-pass scores
    last = wl.calls[-1]
    r = driver.sampled_segment(wl, last, 0, [0], cached=_cached(wl, 3, last.segments[0]),
                               score=True, scope="prompt", threads=4)
    assert np.abs(r["scores"].astype(np.float64) - one["scores"][0].astype(np.float64)).max() <= 1e-7


def test_prompt_kv_before_rebuilds_the_cache():
    """prompt_kv_before returns exactly the raw k, v and positions of the
    prompt's earlier chunks, in position order, and nothing for chunk 0."""
    wl = _small_long_prompt()
    assert driver.prompt_kv_before(wl, 0, 0) is None
    kk, vv, pp = driver.prompt_kv_before(wl, 3, 0)
    assert np.array_equal(pp, np.arange(768))
    assert np.array_equal(kk, np.concatenate([W.to_f64(c.k, wl.dtype) for c in wl.calls[:3]]))
    assert np.array_equal(vv, np.concatenate([W.to_f64(c.v, wl.dtype) for c in wl.calls[:3]]))


def test_sampled_segment_packed_equals_unpacked():
    """A packed segment equals its prompt run alone (Prepacking)."""
    wl = W.custom(lengths=[70, 130, 45], Hq=8, Hkv=2, D=64, dtype="bf16", block_size=16, p=0.9,
                  theta=500000.0, seed=5)
    call = wl.calls[0]
    cu = call.cu_seqlens
    for si, s in enumerate(call.segments):
        a, b = int(cu[si]), int(cu[si + 1])
        alone = oracle.run_call(segments=[(0, 0, s.n, True)], q=W.to_f64(call.q[a:b], "bf16"),
                                k=W.to_f64(call.k[a:b], "bf16"), v=W.to_f64(call.v[a:b], "bf16"),
                                positions=call.positions[a:b], cu_seqlens=np.array([0, s.n]),
                                Hq=8, Hkv=2, D=64, theta=wl.theta, window=0, block_size=16,
                                p=0.9, cache=oracle.KVCacheModel(), select=False)
        r = driver.sampled_segment(wl, call, si, list(range(s.n)), score=True)
        assert np.abs(r["out"] - alone["out"]).max() <= 1e-12
        assert np.array_equal(r["scores"], alone["scores"][0])


def test_sampled_segment_equals_run_workload_mixed_decode_prefill():
    """Decodes over a given cache (taken as already rotated) plus FCFS
    prefill chunks, the continuous-batching step's shape at small size."""
    wl = W.config_mixed_decode_prefill(n_decode=6, budget=6 + 300, ctx_range=(20, 90),
                                       wait_range=(100, 200), n_wait=3, device_cache=False)
    call = wl.calls[0]
    assert sum(1 for s in call.segments if not s.flagged) == 6
    assert sum(s.n for s in call.segments) == 306
    _agree_with_run_workload(wl)


def _small_swa_workload(window):
    wl = W.config_swa_after_selection(n_prompts=3, len_range=(150, 300))
    wl.layer2 = dict(wl.layer2, window=window)
    wl.p = 0.6  # drop blocks inside the segments at this small size
    return wl


def _sdpa_layer2(wl, ro, cu2, si):
    """torch scaled_dot_product_attention, float64, explicit windowed causal
    mask over the kept tokens' original positions."""
    a, b = int(cu2[si]), int(cu2[si + 1])
    pos = np.asarray(ro["positions"][a:b], np.int64)
    q = oracle.apply_rope(W.to_f64(ro["q2"][a:b], "bf16"), pos, wl.layer2["theta"])
    k = oracle.apply_rope(W.to_f64(ro["k2"][a:b], "bf16"), pos, wl.layer2["theta"])
    v = W.to_f64(ro["v2"][a:b], "bf16")
    G = wl.Hq // wl.Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)
    pq, pk = pos[:, None], pos[None, :]
    W_ = wl.layer2["window"]
    mask = pk <= pq
    if W_ > 0:
        mask &= pk > pq - W_
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt,
                                                         attn_mask=torch.from_numpy(mask))
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("window", [4096, 24])
def test_sampled_segment_layer2_equals_run_layer2_and_sdpa(window):
    wl = _small_swa_workload(window)
    call = wl.calls[0]
    res = driver.run_workload(wl, threads=4)[0]
    ro, cu2 = res["rows_out"], res["cu_seqlens_out"]
    l2 = res["layer2"]
    for si in range(len(call.segments)):
        n2 = int(cu2[si + 1] - cu2[si])
        rows = list(range(n2))
        r = driver.sampled_segment(wl, call, si, rows, theta=wl.layer2["theta"],
                                   window=wl.layer2["window"], q=ro["q2"], k=ro["k2"],
                                   v=ro["v2"], positions=ro["positions"], cu=cu2, threads=4)
        want = l2["out"][cu2[si]:cu2[si + 1]]
        assert np.abs(r["out"] - want).max() <= TOL
        ref = _sdpa_layer2(wl, ro, cu2, si)
        assert np.abs(r["out"] - ref).max() <= 1e-10
    # positions are gapped after selection (dropped blocks leave holes)
    gaps = [np.any(np.diff(ro["positions"][cu2[i]:cu2[i + 1]]) > 1) for i in range(len(cu2) - 1)]
    assert any(gaps)


def test_layer2_window_changes_the_result():
    """A window narrower than the segments changes layer 2's output, so a
    glue that dropped the window would be caught by the SDPA check above."""
    wide = _small_swa_workload(4096)
    narrow = _small_swa_workload(24)
    rw = driver.run_workload(wide, threads=4)[0]["layer2"]["out"]
    rn = driver.run_workload(narrow, threads=4)[0]["layer2"]["out"]
    assert rw.shape == rn.shape
    assert np.abs(rw - rn).max() > 1e-2
    # a window of 4096 is wider than every segment here: equals full causal
    full = _small_swa_workload(0)
    rf = driver.run_workload(full, threads=4)[0]["layer2"]["out"]
    assert np.abs(rw - rf).max() <= 1e-12
