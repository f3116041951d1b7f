"""Pins of the oracle's block importance, top-p selection and compaction:
closed forms (checked with exact fractions), a second, independent way of
computing the block mass (per-block log-sum-exp), brute force over every
admissible block subset on small inputs, and invariants of compaction."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle import prefill as P


def _segment(rng, n, c, Hq, Hkv, D, scale=1.0):
    q = rng.standard_normal((n, Hq, D)) * scale
    keys = rng.standard_normal((c + n, Hkv, D)) * scale
    return q, keys, np.arange(c, c + n), np.arange(c + n)


# ---------------------------------------------------------------- block mass
@pytest.mark.parametrize("n,c,B,window", [(37, 0, 16, 0), (64, 0, 16, 0), (16, 0, 16, 0),
                                          (5, 9, 16, 0), (100, 64, 32, 0), (70, 30, 16, 20)])
def test_mass_zero_query_closed_form(n, c, B, window):
    """q = 0: each visible key gets 1/|vis(t)|, so m_k = sum over the last
    query block's rows of |b_k and vis(t)| / |vis(t)| (exact fractions),
    summed over heads."""
    rng = np.random.default_rng(n + c)
    Hq, Hkv, D = 2, 1, 8
    _, keys, q_pos, k_pos = _segment(rng, n, c, Hq, Hkv, D)
    q = np.zeros((n, Hq, D))
    m = oracle.block_mass(q, keys, q_pos, k_pos, c, n, B, window)
    nb = -(-n // B)
    r0 = (nb - 1) * B
    ref = [Fraction(0)] * nb
    for t in range(r0, n):
        pt = c + t
        vis = [j for j in range(c + n) if k_pos[j] <= pt and (window <= 0 or k_pos[j] > pt - window)]
        for j in vis:
            if j >= c:
                ref[(j - c) // B] += Fraction(Hq, len(vis))
    assert len(m) == nb
    for a, b in zip(m, ref):
        assert math.isclose(a, float(b), rel_tol=1e-13, abs_tol=1e-15)


@pytest.mark.parametrize("n,c,B,G", [(45, 0, 16, 1), (128, 0, 32, 2), (33, 50, 16, 4),
                                      (200, 17, 64, 2)])
def test_mass_equals_blockwise_logsumexp(n, c, B, G):
    """Second formulation: for row t and block k the mass is
    exp(LSE_{t,k} - LSE_t) with LSE over the visible keys of block k and over
    all visible keys; sum over heads and the last block's rows."""
    rng = np.random.default_rng(n * 7 + c)
    Hkv, D = 2, 16
    Hq = Hkv * G
    q, keys, q_pos, k_pos = _segment(rng, n, c, Hq, Hkv, D)
    m = oracle.block_mass(q, keys, q_pos, k_pos, c, n, B)
    nb = -(-n // B)
    r0 = (nb - 1) * B
    alt = np.zeros(nb)
    for h in range(Hq):
        z = q[:, h, :] @ keys[:, h // G, :].T / math.sqrt(D)
        for t in range(r0, n):
            zt = z[t, : c + t + 1]
            lse_all = logsumexp(zt)
            for kb in range(nb):
                lo, hi = c + kb * B, min(c + (kb + 1) * B, c + t + 1)
                if hi > lo:
                    alt[kb] += math.exp(logsumexp(z[t, lo:hi]) - lse_all)
    assert np.allclose(m, alt, rtol=1e-12, atol=1e-15)


def test_scores_normalised_and_boosted_block_dominates():
    rng = np.random.default_rng(11)
    n, c, B, Hq, Hkv, D = 96, 0, 16, 2, 1, 16
    q, keys, q_pos, k_pos = _segment(rng, n, c, Hq, Hkv, D, 0.1)
    s = oracle.normalise_scores(oracle.block_mass(q, keys, q_pos, k_pos, c, n, B))
    assert np.all(s >= 0) and math.isclose(s.sum(), 1.0, rel_tol=1e-14)
    # give the last block's queries one direction d and push block 2's keys along d
    d = rng.standard_normal(D)
    d /= np.linalg.norm(d)
    q2 = q.copy()
    q2[80:96] = d
    keys2 = keys.copy()
    keys2[32:48, 0, :] += 100.0 * d
    s2 = oracle.normalise_scores(oracle.block_mass(q2, keys2, q_pos, k_pos, c, n, B))
    assert s2[2] > 0.99


def test_mass_sums_heads():
    rng = np.random.default_rng(12)
    n, B, D = 50, 16, 8
    q, keys, q_pos, k_pos = _segment(rng, n, 0, 4, 2, D)
    m = oracle.block_mass(q, keys, q_pos, k_pos, 0, n, B)
    parts = sum(oracle.block_mass(q[:, h : h + 1], keys[:, h // 2 : h // 2 + 1], q_pos, k_pos,
                                  0, n, B) for h in range(4))
    assert np.allclose(m, parts, rtol=1e-14)


def test_mass_total_is_rows_times_heads_minus_cache_share():
    """Own-key mass of each row is 1 minus its cached-key mass; with c = 0 the
    total is exactly (#rows of the last block) * Hq."""
    rng = np.random.default_rng(13)
    n, B = 77, 16
    q, keys, q_pos, k_pos = _segment(rng, n, 0, 2, 2, 8)
    m = oracle.block_mass(q, keys, q_pos, k_pos, 0, n, B)
    assert math.isclose(m.sum(), (n - 64) * 2, rel_tol=1e-13)


# ---------------------------------------------------------------- top-p
def _fx(s32):
    return [oracle.score_fixed_point(x) for x in s32]


def _target(q, p):
    pf = oracle.p_fixed_point(p)
    return -((-pf * sum(q)) >> 22)


def _brute(s32, p):
    """All keep sets that contain {0, nb-1} and reach the target; return the
    minimum cardinality and the admissible sets of that size."""
    nb = len(s32)
    q = _fx(s32)
    tgt = _target(q, p)
    forced = {0, nb - 1}
    rest = [k for k in range(nb) if k not in forced]
    best = None
    sets = []
    for r in range(len(rest) + 1):
        for comb in itertools.combinations(rest, r):
            sset = forced | set(comb)
            if sum(q[k] for k in sset) >= tgt:
                sets.append(sset)
        if sets:
            best = r + len(forced)
            break
    return best, sets, q, tgt


@pytest.mark.parametrize("seed", range(40))
def test_topp_minimal_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 13))
    kind = seed % 4
    if kind == 0:
        raw = rng.random(nb)
    elif kind == 1:
        raw = rng.integers(1, 4, nb).astype(float)  # many ties
    elif kind == 2:
        raw = np.exp(3 * rng.standard_normal(nb))
    else:
        raw = rng.random(nb)
        raw[rng.random(nb) < 0.3] = 0.0
        raw[0] += 1e-3
    s32 = (raw / raw.sum()).astype(np.float32)
    p = float(rng.choice([0.0, 0.3, 0.5, 0.9, 0.95, 0.999, 1.0]))
    keep = oracle.topp_select(s32, p)
    if p >= 1.0:
        assert keep.all()
        return
    best, sets, q, tgt = _brute(s32, p)
    chosen = set(np.nonzero(keep)[0].tolist())
    assert {0, nb - 1} <= chosen
    if best is None:  # target unreachable: everything kept
        assert keep.all()
        return
    assert len(chosen) == best
    assert chosen in sets
    # the chosen set is a prefix of (score desc, index asc) over the free blocks
    bits = s32.view(np.uint32)
    order = sorted((k for k in range(nb) if k not in {0, nb - 1}), key=lambda k: (-int(bits[k]), k))
    extra = len(chosen) - len({0, nb - 1})
    assert set(order[:extra]) == chosen - {0, nb - 1}


def test_topp_special_values():
    s = np.array([0.1, 0.2, 0.3, 0.15, 0.25], np.float32)
    assert oracle.topp_select(s, 1.0).all()
    assert oracle.topp_select(s, 0.0).tolist() == [True, False, False, False, True]
    # p = 0.5: forced mass 0.1 + 0.25 = 0.35 < 0.5, add the largest (0.3)
    assert oracle.topp_select(s, 0.5).tolist() == [True, False, True, False, True]
    # one block, two blocks
    assert oracle.topp_select(np.array([1.0], np.float32), 0.5).tolist() == [True]
    assert oracle.topp_select(np.array([0.5, 0.5], np.float32), 0.1).tolist() == [True, True]


@pytest.mark.parametrize("nb,p", [(10, 0.9), (33, 0.5), (64, 0.95), (7, 0.01)])
def test_topp_all_equal_count(nb, p):
    s = np.full(nb, 1.0 / nb, np.float32)
    keep = oracle.topp_select(s, p)
    q = _fx(s)
    tgt = _target(q, p)
    expect = max(2 if nb > 1 else 1, -(-tgt // q[0]))
    assert keep.sum() == expect
    # ties go to lower indices
    idx = np.nonzero(keep)[0]
    assert list(idx[:-1]) == list(range(len(idx) - 1)) and idx[-1] == nb - 1


def test_topp_fixed_point_rules():
    assert oracle.p_fixed_point(0.9) == 3774874  # round(0.9 * 2^22)
    assert oracle.p_fixed_point(1.0) == 1 << 22
    assert oracle.score_fixed_point(np.float32(0.5)) == 1 << 39
    assert oracle.score_fixed_point(np.float32(2.0 ** -41)) == 0
    with pytest.raises(ValueError):
        oracle.topp_select(np.array([-0.1, 1.1], np.float32), 0.5)
    with pytest.raises(ValueError):
        oracle.topp_select(np.array([1.5, 1.5], np.float32), 0.5)


# ---------------------------------------------------------------- compaction
def test_compaction_invariants():
    rng = np.random.default_rng(21)
    lens = [37, 1, 64, 100, 16]
    flags = [True, False, True, True, False]
    B = 16
    cu = np.concatenate([[0], np.cumsum(lens)])
    keeps = [rng.random(-(-n // B)) < 0.6 for n in lens]
    T = cu[-1]
    rows = {"h": rng.standard_normal((T, 5)).astype(np.float32), "pos": np.arange(T, dtype=np.int32)}
    im, cu_out, out = oracle.compact(cu, flags, B, keeps, rows)
    assert np.all(np.diff(im) > 0)
    expect = 0
    for s, n in enumerate(lens):
        if flags[s]:
            kept = sum(min((k + 1) * B, n) - k * B for k in range(len(keeps[s])) if keeps[s][k])
        else:
            kept = n
        assert cu_out[s + 1] - cu_out[s] == kept
        expect += kept
        seg = im[cu_out[s] : cu_out[s + 1]]
        assert np.all((seg >= cu[s]) & (seg < cu[s + 1]))
        if flags[s]:
            assert all(keeps[s][(t - cu[s]) // B] for t in seg)
    assert len(im) == expect
    # scatter back reproduces the kept rows, dropped rows stay untouched
    back = np.zeros_like(rows["h"])
    back[im] = out["h"]
    assert np.array_equal(back[im], rows["h"][im])
    assert np.array_equal(out["pos"], im)


def test_compaction_identity_when_all_kept():
    lens = [5, 33, 16]
    cu = np.concatenate([[0], np.cumsum(lens)])
    keeps = [np.ones(-(-n // 16), bool) for n in lens]
    im, cu_out, _ = oracle.compact(cu, [True] * 3, 16, keeps, {})
    assert np.array_equal(im, np.arange(cu[-1])) and np.array_equal(cu_out, cu)


def test_run_call_p_one_keeps_everything():
    rng = np.random.default_rng(22)
    lens = [20, 50]
    T, Hq, Hkv, D = sum(lens), 2, 1, 8
    cu = np.concatenate([[0], np.cumsum(lens)])
    pos = np.concatenate([np.arange(n) for n in lens])
    res = oracle.run_call(segments=[(0, 0, 20, True), (1, 0, 50, True)],
                          q=rng.standard_normal((T, Hq, D)), k=rng.standard_normal((T, Hkv, D)),
                          v=rng.standard_normal((T, Hkv, D)), positions=pos, cu_seqlens=cu, Hq=Hq,
                          Hkv=Hkv, D=D, theta=0.0, window=0, block_size=16, p=1.0,
                          cache=oracle.KVCacheModel(), rows={"r": np.arange(T)})
    assert np.array_equal(res["index_map"], np.arange(T))
    for s in res["scores"]:
        assert math.isclose(float(np.sum(s.astype(np.float64))), 1.0, rel_tol=1e-6)


# ---------------------------------------------------------------- whole workloads
def test_small_chunked_fp32_chunked_calls_equal_one_pass_per_prompt():
    import workloads as W
    from oracle import driver
    wl = W.make("small_chunked_fp32")
    res = driver.run_workload(wl, threads=1)
    # gather each prompt's outputs across calls, in position order
    got = {}
    for call, r in zip(wl.calls, res):
        for i, s in enumerate(call.segments):
            a, b = call.cu_seqlens[i], call.cu_seqlens[i + 1]
            got.setdefault(s.prompt, []).append(r["out"][a:b])
    for pid, L in wl.prompt_len.items():
        q = np.concatenate([W.to_f64(c.q[c.cu_seqlens[i]:c.cu_seqlens[i + 1]], "f32")
                            for c in wl.calls for i, s in enumerate(c.segments) if s.prompt == pid])
        k = np.concatenate([W.to_f64(c.k[c.cu_seqlens[i]:c.cu_seqlens[i + 1]], "f32")
                            for c in wl.calls for i, s in enumerate(c.segments) if s.prompt == pid])
        v = np.concatenate([W.to_f64(c.v[c.cu_seqlens[i]:c.cu_seqlens[i + 1]], "f32")
                            for c in wl.calls for i, s in enumerate(c.segments) if s.prompt == pid])
        one = oracle.run_call(segments=[(0, 0, L, False)], q=q, k=k, v=v, positions=np.arange(L),
                              cu_seqlens=[0, L], Hq=2, Hkv=2, D=64, theta=0.0, window=0,
                              block_size=16, p=0.9, cache=oracle.KVCacheModel(), score=False,
                              select=False)
        assert np.max(np.abs(np.concatenate(got[pid]) - one["out"])) < 1e-12
    # every scored segment: scores sum to one, first/last kept, compaction consistent
    for call, r in zip(wl.calls, res):
        for i, s in enumerate(call.segments):
            sc = r["scores"][i]
            assert abs(float(sc.astype(np.float64).sum()) - 1.0) < 1e-5
            assert r["keep"][i][0] and r["keep"][i][-1]
        assert r["cu_seqlens_out"][-1] == len(r["index_map"])
        assert np.array_equal(r["rows_out"]["positions"], call.positions[r["index_map"]])


def test_layer2_runs_on_compacted_tokens():
    import workloads as W
    from oracle import driver
    wl = W.custom(lengths=[70, 33], Hq=2, Hkv=1, D=16, block_size=16, p=0.5, theta=10000.0,
                  layer2_window=20, seed=4)
    r = driver.run_workload(wl, threads=1)[0]
    l2 = r["layer2"]
    im = r["index_map"]
    assert l2["out"].shape[0] == len(im)
    # the first kept token of each segment sees only itself
    cu = r["cu_seqlens_out"]
    v2 = W.to_f64(wl.calls[0].extra["v2"], "f32")
    for i in range(2):
        t0 = cu[i]
        assert np.allclose(l2["out"][t0, 0], v2[im[t0], 0], atol=1e-14)


def _prompt(rng, n, Hq=4, Hkv=2, D=32):
    return (rng.standard_normal((n, Hq, D)), rng.standard_normal((n, Hkv, D)),
            rng.standard_normal((n, Hkv, D)))


def test_whole_prompt_scores_of_final_chunk_equal_one_pass():
    """Chunked prefill equals one pass (glossary, How chunked prefill
    works), so the final chunk's whole-prompt block masses, selection and
    kept tokens (cached ones listed by position, own ones compacted) equal
    those of the whole prompt scored in one call."""
    rng = np.random.default_rng(11)
    n_total, chunk, B, Hq, Hkv, D = 600, 256, 64, 4, 2, 32
    q, k, v = _prompt(rng, n_total, Hq, Hkv, D)
    pos = np.arange(n_total)
    kw = dict(Hq=Hq, Hkv=Hkv, D=D, theta=500000.0, window=0, block_size=B, p=0.6)
    one = oracle.run_call(segments=[(0, 0, n_total, True)], q=q, k=k, v=v, positions=pos,
                          cu_seqlens=[0, n_total], cache=oracle.KVCacheModel(), **kw)
    cache = oracle.KVCacheModel()
    for c0 in range(0, n_total, chunk):
        n = min(chunk, n_total - c0)
        last = c0 + n == n_total
        res = oracle.run_call(segments=[(0, c0, n, last)], q=q[c0:c0 + n], k=k[c0:c0 + n],
                              v=v[c0:c0 + n], positions=pos[c0:c0 + n], cu_seqlens=[0, n],
                              cache=cache, scope="prompt", **kw)
    assert len(res["mass"][0]) == len(one["mass"][0]) == 10
    assert np.allclose(res["mass"][0], one["mass"][0], rtol=1e-12, atol=0)
    assert np.array_equal(res["keep"][0], one["keep"][0])
    assert 0 < res["keep"][0].sum() < 10
    kept = np.concatenate([res["kept_cache_positions"][0], c0 + res["index_map"]])
    assert np.array_equal(kept, one["index_map"])


def test_whole_prompt_scope_without_cache_equals_segment_scope():
    rng = np.random.default_rng(12)
    q, k, v = _prompt(rng, 150)
    kw = dict(segments=[(0, 0, 150, True)], q=q, k=k, v=v, positions=np.arange(150),
              cu_seqlens=[0, 150], Hq=4, Hkv=2, D=32, theta=0.0, window=0, block_size=32, p=0.7)
    a = oracle.run_call(cache=oracle.KVCacheModel(), **kw)
    b = oracle.run_call(cache=oracle.KVCacheModel(), scope="prompt", **kw)
    assert np.array_equal(a["mass"][0], b["mass"][0])
    assert np.array_equal(a["index_map"], b["index_map"])
    assert len(b["kept_cache_positions"][0]) == 0


def test_whole_prompt_scope_needs_block_aligned_cache():
    rng = np.random.default_rng(13)
    q, k, v = _prompt(rng, 40)
    cache = oracle.KVCacheModel()
    kw = dict(Hq=4, Hkv=2, D=32, theta=0.0, window=0, block_size=16, p=0.9)
    oracle.run_call(segments=[(0, 0, 20, False)], q=q[:20], k=k[:20], v=v[:20],
                    positions=np.arange(20), cu_seqlens=[0, 20], cache=cache, **kw)
    with pytest.raises(ValueError):
        oracle.run_call(segments=[(0, 20, 20, True)], q=q[20:], k=k[20:], v=v[20:],
                        positions=np.arange(20, 40), cu_seqlens=[0, 20], cache=cache,
                        scope="prompt", **kw)
