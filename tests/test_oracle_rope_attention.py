"""Pins of the oracle's rotary embedding and attention against closed forms,
a library routine (torch's scaled_dot_product_attention on the CPU in
float64), the chunked-prefill example of the glossary page, and the packing
property of the Prepacking summary."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import prefill as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- rotary
def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 8))
    y = oracle.apply_rope(x, np.zeros(5, np.int64), 10000.0)
    assert np.array_equal(x, y)


def test_rope_d2_closed_form():
    # D = 2: one pair (0, 1), omega_0 = 1, angle = pos.
    x = np.array([[[1.0, 0.0]], [[0.0, 1.0]], [[2.0, -3.0]]])
    pos = np.array([1, 1, 5])
    y = oracle.apply_rope(x, pos, 123.0)
    c1, s1 = math.cos(1.0), math.sin(1.0)
    assert np.allclose(y[0, 0], [c1, s1], atol=1e-15)
    assert np.allclose(y[1, 0], [-s1, c1], atol=1e-15)
    c5, s5 = math.cos(5.0), math.sin(5.0)
    assert np.allclose(y[2, 0], [2 * c5 + 3 * s5, -3 * c5 + 2 * s5], atol=1e-14)


def test_rope_rotate_half_pairing_and_frequencies():
    # D = 4, theta = 100: omega = [1, 0.1]; pairs are (0, 2) and (1, 3).
    om = oracle.rope_frequencies(4, 100.0)
    assert np.allclose(om, [1.0, 0.1], rtol=1e-15)
    x = np.zeros((1, 1, 4))
    x[0, 0, 1] = 1.0
    y = oracle.apply_rope(x, np.array([10]), 100.0)[0, 0]
    assert np.allclose(y, [0.0, math.cos(1.0), 0.0, math.sin(1.0)], atol=1e-15)
    om = oracle.rope_frequencies(128, 500000.0)
    assert om[0] == 1.0
    assert math.isclose(om[1], math.exp(-math.log(500000.0) / 64), rel_tol=1e-14)
    assert math.isclose(om[63], 500000.0 ** (-126 / 128), rel_tol=1e-14)


def test_rope_preserves_norm_and_is_relative():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    for a, b, d in [(7, 3, 1000), (0, 0, 131000), (40000, 12, 5)]:
        qa = oracle.apply_rope(q, np.array([a]), 500000.0)
        kb = oracle.apply_rope(k, np.array([b]), 500000.0)
        qd = oracle.apply_rope(q, np.array([a + d]), 500000.0)
        kd = oracle.apply_rope(k, np.array([b + d]), 500000.0)
        assert math.isclose(np.linalg.norm(qa), np.linalg.norm(q), rel_tol=1e-13)
        assert math.isclose(float((qa * kb).sum()), float((qd * kd).sum()), rel_tol=1e-9,
                            abs_tol=1e-9)


def test_rope_disabled():
    x = np.random.default_rng(2).standard_normal((3, 2, 4))
    assert np.array_equal(oracle.apply_rope(x, np.array([1, 2, 3]), 0.0), x)


# ---------------------------------------------------------------- attention
def _sdpa_segment(q, k, v, q_pos, k_pos, window):
    """torch SDPA in float64 with an explicit boolean mask; GQA by repeating KV."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    qp = torch.from_numpy(np.asarray(q_pos))[:, None]
    kp = torch.from_numpy(np.asarray(k_pos))[None, :]
    mask = kp <= qp
    if window > 0:
        mask &= kp > qp - window
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv,D,window", [(2, 2, 16, 0), (4, 2, 8, 0), (8, 2, 32, 5),
                                              (4, 1, 16, 1), (3, 3, 8, 17)])
def test_attention_matches_torch_sdpa(Hq, Hkv, D, window):
    rng = np.random.default_rng(Hq * 100 + D + window)
    n, c = 37, 11
    q = rng.standard_normal((n, Hq, D))
    keys = rng.standard_normal((c + n, Hkv, D))
    vals = rng.standard_normal((c + n, Hkv, D))
    q_pos = np.arange(c, c + n)
    k_pos = np.arange(c + n)
    out, lse = oracle.attention(q, keys, vals, q_pos, k_pos, window, threads=1, row_tile=8)
    ref = _sdpa_segment(q, keys, vals, q_pos, k_pos, window)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse: log of the softmax normaliser of the scaled logits
    z = np.einsum("thd,jhd->thj", q, np.repeat(keys, Hq // Hkv, axis=1)) / math.sqrt(D)
    vis = oracle.visible(q_pos, k_pos, window)
    z = np.where(vis[:, None, :], z, -np.inf)
    ref_lse = np.log(np.exp(z).sum(-1))
    assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def _seg_run(segments, q, k, v, positions, cu, Hq, Hkv, D, theta, window, cache, **kw):
    return oracle.run_call(segments=segments, q=q, k=k, v=v, positions=positions, cu_seqlens=cu,
                           Hq=Hq, Hkv=Hkv, D=D, theta=theta, window=window, block_size=16, p=0.9,
                           cache=cache, score=False, select=False, **kw)


def test_chunked_prefill_example_from_glossary_page():
    with open(os.path.join(GOLDEN, "chunked_prefill_example.json")) as f:
        g = json.load(f)
    L, C, H, D = g["prompt_len"], g["chunk"], g["heads"], g["head_dim"]
    # the page's inputs: one seeded draw of q, k and v together (the fixture
    # records the seed and the shape), as [L, H, D] float64
    gen = torch.Generator().manual_seed(g["torch_seed"])
    qkv = torch.randn((3, 1, H, L, D), generator=gen)[:, 0].permute(0, 2, 1, 3).double().numpy()
    q, k, v = qkv
    pos = np.arange(L)
    full = _seg_run([(0, 0, L, False)], q, k, v, pos, [0, L], H, H, D, 0.0, 0,
                    oracle.KVCacheModel())["out"]
    # the chunks come from this repository's chunk scheduler, and each call
    # reads the cache the earlier calls left in the oracle's KV record
    sched = W._chunk_schedule([L], C, flag=False)
    cache = oracle.KVCacheModel()
    outs = []
    for (seg,) in sched:
        a, b = seg.ctx, seg.ctx + seg.n
        outs.append(_seg_run([(0, seg.ctx, seg.n, False)], q[a:b], k[a:b], v[a:b], pos[a:b],
                             [0, seg.n], H, H, D, 0.0, 0, cache)["out"])
    chunked = np.concatenate(outs)
    assert [seg.n for (seg,) in sched] == g["expected_chunk_lengths"]
    assert np.allclose(full, chunked, atol=g["atol"], rtol=0) == g["expected_allclose"]
    # in float64 the two are equal far below the page's tolerance
    assert np.max(np.abs(full - chunked)) < 1e-12


@pytest.mark.parametrize("window,theta", [(0, 0.0), (0, 500000.0), (23, 10000.0)])
def test_chunked_equals_one_pass_with_rope_and_window(window, theta):
    rng = np.random.default_rng(5)
    L, Hq, Hkv, D = 150, 4, 2, 16
    q = rng.standard_normal((L, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    pos = np.arange(L)
    full = _seg_run([(0, 0, L, False)], q, k, v, pos, [0, L], Hq, Hkv, D, theta, window,
                    oracle.KVCacheModel())["out"]
    cache = oracle.KVCacheModel()
    outs = []
    for s, e in [(0, 40), (40, 41), (41, 97), (97, 150)]:
        outs.append(_seg_run([(0, s, e - s, False)], q[s:e], k[s:e], v[s:e], pos[s:e],
                             [0, e - s], Hq, Hkv, D, theta, window, cache)["out"])
    assert np.max(np.abs(full - np.concatenate(outs))) < 1e-12


def test_packed_equals_unpacked_bitwise():
    rng = np.random.default_rng(6)
    lens = [13, 1, 40, 7]
    Hq, Hkv, D, theta = 4, 2, 8, 500000.0
    T = sum(lens)
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    cu = np.concatenate([[0], np.cumsum(lens)])
    pos = np.concatenate([np.arange(n) for n in lens])  # positions restart per prompt
    segs = [(i, 0, n, False) for i, n in enumerate(lens)]
    packed = _seg_run(segs, q, k, v, pos, cu, Hq, Hkv, D, theta, 0, oracle.KVCacheModel(),
                      threads=1)
    for i, n in enumerate(lens):
        a, b = cu[i], cu[i + 1]
        alone = _seg_run([(0, 0, n, False)], q[a:b], k[a:b], v[a:b], pos[a:b], [0, n], Hq, Hkv,
                         D, theta, 0, oracle.KVCacheModel(), threads=1)
        assert np.array_equal(packed["out"][a:b], alone["out"])
        assert np.array_equal(packed["lse"][a:b], alone["lse"])


def test_closed_forms_zero_query_single_key_window():
    rng = np.random.default_rng(7)
    n, c, Hq, Hkv, D = 20, 6, 2, 1, 8
    keys = rng.standard_normal((c + n, Hkv, D))
    vals = rng.standard_normal((c + n, Hkv, D))
    q_pos, k_pos = np.arange(c, c + n), np.arange(c + n)
    # q == 0: uniform weights over the visible keys
    out, lse = oracle.attention(np.zeros((n, Hq, D)), keys, vals, q_pos, k_pos, 0, threads=1)
    for t in range(n):
        ref = vals[: c + t + 1, 0].mean(axis=0)
        assert np.allclose(out[t, 0], ref, atol=1e-14) and np.allclose(out[t, 1], ref, atol=1e-14)
        assert math.isclose(lse[t, 0], math.log(c + t + 1), rel_tol=1e-14)
    # window = 1: each token sees only itself
    q = rng.standard_normal((n, Hq, D))
    out, _ = oracle.attention(q, keys, vals, q_pos, k_pos, 1, threads=1)
    assert np.allclose(out[:, 0], vals[c:, 0], atol=1e-14)
    # window >= every distance: identical to full causal
    full, _ = oracle.attention(q, keys, vals, q_pos, k_pos, 0, threads=1)
    wide, _ = oracle.attention(q, keys, vals, q_pos, k_pos, c + n, threads=1)
    assert np.array_equal(full, wide)
    # q == 0 with a window of 4: mean of the last 4 positions
    out, _ = oracle.attention(np.zeros((n, Hq, D)), keys, vals, q_pos, k_pos, 4, threads=1)
    for t in range(n):
        p = c + t
        assert np.allclose(out[t, 0], vals[p - 3 : p + 1, 0].mean(axis=0), atol=1e-14)


def test_gapped_positions_window():
    # after compaction positions have gaps; the window acts on positions
    rng = np.random.default_rng(8)
    pos = np.array([0, 1, 5, 6, 20, 21, 22, 40])
    n, D = len(pos), 4
    q = np.zeros((n, 1, D))
    keys = rng.standard_normal((n, 1, D))
    vals = rng.standard_normal((n, 1, D))
    out, _ = oracle.attention(q, keys, vals, pos, pos, 6, threads=1)
    for t in range(n):
        vis = [j for j in range(n) if pos[t] - 6 < pos[j] <= pos[t]]
        assert np.allclose(out[t, 0], vals[vis, 0].mean(axis=0), atol=1e-14)
