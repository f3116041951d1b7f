"""Pins of the later-layer oracle (oracle/layers.py) against brute force,
closed forms and identities of the functions it writes out."""
import math

import numpy as np
import pytest

from oracle import layers as L


def _brute_linear(x, w):
    M, K = len(x), len(x[0])
    N = len(w)
    return [[math.fsum(x[m][k] * w[n][k] for k in range(K)) for n in range(N)] for m in range(M)]


def test_linear_matches_brute_force_loops():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 7))
    w = rng.standard_normal((5, 7))
    want = np.array(_brute_linear(x.tolist(), w.tolist()))
    got = L.linear(x, w)
    assert got.shape == (3, 5)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-14)


def test_linear_identity_and_one_hot_rows():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 6))
    assert np.array_equal(L.linear(x, np.eye(6)), x)
    # row n of w = e_j picks column j of x: a transposed operand fails this
    w = np.zeros((3, 6))
    w[0, 5] = w[1, 0] = w[2, 2] = 1.0
    assert np.array_equal(L.linear(x, w), x[:, [5, 0, 2]])
    with pytest.raises(ValueError):
        L.linear(x, np.zeros((3, 5)))


def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4, so silu(ln 3) = 3 ln 3 / 4; sigmoid(-ln 3) = 1/4
    ln3 = math.log(3.0)
    assert L.silu(np.array([ln3]))[0] == pytest.approx(0.75 * ln3, rel=1e-15)
    assert L.silu(np.array([-ln3]))[0] == pytest.approx(-0.25 * ln3, rel=1e-15)
    assert L.silu(np.array([0.0]))[0] == 0.0
    # sigmoid(z) + sigmoid(-z) = 1  =>  silu(z) - silu(-z) = z
    z = np.linspace(-30, 30, 121)
    assert np.allclose(L.silu(z) - L.silu(-z), z, rtol=1e-14, atol=1e-13)
    # limits: silu(z) -> z for large z, -> 0 from below for very negative z
    assert L.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    big_neg = L.silu(np.array([-800.0]))[0]
    assert big_neg <= 0.0 and big_neg > -1e-300
    assert np.all(np.isfinite(L.silu(np.array([-1e4, 1e4]))))


def test_swiglu_matches_brute_force_and_gate_identity():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 5))
    wg = rng.standard_normal((4, 5))
    wu = rng.standard_normal((4, 5))
    g = _brute_linear(x.tolist(), wg.tolist())
    u = _brute_linear(x.tolist(), wu.tolist())
    want = np.array([[g[m][f] / (1.0 + math.exp(-g[m][f])) * u[m][f] for f in range(4)]
                     for m in range(3)])
    assert np.allclose(L.swiglu(x, wg, wu), want, rtol=1e-13, atol=1e-14)
    # identity gate and up weights: silu(x) * x
    assert np.allclose(L.swiglu(x, np.eye(5), np.eye(5)), L.silu(x) * x, rtol=1e-15, atol=0)


def test_later_layer_flops_llama_shapes():
    # per token: 4096x6144 + 4096x4096 + 2x4096x14336 + 14336x4096 multiply-adds
    per_row_macs = 4096 * 6144 + 4096 * 4096 + 2 * 4096 * 14336 + 14336 * 4096
    assert per_row_macs == 218103808
    assert L.later_layer_flops(1) == 2 * per_row_macs
    assert L.later_layer_flops(1000) == 1000 * L.later_layer_flops(1)


def _quadratic_linear_attention(q, k, v, cu):
    """o_t = sum_{s<=t} w_ts v_s / sum_{s<=t} w_ts with w_ts = phi(q_t).phi(k_s),
    the non-recurrent form, written with plain loops."""
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros_like(q)
    for a, b in zip(cu[:-1], cu[1:]):
        for t in range(a, b):
            for h in range(Hq):
                fq = L.feature_map(q[t, h])
                num = np.zeros(D)
                den = 0.0
                for s in range(a, t + 1):
                    w = math.fsum(fq * L.feature_map(k[s, h // G]))
                    num += w * v[s, h // G]
                    den += w
                out[t, h] = num / den
    return out


def test_feature_map_closed_forms():
    x = np.array([-50.0, -1.0, 0.0, 0.5, 3.0])
    want = [math.exp(-50.0), math.exp(-1.0), 1.0, 1.5, 4.0]
    assert np.allclose(L.feature_map(x), want, rtol=1e-15, atol=0)
    assert np.all(L.feature_map(np.linspace(-700, 700, 101)) > 0)


def test_linear_attention_matches_quadratic_form():
    rng = np.random.default_rng(3)
    cu = [0, 5, 6, 13]
    q = rng.standard_normal((13, 4, 6))
    k = rng.standard_normal((13, 2, 6))
    v = rng.standard_normal((13, 2, 6))
    got = L.linear_attention(q, k, v, cu)
    assert np.allclose(got, _quadratic_linear_attention(q, k, v, cu), rtol=1e-12, atol=1e-13)


def test_linear_attention_special_cases():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((7, 2, 5))
    k = rng.standard_normal((7, 1, 5))
    v = rng.standard_normal((7, 1, 5))
    out = L.linear_attention(q, k, v, [0, 7])
    # the first token of a segment sees only itself: o = v
    assert np.allclose(out[0], v[0], rtol=1e-14, atol=1e-15)
    # a value shared by every token comes back unchanged
    vc = np.repeat(v[:1], 7, axis=0)
    assert np.allclose(L.linear_attention(q, k, vc, [0, 7]), np.broadcast_to(vc, (7, 2, 5)),
                       rtol=1e-13, atol=1e-14)
    # segments do not see each other: packing equals running each alone
    packed = L.linear_attention(q, k, v, [0, 3, 7])
    assert np.array_equal(packed[:3], L.linear_attention(q[:3], k[:3], v[:3], [0, 3]))
    assert np.array_equal(packed[3:], L.linear_attention(q[3:], k[3:], v[3:], [0, 4]))
