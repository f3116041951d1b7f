"""The parity checker must have power at the benchmark's scale.

At the Llama-shaped packed workload's input scale (q, k, v ~ N(0,1)/sqrt(128))
attention is nearly uniform and a row's outputs are about 0.09/sqrt(visible
keys), mostly below the 2e-2 absolute bound.  These tests take the oracle's
own output of one 2,048-token prompt at that scale and check that the checker
rejects plausible kernel mistakes (a zeroed row, two rows swapped, a row
computed over another KV head's keys, a row whose output is halved) and
accepts the kernel's legitimate rounding (bf16 probabilities and bf16
outputs)."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_checks import (BF16_OUT_ABS, check_bf16_values, check_out, row_bound,
                           sample_rows)


@pytest.fixture(scope="module")
def c2_scale_prompt():
    wl = W.custom(lengths=[2048], Hq=4, Hkv=1, D=128, dtype="bf16", block_size=64, p=0.95,
                  theta=500000.0, seed=11, scale=1.0 / np.sqrt(128.0), hidden_width=16)
    call = wl.calls[0]
    pos = call.positions.astype(np.int64)
    q = oracle.apply_rope(W.to_f64(call.q, "bf16"), pos, wl.theta)
    k = oracle.apply_rope(W.to_f64(call.k, "bf16"), pos, wl.theta)
    v = W.to_f64(call.v, "bf16")
    out, _ = oracle.attention(q, k, v, pos, pos)
    return wl, q, k, v, pos, out


def _bf16_round(x):
    return W.to_f64(W.f32_to_bf16_bits(np.asarray(x, np.float32)), "bf16")


def test_absolute_bound_alone_is_powerless_at_this_scale(c2_scale_prompt):
    """Most rows lie entirely below the absolute bound (why the row-relative
    bound is needed)."""
    out = c2_scale_prompt[5]
    below = (np.abs(out).max(axis=(1, 2)) < BF16_OUT_ABS).sum()
    assert below > 0.8 * out.shape[0]


def test_checker_accepts_kernel_rounding(c2_scale_prompt):
    """bf16 probabilities (normalised by their own bf16 sum) and a bf16
    output, the kernel's rounding points, stay well inside the bound."""
    wl, q, k, v, pos, out = c2_scale_prompt
    rows = np.arange(0, 2048, 7)
    emu = np.zeros((len(rows), 4, 128))
    for h in range(4):
        P, _ = oracle.softmax_probs(q[rows], k, pos[rows], pos, 0, h, 4)
        Pb = _bf16_round(P * 3.7)  # probabilities against a stale max: scaled, same rounding
        emu[:, h, :] = (Pb @ v[:, 0, :]) / Pb.sum(axis=1, keepdims=True)
    got = W.f32_to_bf16_bits(emu.astype(np.float32))
    ratio = check_out("bf16", got, out[rows], "emulated kernel rounding")
    assert ratio < 0.5


@pytest.mark.parametrize("mutation", ["zero_row", "swap_rows", "other_head_keys", "halve_row",
                                      "drop_first_tile"])
def test_checker_rejects_plausible_mistakes(c2_scale_prompt, mutation):
    wl, q, k, v, pos, out = c2_scale_prompt
    bad = out.copy()
    t = 1500
    if mutation == "zero_row":
        bad[t] = 0.0
    elif mutation == "swap_rows":
        bad[[t, t + 1]] = bad[[t + 1, t]]
    elif mutation == "other_head_keys":
        # query head 1 of row t against key/value rows of a different
        # segment of the stream (keys shifted by 512 positions)
        P, _ = oracle.softmax_probs(q[t:t + 1], k[:t - 511], pos[t:t + 1], pos[:t - 511], 0, 1, 4)
        bad[t, 1] = (P @ v[:t - 511, 0, :])[0]
    elif mutation == "halve_row":
        bad[t, 2] *= 0.5
    elif mutation == "drop_first_tile":
        # row t computed without its first 64 keys
        P, _ = oracle.softmax_probs(q[t:t + 1], k[64:], pos[t:t + 1], pos[64:], 0, 0, 4)
        bad[t, 0] = (P @ v[64:, 0, :])[0]
    # the absolute bound alone would accept every one of these
    assert np.abs(bad - out).max() <= BF16_OUT_ABS
    with pytest.raises(AssertionError):
        check_bf16_values(bad, out, mutation)


def test_row_bound_scales_per_row():
    ref = np.array([[[1.0, -2.0], [0.001, 0.0]]])
    b = row_bound(ref, rel=0.5, floor=0.0)
    assert np.allclose(b, [[[1.0, 1.0], [0.0005, 0.0005]]])


def test_sample_rows_cover_tiles_and_last_block():
    rng = np.random.default_rng(0)
    r = sample_rows(rng, 1000, 64, k_random=4, tile=64)
    assert r[0] == 0 and r[-1] == 999
    assert set(range(960, 1000)) <= set(r)
    for b in range(64, 1000, 64):
        assert b - 1 in r and b in r
    assert sample_rows(rng, 1, 64) == [0]
