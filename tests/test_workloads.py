"""The seeded input generators: shapes, determinism, bf16 rounding, paging."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.0, -2.5, 3.0e-3, 65504.0, 1.00390625, 1.01171875, 0.0, -0.0,
                                  np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45,
                                  1.1754942e-38, -1.0039062], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_small_chunked_fp32_schedule():
    wl = W.make("small_chunked_fp32")
    assert [c.T for c in wl.calls] == [229, 100, 64, 63]
    assert wl.calls[0].q.dtype == np.float32 and wl.calls[0].q.shape == (229, 2, 64)
    assert [(s.prompt, s.ctx, s.n) for s in wl.calls[1].segments] == [(1, 64, 36), (3, 64, 64)]
    assert sum(c.num_blocks(16) for c in wl.calls) == 30
    assert wl.num_pages == 30
    # slots agree with the page table
    for c in wl.calls:
        for i, s in enumerate(c.segments):
            a, b = c.cu_seqlens[i], c.cu_seqlens[i + 1]
            pos = c.positions[a:b]
            assert np.array_equal(pos, np.arange(s.ctx, s.ctx + s.n))
            page = c.block_table[i][pos // 16]
            assert np.array_equal(c.slot_mapping[a:b], page * 16 + pos % 16)


def test_deterministic():
    a, b = W.make("small_chunked_fp32"), W.make("small_chunked_fp32")
    for ca, cb in zip(a.calls, b.calls):
        assert np.array_equal(ca.q, cb.q) and np.array_equal(ca.k, cb.k)
        assert np.array_equal(ca.slot_mapping, cb.slot_mapping)
    c = W.make("small_chunked_fp32", seed=101)
    assert not np.array_equal(a.calls[0].q, c.calls[0].q)


def test_heavy_hitters_c1():
    wl = W.make("small_chunked_fp32")
    # 3 of the 30 groups carry +3u: their keys have a large common component
    ks = np.concatenate([c.k for c in wl.calls])  # packed order differs from prompt order,
    norms = np.linalg.norm(ks.astype(np.float64), axis=-1).mean(axis=1)
    assert (norms > 8.5).sum() >= 3 * 16 - 16  # heavy keys have norm about sqrt(64 + 9)


def test_custom_given_cache_and_paging():
    wl = W.custom(lengths=[5, 20], ctxs=[17, 0], Hq=4, Hkv=2, D=8, dtype="bf16", seed=3)
    assert wl.calls[0].q.dtype == np.uint16
    kc, vc = W.paged_given_cache(wl)
    K, V = wl.given_cache[0]
    pg = wl.prompt_pages[0]
    for pos in range(17):
        assert np.array_equal(kc[pg[pos // 16], :, pos % 16], K[pos])


@pytest.mark.parametrize("name", ["packed_llama8b", "mixed_decode_prefill"])
def test_big_configs_shapes(name):
    wl = W.make(name) if name != "mixed_decode_prefill" else W.make("mixed_decode_prefill", device_cache=True)
    c = wl.calls[0]
    if name == "packed_llama8b":
        assert len(c.segments) == 16 and 16 * 512 <= c.T <= 16 * 8192
        assert c.q.shape == (c.T, 32, 128) and c.hidden.shape == (c.T, 4096)
    else:
        assert c.T == 8192 and sum(1 for s in c.segments if s.n == 1) == 256
        assert all(not s.flagged for s in c.segments[:256])
        assert all(s.flagged for s in c.segments[256:])
        assert wl.device_cache_seed is not None
