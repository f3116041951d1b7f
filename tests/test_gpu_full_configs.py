"""GPU parity at the five workloads' full sizes, launched as the benchmark
launches them (same library calls, same buffers).

The float64 oracle cannot redo 10^14 flops, so these tests check, per
segment, sampled query rows (the first and last rows, every row of the last
block, both sides of every query-tile boundary and 32 seeded rows), whole
short prompts, complete block scores of the listed segments, and - bit-exact
- the selection (the oracle's top-p on the GPU scores) and the compaction of
every call.  Outputs are held to the absolute bf16 bound and a row-relative
one (``parity_checks``).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import driver

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _tile_rows(wl):
    # query positions per attention work item (256 packed rows over G heads)
    return 256 // (wl.Hq // wl.Hkv)


def _rows(wl, rng, n, k=32):
    from parity_checks import sample_rows
    return sample_rows(rng, n, wl.block_size, k_random=k, tile=_tile_rows(wl))


def _check_segments(wl, call, g, cached_of, score_segs, rng, k_rows=32, full_segs=()):
    import gpu_harness as H
    cu = call.cu_seqlens
    cb = g["cu_blocks"]
    worst = 0.0
    for si, s in enumerate(call.segments):
        rows = list(range(s.n)) if si in full_segs else _rows(wl, rng, s.n, k_rows)
        do_score = s.flagged and si in score_segs
        r = driver.sampled_segment(wl, call, si, rows, cached=cached_of(si, s), score=do_score)
        got = g["out"][cu[si] + np.asarray(rows)]
        worst = max(worst, H.check_out(wl.dtype, got, r["out"],
                                       f"segment {si} ({len(rows)} rows)"))
        if do_score:
            H.check_scores(wl.dtype, g["scores"][cb[si]:cb[si + 1]], r["scores"])
    H.check_selection_and_compaction(wl, call, g)
    H.log(f"{wl.name}: worst error / row-relative bound = {worst:.3f}")


# the workload's own seed and a second one (other lengths and values)
@pytest.mark.parametrize("seed", [2, 12])
def test_gpu_packed_llama8b_full(seed):
    import gpu_harness as H
    wl = W.make("packed_llama8b", seed=seed)
    call = wl.calls[0]
    H.log(f"packed_llama8b seed {seed}: T={call.T}")
    kc, vc = H.make_caches(wl)
    g = H.gpu_result(H.launch_call(wl, call, kc, vc))
    H.log("packed_llama8b: gpu done, checking")
    shortest = set(int(x) for x in np.argsort([s.n for s in call.segments])[:3])
    _check_segments(wl, call, g, lambda si, s: None, set(range(len(call.segments))),
                    np.random.default_rng(0), full_segs=shortest)
    H.log("packed_llama8b: ok")


def test_gpu_chunked_128k_full():
    import gpu_harness as H
    wl = W.make("chunked_128k")
    kc, vc = H.make_caches(wl)
    rng = np.random.default_rng(1)
    check = {0, 1, 7, 15}
    for ci, call in enumerate(wl.calls):
        g = H.gpu_result(H.launch_call(wl, call, kc, vc))
        if ci not in check:
            # selection and compaction are checked bit-exact for every call
            H.check_selection_and_compaction(wl, call, g)
            continue
        H.log(f"chunked_128k: call {ci} ctx={call.segments[0].ctx}")

        def cached_of(si, s, ci=ci):
            if s.ctx == 0:
                return None
            kk, vv, pp = driver.prompt_kv_before(wl, ci, s.prompt)
            return oracle.apply_rope(kk, pp, wl.theta), vv

        _check_segments(wl, call, g, cached_of, {0}, rng, k_rows=8)
    H.log("chunked_128k: ok")


def test_gpu_chunked_128k_whole_prompt_full():
    """The 131072-token prompt with only its final chunk scored, over the
    whole prompt: all 1024 block scores, sampled output rows, selection and
    compaction by prompt block, and the kept cached tokens' KV slots."""
    import gpu_harness as H
    from block_sparse_token_amd import binding as Bd
    wl = W.make("chunked_128k")
    kc, vc = H.make_caches(wl)
    last = len(wl.calls) - 1
    for ci, call in enumerate(wl.calls[:-1]):
        H.launch_call(wl, call, kc, vc, flags=False, compact=False)
    call = wl.calls[last]
    H.log(f"chunked_128k whole prompt: final call ctx={call.segments[0].ctx}")
    pc = H.launch_call(wl, call, kc, vc, whole_prompt=True)
    g = H.gpu_result(pc)
    kk, vv, pp = driver.prompt_kv_before(wl, last, call.segments[0].prompt)
    cached = (oracle.apply_rope(kk, pp, wl.theta), vv)
    s = call.segments[0]
    rows = _rows(wl, np.random.default_rng(3), s.n, 8)
    r = driver.sampled_segment(wl, call, 0, rows, cached=cached, score=True, scope="prompt")
    H.check_out(wl.dtype, g["out"][np.asarray(rows)], r["out"], f"final chunk rows {rows}")
    cb = g["cu_blocks"]
    assert cb[1] - cb[0] == 1024
    H.check_scores(wl.dtype, g["scores"][cb[0]:cb[1]], r["scores"])
    H.check_selection_and_compaction(wl, call, g, whole_prompt=True)
    keep = g["keep"][cb[0]:cb[1]].astype(bool)
    pos = oracle.kept_cache_positions([True], wl.block_size, [keep], [s.ctx])[0]
    want = (call.block_table[0][pos // 16] * 16 + pos % 16).astype(np.int32)
    n = int(pc.num_kept_slots.item())
    assert n == len(want)
    assert np.array_equal(pc.kept_slots[:n].cpu().numpy(), want)
    H.log(f"chunked_128k whole prompt: ok ({int(keep.sum())} of 1024 blocks kept)")


@pytest.mark.parametrize("seed", [4, 14])
def test_gpu_mixed_decode_prefill_full(seed):
    """Decodes over a 17.7 GB cache drawn on the device, plus the prefill
    chunks.  The checked decodes' cached K/V are copied to the host before
    the launch (so the oracle's inputs never pass through the library), and
    after it every cache row outside this call's slots must be unchanged."""
    import gpu_harness as H
    wl = W.make("mixed_decode_prefill", seed=seed)
    call = wl.calls[0]
    H.log(f"mixed_decode_prefill seed {seed}: T={call.T} segments={len(call.segments)}")
    kc, vc = H.make_caches(wl)
    n_dec = sum(1 for s in call.segments if not s.flagged)
    rng = np.random.default_rng(2)
    ctxs = [s.ctx for s in call.segments[:n_dec]]
    pick = {int(np.argmax(ctxs)), int(np.argmin(ctxs))}
    pick.update(int(x) for x in rng.choice(n_dec, size=10, replace=False))
    before = {si: H.read_back_cache(wl, kc, vc, call.segments[si].prompt, call.segments[si].ctx)
              for si in sorted(pick)}
    kc0, vc0 = kc.clone(), vc.clone()
    H.log("mixed_decode_prefill: cache snapshot taken")
    g = H.gpu_result(H.launch_call(wl, call, kc, vc))
    H.log("mixed_decode_prefill: gpu done")
    # nothing but this call's own slots changed
    H.assert_cache_unchanged_outside(kc0, kc, call.slot_mapping)
    H.assert_cache_unchanged_outside(vc0, vc, call.slot_mapping)
    del kc0, vc0
    # the call's own slots hold its rotated keys and its values
    H.check_written_slots(wl, call, kc, vc, rng.choice(call.T, size=256, replace=False))
    cu = call.cu_seqlens
    for si in sorted(pick):
        s = call.segments[si]
        K, V = before[si]
        r = driver.sampled_segment(wl, call, si, [0],
                                   cached=(W.to_f64(K, "bf16"), W.to_f64(V, "bf16")))
        H.check_out("bf16", g["out"][cu[si]:cu[si] + 1], r["out"], f"decode {si} ctx {s.ctx}")
    for si in range(n_dec, len(call.segments)):
        s = call.segments[si]
        rows = _rows(wl, rng, s.n, 32)
        r = driver.sampled_segment(wl, call, si, rows, score=True)
        H.check_out("bf16", g["out"][cu[si] + np.asarray(rows)], r["out"], f"prefill {si}")
        H.check_scores("bf16", g["scores"][g["cu_blocks"][si]:g["cu_blocks"][si + 1]],
                       r["scores"])
    H.check_selection_and_compaction(wl, call, g)
    H.log("mixed_decode_prefill: ok")


def test_gpu_swa_after_selection_full():
    import gpu_harness as H
    from block_sparse_token_amd import step as ST
    wl = W.make("swa_after_selection")
    call = wl.calls[0]
    H.log(f"swa_after_selection: T={call.T}")
    kc, vc = H.make_caches(wl)
    pc = H.launch_call(wl, call, kc, vc)
    g = H.gpu_result(pc)
    H.log("swa_after_selection: layer 1 done")
    rng = np.random.default_rng(3)
    _check_segments(wl, call, g, lambda si, s: None, set(range(len(call.segments))), rng)
    # layer 2: sliding window over the kept tokens at their original positions,
    # K/V written at the compacted slots of a second cache
    nk = g["num_kept"]
    S = len(call.segments)
    batch2 = ST.B.Batch(pc.cu_seqlens_out, torch.zeros(S, dtype=torch.int32, device="cuda"),
                        pc.rows_out["positions"][:nk].contiguous(),
                        pc.rows_out["slot_mapping"][:nk].contiguous(), None)
    kc2, vc2 = torch.zeros_like(kc), torch.zeros_like(vc)
    l2 = ST.PrefillCall(batch=batch2, q=pc.rows_out["q2"][:nk].contiguous(),
                        k=pc.rows_out["k2"][:nk].contiguous(),
                        v=pc.rows_out["v2"][:nk].contiguous(), k_cache=kc2, v_cache=vc2,
                        num_blocks=1, flags=None, block_size=wl.block_size, p=wl.p,
                        rope_theta=wl.layer2["theta"], window=wl.layer2["window"])
    l2.launch()
    torch.cuda.synchronize()
    out2 = ST.tensor_to_stored(l2.out)
    H.log(f"swa_after_selection: layer 2 done on {nk} kept tokens")
    ro = g["rows_out"]
    cu2 = g["cu_seqlens_out"]
    for si in range(S):
        n2 = int(cu2[si + 1] - cu2[si])
        rows = _rows(wl, rng, n2, 16)
        r = driver.sampled_segment(wl, call, si, rows, theta=wl.layer2["theta"],
                                   window=wl.layer2["window"], q=ro["q2"], k=ro["k2"],
                                   v=ro["v2"], positions=ro["positions"], cu=cu2)
        H.check_out("bf16", out2[cu2[si] + np.asarray(rows)], r["out"], f"layer2 segment {si}")
    H.log("swa_after_selection: ok")
