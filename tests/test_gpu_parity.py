"""GPU parity: the HIP library against the CPU oracle on seeded inputs.

Attention outputs and scores within the stated tolerances (see
gpu_harness), selection and compaction bit-exact (oracle selection run on the
GPU-emitted scores).  Small shapes span several tiles, ragged tails, cached
prefixes that are and are not page/block multiples, GQA ratios 1..8, head
dims 64 and 128, windows, p in {0, 0.5, 0.9, 1} and both dtypes.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle import driver

pytestmark = pytest.mark.gpu


def _run_and_check(wl, check_lse=True):
    import gpu_harness as H
    H.log(f"case {wl.name} dtype={wl.dtype} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} B={wl.block_size} "
          f"p={wl.p} window={wl.window} lens={[s.n for s in wl.calls[0].segments]} "
          f"ctx={[s.ctx for s in wl.calls[0].segments]}")
    ref = driver.run_workload(wl, layer2=False)
    kc, vc = H.make_caches(wl)
    for ci, call in enumerate(wl.calls):
        pc = H.launch_call(wl, call, kc, vc)
        g = H.gpu_result(pc)
        r = ref[ci]
        H.check_out(wl.dtype, g["out"], r["out"], f"call {ci} out")
        if check_lse:
            if wl.dtype == "bf16":
                assert np.abs(g["lse"] - r["lse"]).max() <= H.BF16_OUT_ABS
            else:
                assert np.allclose(g["lse"], r["lse"], rtol=1e-5, atol=1e-5)
        cb = g["cu_blocks"]
        for i, s in enumerate(call.segments):
            if s.flagged:
                H.check_scores(wl.dtype, g["scores"][cb[i]:cb[i + 1]], r["scores"][i])
        H.check_selection_and_compaction(wl, call, g)
    return True


def test_gpu_small_chunked_fp32():
    assert _run_and_check(W.make("small_chunked_fp32"))


def test_gpu_small_chunked_fp32_second_seed_with_rope():
    wl = W.make("small_chunked_fp32", seed=101)
    wl.theta = 500000.0
    assert _run_and_check(wl)


CASES = [
    dict(lengths=[1, 15, 16, 17, 100], ctxs=[0, 0, 33, 16, 7], Hq=2, Hkv=2, D=64, dtype="f32",
         block_size=16, p=0.9),
    dict(lengths=[200, 3], ctxs=[50, 0], Hq=8, Hkv=2, D=128, dtype="f32", block_size=32, p=0.5,
         theta=10000.0),
    dict(lengths=[300, 70], ctxs=[0, 40], Hq=4, Hkv=4, D=64, dtype="f32", block_size=64, p=0.95,
         theta=500000.0, window=50),
    dict(lengths=[1, 63, 64, 65, 300], ctxs=[0, 17, 64, 0, 129], Hq=8, Hkv=2, D=128,
         dtype="bf16", block_size=64, p=0.9, theta=500000.0),
    dict(lengths=[130, 257], ctxs=[0, 0], Hq=2, Hkv=2, D=64, dtype="bf16", block_size=16, p=0.0),
    dict(lengths=[513, 129], ctxs=[0, 256], Hq=16, Hkv=2, D=128, dtype="bf16", block_size=128,
         p=1.0, theta=500000.0),
    dict(lengths=[400, 90], ctxs=[0, 0], Hq=4, Hkv=2, D=128, dtype="bf16", block_size=32, p=0.5,
         theta=500000.0, window=100),
    dict(lengths=[1] * 10 + [200], ctxs=[100, 300, 17, 1000, 2000, 5, 64, 128, 129, 700, 0],
         flags=[False] * 10 + [True], Hq=8, Hkv=2, D=128, dtype="bf16", block_size=64, p=0.95,
         theta=500000.0),
    dict(lengths=[700], ctxs=[0], Hq=32, Hkv=8, D=128, dtype="bf16", block_size=64, p=0.95,
         theta=500000.0, scale=1.0 / np.sqrt(128.0)),
    # largest query group (G = 32: 8 positions per tile), D = 64, cached keys and a window
    dict(lengths=[150, 40], ctxs=[33, 200], Hq=64, Hkv=2, D=64, dtype="bf16", block_size=16,
         p=0.9, theta=500000.0, window=70),
    # G = 1 at D = 64 with long cached context
    dict(lengths=[90, 300], ctxs=[1000, 5], Hq=8, Hkv=8, D=64, dtype="bf16", block_size=32,
         p=0.8, theta=10000.0),
    # large logits (queries scaled, values not; no rotation, so the bf16
    # queries are exact): a row's max rises by up to ~50 log2 units over
    # its first tile's, and by up to ~290 in the second case, so the running
    # max is raised often and far
    dict(lengths=[700, 260], ctxs=[0, 150], Hq=16, Hkv=4, D=128, dtype="bf16", block_size=64,
         p=0.9, theta=0.0, q_mult=12.0),
    dict(lengths=[500, 90], ctxs=[64, 0], Hq=8, Hkv=2, D=64, dtype="bf16", block_size=32,
         p=0.9, theta=0.0, q_mult=40.0, window=200),
    # block sizes that are multiples of 16 but not powers of two, and the
    # largest (runs of 16, 32 and 64 keys; last blocks of up to 256 rows)
    dict(lengths=[700, 100, 48], ctxs=[0, 37, 0], Hq=8, Hkv=2, D=128, dtype="bf16", block_size=48,
         p=0.8, theta=500000.0),
    dict(lengths=[1000, 333], ctxs=[0, 64], Hq=16, Hkv=4, D=128, dtype="bf16", block_size=96,
         p=0.7, theta=500000.0, window=300),
    dict(lengths=[1300, 257], ctxs=[0, 0], Hq=8, Hkv=8, D=64, dtype="bf16", block_size=256,
         p=0.9, theta=500000.0),
    dict(lengths=[900, 200], ctxs=[0, 100], Hq=32, Hkv=8, D=128, dtype="bf16", block_size=192,
         p=0.6, theta=500000.0),
    dict(lengths=[300, 81], ctxs=[0, 17], Hq=2, Hkv=2, D=64, dtype="f32", block_size=80,
         p=0.7),
    dict(lengths=[400, 70], ctxs=[16, 0], Hq=4, Hkv=2, D=64, dtype="f32", block_size=48,
         p=0.5, theta=500000.0, window=90),
    dict(lengths=[600], ctxs=[0], Hq=2, Hkv=2, D=128, dtype="f32", block_size=256, p=0.9),
    # query groups that are not powers of two: a tile holds 256 // G
    # positions (bf16) or 128 // G (fp32) and leaves the remaining rows
    # unused; G = 12 takes the per-quad rotary path, the others the per-lane
    # one; the fp32 scoring passes cover whole tokens (126 rows at G = 6)
    dict(lengths=[700, 1, 130], ctxs=[0, 500, 70], Hq=12, Hkv=4, D=128, dtype="bf16",
         block_size=64, p=0.9, theta=500000.0),
    dict(lengths=[333, 90], ctxs=[64, 0], Hq=40, Hkv=8, D=128, dtype="bf16", block_size=32,
         p=0.8, theta=500000.0, window=150),
    dict(lengths=[500, 47], ctxs=[0, 200], Hq=28, Hkv=4, D=64, dtype="bf16", block_size=16,
         p=0.95, theta=1000000.0),
    dict(lengths=[400, 5], ctxs=[0, 100], Hq=24, Hkv=2, D=128, dtype="bf16", block_size=64,
         p=0.9, theta=500000.0),
    dict(lengths=[300, 45], ctxs=[0, 20], Hq=12, Hkv=2, D=64, dtype="f32", block_size=64,
         p=0.9, theta=10000.0),
    dict(lengths=[200], ctxs=[30], Hq=6, Hkv=2, D=128, dtype="f32", block_size=32, p=0.8,
         theta=500000.0, window=60),
    # D = 64 at G = 6 (42 positions per tile) with decodes and a window
    dict(lengths=[1, 250, 1, 90], ctxs=[700, 0, 45, 33], flags=[False, True, False, True],
         Hq=12, Hkv=2, D=64, dtype="bf16", block_size=32, p=0.9, theta=500000.0, window=120),
    # the largest KV head count the cache addressing accepts (255, G = 1)
    dict(lengths=[40, 17], ctxs=[20, 0], Hq=255, Hkv=255, D=64, dtype="bf16", block_size=16,
         p=0.9, theta=500000.0),
    # degenerate windows: one key (each token sees itself only) and one wider
    # than every distance (full causal), with cached prefixes
    dict(lengths=[130, 64, 1], ctxs=[0, 40, 90], Hq=8, Hkv=2, D=128, dtype="bf16", block_size=64,
         p=0.9, theta=500000.0, window=1),
    dict(lengths=[300, 77], ctxs=[50, 0], Hq=8, Hkv=2, D=128, dtype="bf16", block_size=64,
         p=0.9, theta=500000.0, window=1 << 20),
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_gpu_fuzz_cases(idx):
    kw = dict(CASES[idx])
    wl = W.custom(seed=1000 + idx, hidden_width=64, **kw)
    assert _run_and_check(wl)


def test_gpu_scored_segment_after_many_one_block_segments():
    """300 unscored one-token segments ahead of scored ones, so the block-mass
    kernel's segment search runs with every probe of a round below the
    block (regression: the search once excluded the unprobed candidates)."""
    lengths = [1] * 300 + [700, 130]
    ctxs = [int(x) for x in np.random.default_rng(9).integers(1, 200, size=300)] + [0, 64]
    flags = [False] * 300 + [True, True]
    wl = W.custom(seed=4300, hidden_width=16, lengths=lengths, ctxs=ctxs, flags=flags, Hq=8,
                  Hkv=2, D=128, dtype="bf16", block_size=64, p=0.9, theta=500000.0)
    assert _run_and_check(wl)


def test_gpu_most_segments_per_call():
    """4096 segments (the planner's limit) of 1..9 tokens, some with cached
    prefixes, alternate segments scored."""
    rng = np.random.default_rng(5)
    S = 4096
    lengths = [int(x) for x in rng.integers(1, 10, size=S)]
    ctxs = [int(x) if i % 3 == 0 else 0 for i, x in enumerate(rng.integers(1, 40, size=S))]
    flags = [i % 2 == 0 for i in range(S)]
    wl = W.custom(seed=4096, hidden_width=16, lengths=lengths, ctxs=ctxs, flags=flags, Hq=4,
                  Hkv=2, D=64, dtype="bf16", block_size=16, p=0.9, theta=500000.0)
    assert _run_and_check(wl)


def test_gpu_bin_packed_rows_with_padding_segments():
    """Prompts bin-packed into rows of a fixed capacity, each row closed by an
    unscored padding segment (the layout bench.py --sweep times against the
    packed one)."""
    from block_sparse_token_amd import packing as PK
    segs, pad_flags, pad, nrows = PK.bin_packed_segments([100, 37, 250, 64, 180, 256, 5], 256)
    assert pad > 0 and nrows >= 4
    wl = W.custom(seed=4242, hidden_width=64, lengths=segs, flags=[not f for f in pad_flags],
                  Hq=8, Hkv=2, D=128, dtype="bf16", block_size=64, p=0.95, theta=500000.0,
                  scale=1.0 / np.sqrt(128.0))
    assert _run_and_check(wl)


@pytest.mark.parametrize("B,lengths,ctxs,flags,p", [
    (64, [88, 200, 64, 5], [512, 256, 0, 700], [True, True, True, False], 0.6),
    (16, [40, 1, 33], [48, 160, 0], [True, True, True], 0.5),
    (128, [300], [1024], [True], 0.7),
    (48, [100, 30], [480, 96], [True, True], 0.6),
    (256, [400], [512], [True], 0.8),
])
def test_gpu_whole_prompt_scoring(B, lengths, ctxs, flags, p):
    """Final chunks scored over their whole prompt (cached blocks included):
    block scores, selection and compaction by prompt block, and the KV slots
    of the kept cached tokens, against the oracle."""
    _whole_prompt_case(B, lengths, ctxs, flags, p)


def test_gpu_whole_prompt_scoring_query_group_of_five():
    """The same with 20 query heads over 4 KV heads (a tile of 51 positions,
    one packed row unused) and a decode segment beside the scored ones."""
    _whole_prompt_case(64, [150, 1, 70], [256, 300, 128], [True, False, True], 0.7, Hq=20, Hkv=4,
                       seed=7105)


def _whole_prompt_case(B, lengths, ctxs, flags, p, Hq=8, Hkv=2, seed=None):
    import torch
    import gpu_harness as H
    from block_sparse_token_amd import binding as Bd

    wl = W.custom(seed=7000 + B if seed is None else seed, hidden_width=64, lengths=lengths,
                  ctxs=ctxs, flags=flags, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", block_size=B, p=p,
                  theta=500000.0, scale=1.0 / np.sqrt(128.0))
    call = wl.calls[0]
    H.log(f"whole-prompt scoring B={B} lens={lengths} ctx={ctxs} flags={flags} p={p}")
    ref = driver.run_workload(wl, layer2=False, scope="prompt")[0]
    kc, vc = H.make_caches(wl)
    pc = H.launch_call(wl, call, kc, vc, whole_prompt=True)
    g = H.gpu_result(pc)
    H.check_out(wl.dtype, g["out"], ref["out"], "out")
    cb = g["cu_blocks"]
    for i, s in enumerate(call.segments):
        if s.flagged:
            assert cb[i + 1] - cb[i] == -(-(s.ctx + s.n) // B)
            H.check_scores(wl.dtype, g["scores"][cb[i]:cb[i + 1]], ref["scores"][i])
    H.check_selection_and_compaction(wl, call, g, whole_prompt=True)
    # kept cached tokens: the oracle's positions (on the GPU's keep masks)
    # mapped to slots through the block table
    keeps = [g["keep"][cb[i]:cb[i + 1]].astype(bool) for i in range(len(call.segments))]
    pos = oracle.kept_cache_positions(flags, B, keeps, ctxs)
    bt = call.block_table
    want = np.concatenate([bt[i][u // 16] * 16 + u % 16 for i, u in enumerate(pos)]).astype(np.int32)
    S = len(lengths)
    cap = int(sum(ctxs))
    slots = torch.full((cap + 8,), -7, dtype=torch.int32, device="cuda")
    cu_out = torch.zeros(S + 1, dtype=torch.int32, device="cuda")
    num = torch.zeros(1, dtype=torch.int32, device="cuda")
    Bd.up_kept_cache_slots(pc.batch, B, pc.cu_blocks, pc.flags, pc.keep, pc.num_blocks, slots,
                           cu_out, num, pc.compact_ws)
    torch.cuda.synchronize()
    n = int(num.item())
    assert n == len(want)
    assert np.array_equal(slots[:n].cpu().numpy(), want)
    assert np.all(slots[n:].cpu().numpy() == -7)
    counts = [len(u) for u in pos]
    assert np.array_equal(cu_out.cpu().numpy(), np.concatenate([[0], np.cumsum(counts)]))


def test_gpu_fused_score_select_equals_separate_stages():
    """up_score_select gives bit for bit what up_block_scores followed by
    up_topp_select give on the same block mass (ragged segments, unscored
    segments, p below and at 1)."""
    import torch
    import gpu_harness as H

    for p in (0.0, 0.6, 0.95, 1.0):
        wl = W.custom(seed=31, hidden_width=16, lengths=[700, 1, 130, 64, 257],
                      ctxs=[0, 40, 0, 16, 0], flags=[True, False, True, True, True], Hq=8, Hkv=2,
                      D=128, dtype="bf16", block_size=64, p=p, theta=500000.0)
        call = wl.calls[0]
        kc, vc = H.make_caches(wl)
        pc = H.launch_call(wl, call, kc, vc, compact=False)
        fused = (pc.scores.clone(), pc.keep.clone(), pc.kept_blocks.clone())
        pc.scores.fill_(-1.0)
        pc.keep.fill_(7)
        pc.kept_blocks.fill_(-1)
        pc.scores_stage()
        pc.select_stage()
        torch.cuda.synchronize()
        assert torch.equal(fused[0].view(torch.int32), pc.scores.view(torch.int32)), p
        assert torch.equal(fused[1], pc.keep), p
        assert torch.equal(fused[2], pc.kept_blocks), p
        H.check_selection_and_compaction(wl, call, H.gpu_result(pc))
