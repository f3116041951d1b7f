"""Whole-step determinism: the same inputs run twice give bit-identical
attention outputs, log-sum-exps, block scores, keep masks, index maps,
compacted offsets and compacted rows, and the same KV cache.

Top-p selection has to be reproducible (UniPrefill review, "Key Terms &
Definitions", Top-p Token Selection): the kept set must not depend on the
order in which threads finish.  The library sums the block mass in a fixed
order and selects with integer sums, so nothing may differ by even one bit.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def _bits(t):
    """Bit pattern view (so -0.0 against 0.0 or two NaNs compare exactly)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _outputs(pc):
    t = {"out": pc.out, "lse": pc.lse, "scores": pc.scores, "keep": pc.keep,
         "kept_blocks": pc.kept_blocks, "cu_blocks": pc.cu_blocks}
    if pc.compact:
        nk = int(pc.num_kept.item())
        t["num_kept"] = pc.num_kept
        t["index_map"] = pc.index_map[:nk]
        t["cu_seqlens_out"] = pc.cu_seqlens_out
        for name, r in pc.rows_out.items():
            t["rows_" + name] = r[:nk]
    return {k: v.clone() for k, v in t.items() if v is not None}


def _run_twice(name):
    import gpu_harness as H
    wl = W.make(name)
    runs = []
    for rep in range(2):
        kc, vc = H.make_caches(wl)
        outs = []
        for ci, call in enumerate(wl.calls):
            pc = H.launch_call(wl, call, kc, vc)
            outs.append(_outputs(pc))
            del pc
        torch.cuda.synchronize()
        runs.append((outs, kc, vc))
        H.log(f"{name}: run {rep} done ({len(wl.calls)} calls)")
    (o1, k1, v1), (o2, k2, v2) = runs
    for ci, (a, b) in enumerate(zip(o1, o2)):
        assert a.keys() == b.keys()
        for key in a:
            assert a[key].shape == b[key].shape, (ci, key)
            assert torch.equal(_bits(a[key]), _bits(b[key])), f"{name}: call {ci}: {key} differs between two identical runs"
    assert torch.equal(_bits(k1), _bits(k2)) and torch.equal(_bits(v1), _bits(v2)), "KV cache"
    H.log(f"{name}: bit-identical")


def test_gpu_determinism_packed_llama8b():
    _run_twice("packed_llama8b")


def test_gpu_determinism_chunked_128k():
    _run_twice("chunked_128k")
