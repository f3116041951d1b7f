"""The no-allocation attention entry point against the ordinary one.

up_prefill_attn_noalloc takes no workspace: its scratch is the library's
per-GPU device array.  On the same inputs it must give bit for bit what
up_prefill_attn gives with a caller's workspace (attention output, log-sum-
exp, block mass, the KV caches it writes), on two calls in a row - the second
with a smaller batch, so stale scratch contents of the first call must not
leak into it - in both dtypes and under whole-prompt scoring, and it must
refuse, before launching anything, a call that needs more scratch than the
array holds.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _run(wl, noalloc, scope):
    from block_sparse_token_amd import binding as B
    from block_sparse_token_amd import step as ST
    from workloads import device as WD

    call = wl.calls[0]
    kc, vc = WD.make_caches(wl)
    batch = ST.make_batch(call.cu_seqlens, call.ctx_lens, call.positions, call.slot_mapping,
                          call.block_table)
    whole = scope == B.UP_SCOPE_PROMPT
    flags = torch.from_numpy(call.flags.astype(np.uint8)).cuda()
    cu_blocks = torch.empty(call.S + 1, dtype=torch.int32, device="cuda")
    B.up_block_offsets(batch, wl.block_size, cu_blocks, score_flags=flags, score_scope=scope)
    q, k, v = (WD.stored_to_tensor(x) for x in (call.q, call.k, call.v))
    out = torch.full_like(q, 7.0)
    lse = torch.full((call.T, wl.Hq), 7.0, dtype=torch.float32, device="cuda")
    mass = torch.full((call.num_blocks(wl.block_size, whole) * wl.Hq,), 7.0,
                      dtype=torch.float32, device="cuda")
    kw = dict(rope_theta=wl.theta, window=wl.window, score_flags=flags,
              block_size=wl.block_size, score_scope=scope, cu_blocks=cu_blocks,
              block_mass=mass, lse=lse)
    if noalloc:
        B.up_prefill_attn_noalloc(batch, q, k, v, kc, vc, out, **kw)
    else:
        nbytes = B.up_attn_workspace_bytes(batch, q.dtype, wl.Hq, wl.Hkv, wl.D, wl.block_size,
                                           scope)
        ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
        B.up_prefill_attn(batch, q, k, v, kc, vc, out, ws, **kw)
    torch.cuda.synchronize()
    return {"out": out, "lse": lse, "mass": mass, "k_cache": kc, "v_cache": vc}


CALLS = [
    # a larger batch first, then a smaller one on the same scratch
    [dict(lengths=[1500, 700, 90, 333], ctxs=[0, 64, 17, 0], Hq=32, Hkv=8, D=128, dtype="bf16",
          block_size=64, p=0.9, theta=500000.0, seed=61),
     dict(lengths=[100, 37], ctxs=[0, 0], Hq=32, Hkv=8, D=128, dtype="bf16", block_size=64,
          p=0.9, theta=500000.0, seed=62)],
    [dict(lengths=[400, 129], ctxs=[33, 0], Hq=4, Hkv=2, D=64, dtype="f32", block_size=16,
          p=0.9, seed=63),
     dict(lengths=[40, 1], ctxs=[0, 5], Hq=4, Hkv=2, D=64, dtype="f32", block_size=16, p=0.9,
          seed=64)],
]


@pytest.mark.parametrize("pair", range(len(CALLS)))
def test_gpu_noalloc_matches_workspace_entry(pair):
    from block_sparse_token_amd import binding as B
    for kw in CALLS[pair]:
        wl = W.custom(hidden_width=16, **kw)
        a = _run(wl, False, B.UP_SCOPE_SEGMENT)
        b = _run(wl, True, B.UP_SCOPE_SEGMENT)
        for key in a:
            assert torch.equal(_bits(a[key]), _bits(b[key])), (pair, kw["lengths"], key)


def test_gpu_noalloc_whole_prompt_then_smaller():
    from block_sparse_token_amd import binding as B
    for kw in (dict(lengths=[300, 90], ctxs=[1024, 192], flags=[True, True]),
               dict(lengths=[50], ctxs=[64], flags=[True])):
        wl = W.custom(hidden_width=16, Hq=8, Hkv=2, D=128, dtype="bf16", block_size=64, p=0.7,
                      theta=500000.0, seed=65, **kw)
        a = _run(wl, False, B.UP_SCOPE_PROMPT)
        b = _run(wl, True, B.UP_SCOPE_PROMPT)
        for key in a:
            assert torch.equal(_bits(a[key]), _bits(b[key])), (kw["lengths"], key)


def test_gpu_noalloc_refuses_more_than_its_scratch():
    """A batch whose scratch need passes the array's size is refused on the
    host with the sizes in the message; nothing is launched (the tensors are
    far smaller than the batch claims, and are left untouched)."""
    from block_sparse_token_amd import binding as B
    from block_sparse_token_amd import step as ST

    wl = W.custom(lengths=[64, 64], Hq=32, Hkv=8, D=128, dtype="bf16", block_size=64, p=0.9,
                  seed=66, hidden_width=16)
    call = wl.calls[0]
    n_claimed = 600000  # about 600K tokens: 75 MB of per-run score sums at 32 heads
    batch = ST.make_batch(call.cu_seqlens, call.ctx_lens, call.positions, call.slot_mapping,
                          call.block_table, num_tokens=n_claimed)
    need = B.up_attn_workspace_bytes(batch, torch.bfloat16, 32, 8, 128, 64)
    assert need > B.UP_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((call.T, 32, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((call.T, 8, 128), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((8, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    flags = torch.ones(call.S, dtype=torch.uint8, device="cuda")
    cu_blocks = torch.zeros(call.S + 1, dtype=torch.int32, device="cuda")
    mass = torch.zeros(64, dtype=torch.float32, device="cuda")
    with pytest.raises(B.UniprefillError, match="bytes of scratch"):
        B.up_prefill_attn_noalloc(batch, q, kv, kv, cache, cache.clone(), out, score_flags=flags,
                                  block_size=64, cu_blocks=cu_blocks, block_mass=mass)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
