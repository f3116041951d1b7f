"""The batch check (up_check_batch and the UP_DEBUG_CHECKS hook of
up_prefill_attn) on the GPU: a valid batch passes, and each broken
device-side precondition is reported by name.  Broken batches go to the
check only; the one passed to up_prefill_attn (cu_seqlens[0] = 1) stays
inside every array, so nothing reads out of bounds even without the check.
"""
import os

import numpy as np
import pytest
import torch

import workloads as W
from block_sparse_token_amd import binding as Bd
from block_sparse_token_amd import step as ST

pytestmark = pytest.mark.gpu


def _wl():
    return W.custom(seed=7, hidden_width=64, lengths=[40, 70, 5], ctxs=[0, 33, 20], Hq=8, Hkv=2,
                    D=128, dtype="bf16", block_size=32, p=0.9, theta=500000.0)


def _arrays(call):
    return dict(cu=call.cu_seqlens.copy(), ctx=call.ctx_lens.copy(), pos=call.positions.copy(),
                slots=call.slot_mapping.copy(), bt=call.block_table.copy())


def _check(a, num_pages, num_tokens=None):
    b = ST.make_batch(a["cu"], a["ctx"], a["pos"], a["slots"], a["bt"], num_tokens=num_tokens,
                      device="cuda")
    err = torch.empty(4, dtype=torch.int32, device="cuda")
    Bd.up_check_batch(b, num_pages, err)


def test_gpu_batch_check_accepts_valid_batches():
    wl = _wl()
    for call in wl.calls:
        _check(_arrays(call), wl.num_pages)
        _check(_arrays(call), 0)


def _broken(call, num_pages):
    a = _arrays(call)
    cases = []

    def case(name, msg, edit, pages=num_pages, num_tokens=None):
        b = {k: v.copy() for k, v in a.items()}
        b = edit(b) or b
        cases.append((name, msg, b, pages, num_tokens))

    def cu_start(b):
        b["cu"][0] = 1
    case("cu_start", "cu_seqlens[0] != 0", cu_start)

    def empty_segment(b):
        b["cu"][1] = b["cu"][2]
    case("empty_segment", "a segment has no token", empty_segment)
    case("cu_end", "cu_seqlens[S] > num_tokens", lambda b: None,
         num_tokens=int(a["cu"][-1]) - 1)

    def neg_ctx(b):
        b["ctx"][0] = -1
    case("neg_ctx", "negative ctx_lens", neg_ctx)

    def swapped(b):
        i = int(b["cu"][1]) + 3
        b["pos"][i], b["pos"][i + 1] = b["pos"][i + 1], b["pos"][i]
    case("swapped_positions", "positions not increasing", swapped)

    def below_ctx(b):
        b["pos"][int(b["cu"][1])] = int(b["ctx"][1]) - 1
    case("position_below_ctx", "positions not increasing", below_ctx)

    def neg_slot(b):
        b["slots"][5] = -1
    case("negative_slot", "slot out of range", neg_slot, pages=0)

    def big_slot(b):
        b["slots"][int(b["cu"][2])] = num_pages * 16
    case("slot_past_pool", "slot out of range", big_slot)

    def big_page(b):
        b["bt"][1, 0] = num_pages
    case("page_past_pool", "page id out of range", big_page)

    def neg_page(b):
        b["bt"][2, 1] = -3
    case("negative_page", "page id out of range", neg_page, pages=0)

    def short_table(b):
        b["bt"] = np.ascontiguousarray(b["bt"][:, :1])
    case("short_block_table", "block table", short_table)

    def no_table(b):
        b["bt"] = None
    case("missing_block_table", "block table", no_table)
    return cases


@pytest.mark.parametrize("which", range(12))
def test_gpu_batch_check_reports_each_violation(which):
    wl = _wl()
    call = wl.calls[0]
    name, msg, b, pages, nt = _broken(call, wl.num_pages)[which]
    print(f"broken batch: {name}", flush=True)
    with pytest.raises(Bd.UniprefillError, match=msg.replace("[", r"\[").replace("]", r"\]")):
        _check(b, pages, num_tokens=nt)


def test_gpu_debug_checks_hook_in_attention():
    import gpu_harness as H
    wl = _wl()
    call = wl.calls[0]
    kc, vc = H.make_caches(wl)
    ref = H.gpu_result(H.launch_call(wl, call, kc.clone(), vc.clone(), compact=False))
    old = os.environ.get("UP_DEBUG_CHECKS")
    os.environ["UP_DEBUG_CHECKS"] = "1"
    try:
        got = H.gpu_result(H.launch_call(wl, call, kc.clone(), vc.clone(), compact=False))
        assert np.array_equal(got["out"].view(np.uint16), ref["out"].view(np.uint16))
        a = _arrays(call)
        a["cu"][0] = 1
        b = ST.make_batch(a["cu"], a["ctx"], a["pos"], a["slots"], a["bt"], device="cuda")
        T, Hq, D = call.q.shape
        q = ST.stored_to_tensor(call.q)
        k, v = ST.stored_to_tensor(call.k), ST.stored_to_tensor(call.v)
        out = torch.empty_like(q)
        ws = torch.empty(Bd.up_attn_workspace_bytes(b, q.dtype, Hq, wl.Hkv, D), dtype=torch.uint8,
                         device="cuda")
        with pytest.raises(Bd.UniprefillError, match=r"cu_seqlens\[0\] != 0"):
            Bd.up_prefill_attn(b, q, k, v, kc.clone(), vc.clone(), out, ws, rope_theta=wl.theta)
    finally:
        if old is None:
            del os.environ["UP_DEBUG_CHECKS"]
        else:
            os.environ["UP_DEBUG_CHECKS"] = old


def test_gpu_debug_checks_whole_prompt_block_grid():
    """Whole-prompt scoring needs every scored segment's ctx_len on the block
    grid: the debug hook passes a batch whose only off-grid ctx_len belongs
    to an unscored segment (same results as without the hook) and names the
    violation when a scored one is off the grid."""
    import gpu_harness as H
    good = W.custom(seed=7064, hidden_width=64, lengths=[88, 200, 64, 5], ctxs=[512, 256, 0, 700],
                    flags=[True, True, True, False], Hq=8, Hkv=2, D=128, dtype="bf16",
                    block_size=64, p=0.6, theta=500000.0)
    bad = W.custom(seed=7065, hidden_width=64, lengths=[40, 70, 5], ctxs=[0, 33, 64], Hq=8, Hkv=2,
                   D=128, dtype="bf16", block_size=32, p=0.9, theta=500000.0)
    kc, vc = H.make_caches(good)
    ref = H.gpu_result(H.launch_call(good, good.calls[0], kc.clone(), vc.clone(),
                                     whole_prompt=True))
    old = os.environ.get("UP_DEBUG_CHECKS")
    os.environ["UP_DEBUG_CHECKS"] = "1"
    try:
        got = H.gpu_result(H.launch_call(good, good.calls[0], kc.clone(), vc.clone(),
                                         whole_prompt=True))
        for key in ("out", "scores", "keep", "index_map"):
            assert np.array_equal(np.asarray(got[key]).view(np.uint8),
                                  np.asarray(ref[key]).view(np.uint8)), key
        kb, vb = H.make_caches(bad)
        with pytest.raises(Bd.UniprefillError, match="not a multiple of block_size"):
            H.launch_call(bad, bad.calls[0], kb, vb, whole_prompt=True)
    finally:
        if old is None:
            del os.environ["UP_DEBUG_CHECKS"]
        else:
            os.environ["UP_DEBUG_CHECKS"] = old
