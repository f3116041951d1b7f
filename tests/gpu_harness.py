"""GPU-side test helpers: stage a generated workload on the device, run the
library through its binding, and compare with the oracle.  The element-wise
checks and their tolerances live in ``parity_checks`` (NumPy only)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import workloads as W
from workloads import device as WD
from block_sparse_token_amd import binding as B
from block_sparse_token_amd import step as ST

from parity_checks import (BF16_OUT_ABS, BF16_SCORE_ABS, F32_REL, check_bf16_values,  # noqa: F401
                           check_out, check_scores, sample_rows)


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def make_caches(wl, device="cuda"):
    """Zeroed page pools plus any KV that exists before the first call."""
    return WD.make_caches(wl, device)


def read_back_cache(wl, kc, vc, pid, c):
    """K, V of a prompt's first c positions from the device pools (storage form)."""
    pg = torch.from_numpy(wl.prompt_pages[pid].astype(np.int64)).to(kc.device)
    lp = torch.arange(c, device=kc.device)
    page, off = pg[lp // W.PAGE_SIZE], lp % W.PAGE_SIZE
    return ST.tensor_to_stored(kc[page, :, off, :]), ST.tensor_to_stored(vc[page, :, off, :])


def assert_cache_unchanged_outside(before, after, slot_mapping):
    """Every cache row [page, :, offset, :] outside ``slot_mapping`` is
    bit-identical before and after a call (nothing wrote a wrong slot)."""
    sm = torch.from_numpy(np.asarray(slot_mapping, np.int64)).to(after.device)
    sm = sm[sm >= 0]
    page, off = sm // W.PAGE_SIZE, sm % W.PAGE_SIZE
    before[page, :, off, :] = after[page, :, off, :]
    same = torch.equal(before, after)
    assert same, "cache rows outside the call's slots changed"


def check_written_slots(wl, call, kc, vc, tokens):
    """The cache rows at the given tokens' slots hold the rotated key (bf16
    bound against the oracle's rotation) and the value (bit-exact)."""
    tokens = np.asarray(sorted(int(t) for t in tokens), np.int64)
    sm = call.slot_mapping[tokens].astype(np.int64)
    page = torch.from_numpy(sm // W.PAGE_SIZE).to(kc.device)
    off = torch.from_numpy(sm % W.PAGE_SIZE).to(kc.device)
    k_got = ST.tensor_to_stored(kc[page, :, off, :])
    v_got = ST.tensor_to_stored(vc[page, :, off, :])
    pos = call.positions[tokens].astype(np.int64)
    k_ref = oracle.apply_rope(W.to_f64(call.k[tokens], wl.dtype), pos, wl.theta)
    if wl.dtype == "bf16":
        check_bf16_values(W.to_f64(k_got, "bf16"), k_ref, "cache K at the call's slots")
    else:
        check_out("f32", k_got, k_ref, "cache K at the call's slots")
    assert np.array_equal(v_got, call.v[tokens]), "cache V at the call's slots"


def row_sources(call, device="cuda"):
    return WD.row_sources(call, device)


def launch_call(wl, call, kc, vc, *, with_lse=True, compact=True, device="cuda", flags=True,
                whole_prompt=False):
    batch = ST.make_batch(call.cu_seqlens, call.ctx_lens, call.positions, call.slot_mapping,
                          call.block_table, device=device)
    fl = torch.from_numpy(call.flags.astype(np.uint8)).to(device) if flags else None
    pc = ST.PrefillCall(batch=batch, q=ST.stored_to_tensor(call.q, device),
                        k=ST.stored_to_tensor(call.k, device), v=ST.stored_to_tensor(call.v, device),
                        k_cache=kc, v_cache=vc,
                        num_blocks=call.num_blocks(wl.block_size, whole_prompt),
                        flags=fl, block_size=wl.block_size, p=wl.p, rope_theta=wl.theta,
                        window=wl.window, rows=row_sources(call, device) if compact else [],
                        with_lse=with_lse, compact=compact,
                        score_scope=B.UP_SCOPE_PROMPT if whole_prompt else B.UP_SCOPE_SEGMENT)
    pc.launch()
    torch.cuda.synchronize()
    return pc


def gpu_result(pc):
    """Host copies of a launched call's outputs."""
    r = {"out": ST.tensor_to_stored(pc.out)}
    if pc.lse is not None:
        r["lse"] = pc.lse.cpu().numpy()
    if pc.flags is not None:
        r["scores"] = pc.scores.cpu().numpy()
        r["keep"] = pc.keep.cpu().numpy()
        r["cu_blocks"] = pc.cu_blocks.cpu().numpy()
        r["kept_blocks"] = pc.kept_blocks.cpu().numpy()
        if pc.compact:
            nk = int(pc.num_kept.item())
            r["num_kept"] = nk
            r["index_map"] = pc.index_map[:nk].cpu().numpy()
            r["cu_seqlens_out"] = pc.cu_seqlens_out.cpu().numpy()
            r["rows_out"] = {n: ST.tensor_to_stored(t[:nk]) for n, t in pc.rows_out.items()}
    return r


def check_selection_and_compaction(wl, call, g, whole_prompt=False):
    """Bit-exact: the oracle's top-p on the GPU scores, then the oracle's
    compaction on those keep masks, against the GPU outputs."""
    cb = g["cu_blocks"]
    assert np.array_equal(cb, call.cu_blocks(wl.block_size, whole_prompt))
    keeps = []
    for i, s in enumerate(call.segments):
        a, b = int(cb[i]), int(cb[i + 1])
        gk = g["keep"][a:b].astype(bool)
        if s.flagged:
            ok = oracle.topp_select(g["scores"][a:b], wl.p)
            assert np.array_equal(gk, ok), f"segment {i}: keep mask differs"
            assert np.all(g["scores"][a:b] >= 0)
        else:
            assert gk.all() and np.all(g["scores"][a:b] == 0)
        assert g["kept_blocks"][i] == gk.sum()
        keeps.append(gk)
    if "index_map" not in g:
        return
    from oracle.driver import row_tensors
    im, cu_out, rows_out = oracle.compact(call.cu_seqlens, [s.flagged for s in call.segments],
                                          wl.block_size, keeps, row_tensors(call),
                                          ctx=[s.ctx for s in call.segments],
                                          scope="prompt" if whole_prompt else "segment")
    assert np.array_equal(g["index_map"], im)
    assert np.array_equal(g["cu_seqlens_out"], cu_out)
    for name, ref in rows_out.items():
        assert np.array_equal(g["rows_out"][name].view(np.uint8), np.ascontiguousarray(ref).view(np.uint8)), name
