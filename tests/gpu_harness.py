"""GPU-side test helpers: stage a generated workload on the device, run the
library through its binding, and compare with the oracle.

Tolerances (element-wise):
  * float32 path: |gpu - oracle| <= 1e-5 * max(|oracle|, rms(oracle)) for
    attention outputs and scores (relative 1e-5, with the tensor's rms as the
    floor so elements near zero are not held to an impossible relative bound);
  * bf16 path: |gpu - oracle| <= 2e-2 for attention outputs, <= 1e-3 for
    normalised scores;
  * selection and compaction: bit-exact, with the oracle's selection run on
    the scores the GPU emitted.
"""
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

F32_REL = 1e-5
BF16_OUT_ABS = 2e-2
BF16_SCORE_ABS = 1e-3


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


def check_out(dtype, got_stored, ref, what="out"):
    got = W.to_f64(got_stored, dtype)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    if dtype == "bf16":
        worst = float(err.max()) if err.size else 0.0
        assert worst <= BF16_OUT_ABS, f"{what}: max abs err {worst:.3e} > {BF16_OUT_ABS}"
        return worst
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = F32_REL * np.maximum(np.abs(ref), rms)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond relative 1e-5; worst "
                           f"ratio {float((err / np.maximum(bound, 1e-300)).max()):.3f}")
    return float((err / np.maximum(bound, 1e-300)).max())


def check_scores(dtype, got, ref32):
    ref = ref32.astype(np.float64)
    g = got.astype(np.float64)
    err = np.abs(g - ref)
    if dtype == "bf16":
        assert err.max() <= BF16_SCORE_ABS, f"scores: max abs err {err.max():.3e}"
    else:
        rms = float(np.sqrt(np.mean(ref * ref)))
        bound = F32_REL * np.maximum(np.abs(ref), rms)
        assert np.all(err <= bound), f"scores: worst ratio {float((err / bound).max()):.3f}"
    assert np.all(g >= 0)


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
