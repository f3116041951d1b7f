"""Benchmark: packed prefill tokens/s of the operator on one MI355X.

One step = the whole hot path over one batch: rotary embedding and paged
KV-cache write, attention with the fused block mass, block scores with top-p
selection, and compaction of the kept rows (every call of a chunked
workload, and the sliding-window second layer where the workload has one).
Inputs are synthetic and resident on the GPU before timing starts.

The default run prints one JSON line for the headline workload - the
Llama-3.1-8B-shaped packed prefill (16 prompts, lengths uniform in
[512, 8192] from seed 2, about 70K tokens; 32 query / 8 KV heads x 128,
bf16; rotary base 500000; block 64, top-p 0.95; hidden width 4096) - and
the same measurements of the four other workloads under ``configs`` (the
tiny fp32 chunked batch, the chunked 128K prompt, the decode + prefill
step, the selection followed by a sliding-window layer).

``roofline`` covers the attention kernel (the dominant one): algorithmic
flops 4 * D * Hq * (visible query/key pairs) per launch over its average
duration, timed with HIP events the library records around that kernel on
its stream; ``attainable`` beside the published ``peak`` is what a plain
bf16 matrix-core loop sustains on the same GPU in the same run.  Every other
pass is set against HBM with the bytes it must move (``passes``), and the
rotary/cache-write and compaction passes also against a plain streaming copy
of the same bytes per call (``copy_us_same_bytes``, ``frac_of_copy``): at a
few tens of MB a copy's own launch and ramp keep it well below the HBM peak.
``cpu_baseline`` is the float64 NumPy oracle timed on this host on a bounded
sample of the same workload, scaled to the whole workload by visible pairs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PEAK_F32_VECTOR_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
WORKLOAD = "packed_llama8b"
METRIC = "packed prefill tokens/s (attn+score+select+compact) + % MFMA/HBM roofline"
OTHER_WORKLOADS = ("small_chunked_fp32", "chunked_128k", "mixed_decode_prefill",
                   "swa_after_selection")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="throughput against the number of packed prompts, and packed vs "
                         "bin-packed rows vs padded layouts of the headline batch")
    ap.add_argument("--p", type=float, default=None,
                    help="with --propagation: top-p of the selection instead of the workload's "
                         "0.95 (shows how the later-layer saving follows the kept fraction)")
    ap.add_argument("--whole-prompt", action="store_true",
                    help="with --workload chunked_128k: earlier chunks unscored, the final chunk "
                         "scores every block of the prompt (cached ones included)")
    ap.add_argument("--propagation", action="store_true",
                    help="time one later layer's linear maps on all vs the kept tokens of the "
                         "headline batch")
    ap.add_argument("--workload", default="all", choices=("all", WORKLOAD) + OTHER_WORKLOADS,
                    help="all (default): the headline workload's bench line with every other "
                         "workload under 'configs'; or one workload, timed over all its calls")
    ap.add_argument("--library", action="store_true",
                    help="also time torch's flash attention on the headline batch (reference)")
    return ap.parse_args()


def visible_pairs(cu, ctx, positions, window):
    """(query, key) pairs the attention computes for one call: cached keys at
    positions 0..c-1 plus the segment's own keys, key position <= query
    position, and within the window when there is one."""
    total = 0
    for s in range(len(ctx)):
        a, b, c = int(cu[s]), int(cu[s + 1]), int(ctx[s])
        pos = np.asarray(positions[a:b], dtype=np.int64)
        keys = np.concatenate([np.arange(c, dtype=np.int64), pos])
        hi = np.searchsorted(keys, pos, side="right")
        lo = np.searchsorted(keys, pos - window, side="right") if window > 0 else 0
        total += int(np.sum(hi - lo))
    return total


# ---------------------------------------------------------------------------
# every workload: staging, timing, algorithmic work, oracle sample
# ---------------------------------------------------------------------------
# (name, label of the configuration it stands for, steps cap, warm-up cap)
CONFIGS = [("packed_llama8b", "C2", None, None), ("small_chunked_fp32", "C1", 20, 3),
           ("chunked_128k", "C3", 3, 1), ("mixed_decode_prefill", "C4", 10, 2),
           ("swa_after_selection", "C5", 3, 1)]
DESCRIBE = {
    "small_chunked_fp32": "tiny packed prefill, fp32: prompts {37,100,64,255}, 2+2 heads x 64, "
                          "block 16, top-p 0.9, chunk 64 (4 calls over the paged cache)",
    "packed_llama8b": "Llama-3.1-8B-shaped packed prefill: 16 prompts U{512..8192} (seed 2), "
                      "32/8 heads x 128, bf16, rope 5e5, block 64, top-p 0.95, hidden 4096",
    "chunked_128k": "one 131072-token prompt in 16 chunks of 8192 over a paged cache, 32/8 x 128, "
                    "bf16, rope 5e5, block 128, top-p 0.9, hidden 4096",
    "mixed_decode_prefill": "continuous-batching step: 256 decodes (context U{1024..32768}) + "
                            "FCFS prefill chunks to 8192 tokens, 32/8 x 128, bf16, block 64, "
                            "top-p 0.95 on the prefill",
    "swa_after_selection": "8 prompts U{8192..32768}: full-attention layer with scoring, block "
                           "64, top-p 0.9, compaction of hidden/positions/slots/layer-2 q,k,v, "
                           "then sliding-window (4096) attention on the kept tokens",
}


class Staged:
    """A workload's calls staged on the GPU (inputs resident before timing)."""

    def __init__(self, torch, wl, whole=False):
        from workloads import device as WD
        from block_sparse_token_amd import binding as B
        from block_sparse_token_amd import step as ST

        self.wl = wl
        self.kc, self.vc = WD.make_caches(wl)
        self.calls = []
        for ci, call in enumerate(wl.calls):
            batch = ST.make_batch(call.cu_seqlens, call.ctx_lens, call.positions,
                                  call.slot_mapping, call.block_table)
            final = ci == len(wl.calls) - 1
            fl = call.flags.astype(np.uint8)
            if whole:  # earlier chunks pass through; the final one scores the prompt
                fl = fl * np.uint8(final)
            self.calls.append((call, ST.PrefillCall(
                batch=batch, q=WD.stored_to_tensor(call.q), k=WD.stored_to_tensor(call.k),
                v=WD.stored_to_tensor(call.v), k_cache=self.kc, v_cache=self.vc,
                num_blocks=call.num_blocks(wl.block_size, whole and final),
                flags=torch.from_numpy(fl).cuda(), block_size=wl.block_size, p=wl.p,
                rope_theta=wl.theta, window=wl.window, rows=WD.row_sources(call),
                score_scope=B.UP_SCOPE_PROMPT if whole and final else B.UP_SCOPE_SEGMENT)))
        self.layer2 = None
        if wl.layer2:
            # the second layer runs on the compacted rows at full row capacity
            # (its token count stays on the device)
            pc = self.calls[0][1]
            S = len(self.calls[0][0].segments)
            batch2 = B.Batch(pc.cu_seqlens_out, torch.zeros(S, dtype=torch.int32, device="cuda"),
                             pc.rows_out["positions"], pc.rows_out["slot_mapping"], None)
            self.layer2 = ST.PrefillCall(batch=batch2, q=pc.rows_out["q2"], k=pc.rows_out["k2"],
                                         v=pc.rows_out["v2"], k_cache=torch.zeros_like(self.kc),
                                         v_cache=torch.zeros_like(self.vc), num_blocks=1,
                                         flags=None, block_size=wl.block_size, p=wl.p,
                                         rope_theta=wl.layer2["theta"],
                                         window=wl.layer2["window"])


def time_workload(torch, st, steps, warmup, flush=None):
    """Time ``steps`` steps (every call, then the second layer if any) after
    ``warmup`` untimed ones: ``ms_per_step`` is the wall time of the steps
    run back to back (no event, no synchronisation between them; one
    synchronisation before and one after).  Then a second run of the same
    steps, each synchronised, gives HIP-event times of the rotary/cache-write
    kernel, the attention kernel (both recorded by the library on its
    stream), and of each stage: the attention call (block offsets,
    rotary/cache write, work plan, attention, block mass), scores with top-p,
    compaction.  ``flush``: a buffer written before every step (outside the
    timed stages) so no pass finds its inputs in the 256 MB Infinity Cache;
    with it, ``ms_per_step`` comes from the synchronised run."""
    from block_sparse_token_amd import binding as B

    stream = torch.cuda.current_stream()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)  # creates the event the library records again
        return e

    def one_step(rec):
        for call, pc in st.calls:
            if rec is not None:
                re, ae = (ev(), ev()), (ev(), ev())
                B.up_profile_rope_events(*re)
                B.up_profile_attn_events(*ae)
                e = [ev()]
            pc.attention()
            if rec is not None:
                e.append(ev())
            if pc.flags is not None:
                pc.score_select_stage()
            if rec is not None:
                e.append(ev())
            if pc.flags is not None and pc.compact:
                pc.compact_stage()
            if rec is not None:
                e.append(ev())
                rec.append(("call", re, ae, e))
        if st.layer2 is not None:
            if rec is not None:
                re, ae = (ev(), ev()), (ev(), ev())
                B.up_profile_rope_events(*re)
                B.up_profile_attn_events(*ae)
                e = [ev()]
            st.layer2.attention()
            if rec is not None:
                e.append(ev())
                rec.append(("layer2", re, ae, e))
        if rec is not None:
            B.up_profile_rope_events()
            B.up_profile_attn_events()

    for _ in range(warmup):
        one_step(None)
    torch.cuda.synchronize()
    back_to_back = None
    if flush is None:
        t0 = time.perf_counter()
        for _ in range(steps):
            one_step(None)
        torch.cuda.synchronize()
        back_to_back = (time.perf_counter() - t0) * 1e3 / steps
    recs, wall = [], 0.0
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 255)
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        one_step(recs)
        torch.cuda.synchronize()
        wall += time.perf_counter() - t0
    K = float(steps)
    t = {"ms_per_step": back_to_back if back_to_back is not None else wall * 1e3 / K,
         "ms_per_step_synchronised": wall * 1e3 / K}
    for kind in ("call", "layer2"):
        rs = [r for r in recs if r[0] == kind]
        if not rs:
            continue
        pre = "" if kind == "call" else "layer2_"
        t[pre + "rope_ms"] = sum(a.elapsed_time(b) for _, (a, b), _, _ in rs) / K
        t[pre + "attn_ms"] = sum(a.elapsed_time(b) for _, _, (a, b), _ in rs) / K
        t[pre + "attn_stage_ms"] = sum(e[0].elapsed_time(e[1]) for *_, e in rs) / K
        if kind == "call":
            t["score_select_ms"] = sum(e[1].elapsed_time(e[2]) for *_, e in rs) / K
            t["compact_ms"] = sum(e[2].elapsed_time(e[3]) for *_, e in rs) / K
    return t


def _pass(nbytes, ms):
    gbs = nbytes / (ms * 1e-3) / 1e9 if ms > 0 else None
    return {"bytes": int(nbytes), "us": ms * 1e3, "GB/s": gbs,
            "frac": gbs / PEAK_HBM_GBS if gbs else None}


def workload_metrics(st, t):
    """Throughput, the attention pass against the matrix (or vector) peak,
    and every other pass against HBM, from algorithmic work only: visible
    (query, key) pairs, bytes each pass must move."""
    wl = st.wl
    bf16 = wl.dtype == "bf16"
    e_b = 2 if bf16 else 4
    pairs = sum(visible_pairs(c.cu_seqlens, c.ctx_lens, c.positions, wl.window)
                for c, _ in st.calls)
    flops = 4.0 * wl.D * wl.Hq * pairs
    T_all = sum(c.T for c, _ in st.calls)
    S_all = sum(c.S for c, _ in st.calls)
    NB_all = sum(int(pc.cu_blocks[-1].item()) for _, pc in st.calls)
    kept = [int(pc.num_kept.item()) for _, pc in st.calls]
    row_b = sum(src[0].numel() * src.element_size() for _, src in st.calls[0][1].rows)
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_VECTOR_TFLOPS
    tokens = T_all
    m = {"calls": len(st.calls), "tokens": T_all, "kept_tokens": int(sum(kept)),
         "blocks": NB_all, "segments": S_all}
    if wl.name == "mixed_decode_prefill":
        c = st.calls[0][0]
        dec = [i for i, s in enumerate(c.segments) if not s.flagged]
        tokens = int(sum(s.n for s in c.segments if s.flagged))
        dec_keys = sum(c.segments[i].ctx + c.segments[i].n for i in dec)
        dec_bytes = dec_keys * wl.Hkv * wl.D * e_b * 2 + len(dec) * wl.Hq * wl.D * e_b * 2
        pre_pairs = pairs - sum(c.segments[i].ctx + 1 for i in dec)
        floor_ms = (dec_bytes / (PEAK_HBM_GBS * 1e9) +
                    4.0 * wl.D * wl.Hq * pre_pairs / (PEAK_BF16_TFLOPS * 1e12)) * 1e3
        m["decode_part"] = {
            "decode_segments": len(dec), "decode_kv_bytes": dec_bytes,
            "decode_kv_GB/s_if_alone": dec_bytes / (t["attn_ms"] * 1e-3) / 1e9,
            "prefill_pairs": pre_pairs,
            "serial_floor_ms": floor_ms, "attention_vs_serial_floor": floor_ms / t["attn_ms"],
            "note": "the attention launch serves both parts at once; the floor is the decode KV "
                    "read at 8 TB/s plus the prefill products at 2.5 PFLOP/s"}
        m["all_tokens_per_s"] = T_all / (t["ms_per_step"] * 1e-3)
    m["tokens_counted"] = tokens
    m["ms_per_step"] = t["ms_per_step"]
    m["ms_per_step_synchronised"] = t["ms_per_step_synchronised"]
    m["tokens_per_s"] = tokens / (t["ms_per_step"] * 1e-3)
    att = flops / (t["attn_ms"] * 1e-3) / 1e12
    m["attention"] = {"kernel": "attn_bf16_kernel" if bf16 else "attn_f32_kernel",
                      "bound": "mfma" if bf16 else "alu", "pairs": pairs, "flops": flops,
                      "ms": t["attn_ms"], "TFLOP/s": att, "peak": peak, "frac": att / peak}
    a1_b = T_all * (4 * wl.Hkv * wl.D * e_b + 8)
    sel_b = 4 * wl.Hq * NB_all + 4 * NB_all + 4 * NB_all + NB_all + 4 * S_all
    comp_b = sum(k * (2 * row_b + 4) for k in kept) + NB_all
    m["passes"] = {
        "rope_kv_write": _pass(a1_b, t["rope_ms"]),
        "scores_select": dict(_pass(sel_b, t["score_select_ms"]), bound="latency"),
        "compact": _pass(comp_b, t["compact_ms"]),
        "plan_offsets_mass_us": (t["attn_stage_ms"] - t["rope_ms"] - t["attn_ms"]) * 1e3,
    }
    if st.layer2 is not None:
        nk = kept[0]
        pc = st.calls[0][1]
        cu2 = pc.cu_seqlens_out.cpu().numpy()
        pos2 = pc.rows_out["positions"][:nk].cpu().numpy()
        pairs2 = visible_pairs(cu2, np.zeros(len(cu2) - 1, dtype=np.int64), pos2,
                               wl.layer2["window"])
        f2 = 4.0 * wl.D * wl.Hq * pairs2
        a2 = f2 / (t["layer2_attn_ms"] * 1e-3) / 1e12
        m["swa_layer"] = {"kept_tokens": nk, "window": wl.layer2["window"], "pairs": pairs2,
                          "flops": f2, "ms": t["layer2_attn_ms"], "TFLOP/s": a2,
                          "frac": a2 / PEAK_BF16_TFLOPS,
                          "rope_kv_write": _pass(nk * (4 * wl.Hkv * wl.D * e_b + 8),
                                                 t["layer2_rope_ms"])}
    return m


def oracle_sample(wl, budget_s, layer2_pairs=None):
    """The float64 oracle on a bounded sample of the workload, timed on this
    host's cores: whole segments, each in one pass (no cache needed), picked
    as the workload allows; the whole-workload rate is the sample's rate
    scaled by visible (query, key) pairs (its cost grows with them, and the
    second layer's are included for the sliding-window workload)."""
    import oracle
    from oracle import driver
    from oracle.prefill import default_threads
    from workloads import to_f64

    threads = default_threads()
    dt = wl.dtype

    def seg_args(call, si, extra_rows=()):
        s = call.segments[si]
        a, b = int(call.cu_seqlens[si]), int(call.cu_seqlens[si + 1])
        rows = {"hidden": call.hidden[a:b], "positions": call.positions[a:b],
                "slot_mapping": call.slot_mapping[a:b]}
        for r in extra_rows:
            rows[r] = call.extra[r][a:b]
        return dict(segments=[(0, 0, s.n, s.flagged)], q=to_f64(call.q[a:b], dt),
                    k=to_f64(call.k[a:b], dt), v=to_f64(call.v[a:b], dt),
                    positions=call.positions[a:b], cu_seqlens=[0, s.n], Hq=wl.Hq, Hkv=wl.Hkv,
                    D=wl.D, theta=wl.theta, window=wl.window, block_size=wl.block_size,
                    p=wl.p, cache=oracle.KVCacheModel(), rows=rows, threads=threads)

    def seg_pairs(n):
        return n * (n + 1) // 2

    total_pairs = sum(visible_pairs(c.cu_seqlens, c.ctx_lens, c.positions, wl.window)
                      for c in wl.calls)
    tokens = sum(c.T for c in wl.calls)
    spent, s_tok, s_pairs, what = 0.0, 0, 0, ""
    if wl.name == "small_chunked_fp32":
        t0 = time.perf_counter()
        driver.run_workload(wl, threads=threads)
        spent = time.perf_counter() - t0
        s_tok, s_pairs = tokens, total_pairs
        what = "the whole workload (4 chunked calls)"
    elif wl.layer2 is None:
        call = wl.calls[0]
        cand = [i for i, s in enumerate(call.segments) if s.ctx == 0 and s.flagged]
        if wl.name == "mixed_decode_prefill":
            c = wl.calls[0]
            tokens = int(sum(s.n for s in c.segments if s.flagged))
            total_pairs = sum(s.n * s.ctx + seg_pairs(s.n) for s in c.segments if s.flagged)
        lens = np.array([call.segments[i].n for i in cand])
        wmean = float((lens ** 2).sum() / lens.sum())
        used = []
        for j in np.argsort(np.abs(lens - wmean)):
            si = cand[int(j)]
            args = seg_args(call, si)
            t0 = time.perf_counter()
            oracle.run_call(**args)
            spent += time.perf_counter() - t0
            n = call.segments[si].n
            s_tok += n
            s_pairs += seg_pairs(n)
            used.append(n)
            if spent >= budget_s:
                break
        what = (f"{len(used)} whole prompt segment(s) of the first call (lengths {used}), "
                "each in one pass")
        if wl.name == "mixed_decode_prefill":
            what += "; rate in prefill tokens, scaled by the prefill's pairs"
    else:
        call = wl.calls[0]
        si = int(np.argmin([s.n for s in call.segments]))
        t0 = time.perf_counter()
        r1 = oracle.run_call(**seg_args(call, si, ("q2", "k2", "v2")))
        ro, cu2 = r1["rows_out"], r1["cu_seqlens_out"]
        n2 = int(cu2[-1])
        oracle.run_call(segments=[(0, 0, n2, False)], q=to_f64(ro["q2"], dt),
                        k=to_f64(ro["k2"], dt), v=to_f64(ro["v2"], dt),
                        positions=ro["positions"], cu_seqlens=cu2, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                        theta=wl.layer2["theta"], window=wl.layer2["window"],
                        block_size=wl.block_size, p=wl.p, cache=oracle.KVCacheModel(),
                        score=False, select=False, threads=threads)
        spent = time.perf_counter() - t0
        n = call.segments[si].n
        w2 = wl.layer2["window"]
        p2 = visible_pairs(cu2, [0], ro["positions"], w2)
        s_tok, s_pairs = n, seg_pairs(n) + p2
        # the whole workload's second-layer pairs: from the GPU's compaction,
        # which the parity tests hold bit-exact to the oracle's
        total_pairs += int(layer2_pairs)
        what = (f"the shortest prompt (length {n}) through the scored layer, compaction and "
                f"the sliding-window layer on its {n2} kept tokens")
    rate = s_tok / spent
    scaled = tokens / (spent * total_pairs / s_pairs)
    return {"value": scaled, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}: {s_tok} tokens, {spent:.1f} s of float64 NumPy on {threads} "
                      f"threads ({rate:.0f} tokens/s on the sample), scaled to the whole "
                      f"workload by visible (query, key) pairs ({s_pairs} in the sample, "
                      f"{total_pairs} in the workload)",
            "sample_tokens_per_s": rate, "sample_seconds": spent}


def kernel_code_hash(path):
    """sha256 of a source file with its comments and whitespace removed, and
    of the file's own compile flags when it has any, so that a profile stays
    matched to a kernel whose comments were edited and to no other build."""
    from block_sparse_token_amd.build import FILE_FLAGS
    txt = open(path).read()
    txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
    txt = re.sub(r"//[^\n]*", " ", txt)
    flags = FILE_FLAGS.get(os.path.basename(path), [])
    key = " ".join(txt.split()) + (" | " + " ".join(flags) if flags else "")
    return hashlib.sha256(key.encode()).hexdigest()


def traffic_from_profile(src_hash, name="attn_bf16_packed_llama8b_counters.md"):
    """HBM bytes per launch of a kernel from its committed counter summary
    under profiles/, if the summary was taken on the current kernel source;
    else None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel code sha256[^:\n]*: ([0-9a-f]{64})", txt)
    t = re.search(r"HBM bytes per launch \(scaled\)[^:\n]*: ([0-9.eE+]+)", txt)
    if not m or not t or m.group(1) != src_hash:
        return None
    return float(t.group(1))


def attainable_peaks(torch, B, stream):
    """What the chip sustains: a bf16 matrix-core loop (2048 workgroups of
    four waves, about 10 ms a launch) and a 1 GiB device-to-device copy,
    each the median of several event-timed launches after a warm-up."""
    wgs, iters = 2048, 16384
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    flops = wgs * 4.0 * iters * 4 * 32768
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.median(ms))

    mfma_ms = timed(lambda: B.up_peak_mfma_bf16(wgs, iters, sink), 5)
    copy_ms = timed(lambda: B.up_peak_copy(src, dst), 10)
    if not torch.equal(dst[:: 1 << 20], src[:: 1 << 20]):
        raise RuntimeError("peak copy produced wrong data")
    del src, dst, sink
    return {"mfma_bf16_TFLOP/s": flops / (mfma_ms * 1e-3) / 1e12,
            "hbm_copy_GB/s": 2.0 * n / (copy_ms * 1e-3) / 1e9,
            "method": "up_peak_mfma_bf16 (2048 x 4 waves, 4 independent 32x32x16 chains) and "
                      "up_peak_copy (1 GiB read + 1 GiB written), medians of event-timed launches"}


def copy_us_same_bytes(torch, B, stream, nbytes, cache):
    """Median event-timed duration (us) of the library's streaming copy
    (``up_peak_copy``) moving ``nbytes`` in all, half read and half written:
    what a plain copy of a pass's size sustains, launch and ramp included."""
    half = max(4096, (int(nbytes) // 2) // 4096 * 4096)
    if half not in cache:
        src = torch.ones(half // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        B.up_peak_copy(src, dst)
        torch.cuda.synchronize()
        ms = []
        for _ in range(10):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            B.up_peak_copy(src, dst)
            b.record(stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        if not torch.equal(dst[:: 1 << 16], src[:: 1 << 16]):
            raise RuntimeError("peak copy produced wrong data")
        del src, dst
        cache[half] = float(np.median(ms)) * 1e3
    return cache[half]


def add_copy_comparison(torch, B, stream, m, cache):
    """For each HBM pass of a workload: the time a plain copy of the same
    bytes per call takes (times the number of calls) and the pass's rate as
    a fraction of that copy's."""
    calls = m["calls"]
    for name in ("rope_kv_write", "compact"):
        p = m["passes"][name]
        if not p["bytes"] or not p["us"]:
            continue
        c_us = calls * copy_us_same_bytes(torch, B, stream, p["bytes"] / calls, cache)
        p["copy_us_same_bytes"] = c_us
        p["frac_of_copy"] = c_us / p["us"]


def headline_call(torch, p=None):
    """The headline workload's one call, staged on the GPU: inputs, caches,
    batch metadata, and the hidden states, positions and KV slots to compact
    (top-p ``p`` instead of the workload's when given)."""
    import workloads as W
    from block_sparse_token_amd import step as ST

    wl = W.make(WORKLOAD)
    call = wl.calls[0]
    dev = "cuda"
    kc = torch.zeros((wl.num_pages, wl.Hkv, W.PAGE_SIZE, wl.D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    batch = ST.make_batch(call.cu_seqlens, call.ctx_lens, call.positions, call.slot_mapping,
                          call.block_table, device=dev)
    rows = [("hidden", ST.stored_to_tensor(call.hidden, dev)),
            ("positions", torch.from_numpy(call.positions.astype(np.int32)).to(dev)),
            ("slot_mapping", torch.from_numpy(call.slot_mapping.astype(np.int32)).to(dev))]
    pc = ST.PrefillCall(batch=batch, q=ST.stored_to_tensor(call.q, dev),
                        k=ST.stored_to_tensor(call.k, dev), v=ST.stored_to_tensor(call.v, dev),
                        k_cache=kc, v_cache=vc, num_blocks=call.num_blocks(wl.block_size),
                        flags=torch.from_numpy(call.flags.astype(np.uint8)).to(dev),
                        block_size=wl.block_size, p=wl.p if p is None else p,
                        rope_theta=wl.theta, rows=rows)
    return wl, call, pc


def library_attention(torch, wl, call, pc, steps):
    """Reference point outside the path: PyTorch's fused flash attention
    (scaled_dot_product_attention held to its flash backend, so it never
    falls back to the unfused math) on the same q, k, v, one causal call per
    prompt (it has no packed variable-length form), timed back to back; and
    the longest prompt alone, which fills the chip by itself.  No RoPE, no
    paged cache and no block mass there."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    try:
        cu = [int(c) for c in call.cu_seqlens]
        segs = []
        for a, b in zip(cu[:-1], cu[1:]):
            segs.append(tuple(x[a:b].transpose(0, 1).unsqueeze(0).contiguous()
                              for x in (pc.q, pc.k, pc.v)))
        longest = max(range(len(segs)), key=lambda i: cu[i + 1] - cu[i])

        def run(idx):
            for i in idx:
                q, k, v = segs[i]
                F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)

        out = {"what": "torch scaled_dot_product_attention, flash backend only, one causal call "
                       "per prompt on the same q/k/v (no RoPE, cache or block mass); reference "
                       "only, not part of the path"}
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            for name, idx in (("all_prompts_serial", list(range(len(segs)))),
                              ("longest_prompt", [longest])):
                run(idx)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    run(idx)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / steps
                pairs = sum((cu[i + 1] - cu[i]) * (cu[i + 1] - cu[i] + 1) / 2 for i in idx)
                out[name] = {"prompts": len(idx), "ms": ms,
                             "TFLOP/s": 4.0 * wl.D * wl.Hq * pairs / (ms * 1e-3) / 1e12}
        del segs
        return out
    except Exception as ex:  # a reference only: report, never fail the bench
        return {"error": f"{type(ex).__name__}: {str(ex)[:200]}"}


def run_propagation(args):
    """Payoff of the selection in the later layers: one Llama-3.1-8B-shaped
    later layer of a linear/full hybrid - query/key/value projection 4096 ->
    6144, causal linear attention (phi = elu + 1) over each prompt's rows,
    output projection 4096 -> 4096 of its result, SwiGLU gate and up
    projections 4096 -> 2 x 14336 and down projection 14336 -> 4096; random
    bf16 weights - runs on all tokens of the headline batch and on the tokens
    its selection kept (the compacted hidden states and per-prompt kept
    counts, with the kept total read on the device).  The MLP takes the
    hidden states as its input (no norms or residuals: their cost does not
    change the comparison).  Prints one JSON line."""
    import torch
    import oracle
    from block_sparse_token_amd import binding as B
    from oracle.prefill import default_threads

    wl, call, pc = headline_call(torch, args.p)
    pc.launch()
    torch.cuda.synchronize()
    T = call.T
    kept = int(pc.num_kept.item())
    H, D = wl.hidden_width, wl.D
    QKV, MLP = (wl.Hq + 2 * wl.Hkv) * D, 14336
    g = torch.Generator(device="cuda")
    g.manual_seed(77)

    def weight(n, k):
        return (torch.randn((n, k), generator=g, device="cuda") * (k ** -0.5)).to(torch.bfloat16)

    w_qkv, w_o = weight(QKV, H), weight(H, H)
    w_gate, w_up = weight(MLP, H), weight(MLP, H)
    w_gu = B.interleave_gate_up(w_gate, w_up)
    w_down = weight(H, MLP)
    x_all = dict(pc.rows)["hidden"]
    x_kept = pc.rows_out["hidden"]
    qkv = torch.empty((T, QKV), dtype=torch.bfloat16, device="cuda")
    attn = torch.zeros((T, wl.Hq, D), dtype=torch.bfloat16, device="cuda")
    q_v = qkv[:, : wl.Hq * D].view(T, wl.Hq, D)
    k_v = qkv[:, wl.Hq * D: (wl.Hq + wl.Hkv) * D].view(T, wl.Hkv, D)
    v_v = qkv[:, (wl.Hq + wl.Hkv) * D:].view(T, wl.Hkv, D)
    o = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    hmid = torch.empty((T, MLP), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    maps = [("qkv", H, QKV), ("linear_attention", None, None), ("o", H, H),
            ("gate_up_swiglu", H, 2 * MLP), ("down", MLP, H)]
    stream = torch.cuda.current_stream()
    cu_all = pc.batch.cu_seqlens
    # chunk-parallel linear attention: its workspace, allocated once
    la_ws = torch.empty(B.up_linear_attn_workspace_bytes(T, len(call.segments), wl.Hq),
                        dtype=torch.uint8, device="cuda")

    def layer(x, rows_dev, cu, ev=None):
        args_ = [(x, w_qkv, qkv, B.UP_ACT_NONE), None, (attn.view(T, H), w_o, o, B.UP_ACT_NONE),
                 (x, w_gu, hmid, B.UP_ACT_SWIGLU), (hmid, w_down, y, B.UP_ACT_NONE)]
        for j, a_ in enumerate(args_):
            if ev is not None:
                ev[j][0].record(stream)
            if a_ is None:
                B.up_linear_attn_bf16(cu, q_v, k_v, v_v, attn, workspace=la_ws)
            else:
                inp, w, out, act = a_
                B.up_linear_bf16(inp, w, out, rows_in_use=rows_dev, act=act)
            if ev is not None:
                ev[j][1].record(stream)

    def timed(x, rows_dev, cu):
        for _ in range(args.warmup):
            layer(x, rows_dev, cu)
        torch.cuda.synchronize()
        evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in maps] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for ev in evs:
            layer(x, rows_dev, cu, ev)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / args.steps
        per_map = [float(np.mean([ev[j][0].elapsed_time(ev[j][1]) for ev in evs]))
                   for j in range(len(maps))]
        return wall, per_map

    wall_all, ms_all = timed(x_all, None, cu_all)
    wall_kept, ms_kept = timed(x_kept, pc.num_kept, pc.cu_seqlens_out)
    res_maps = {}
    # linear attention, recurrent-form flops per token: the state update per
    # KV head, numerator and denominator per query head
    la_per_tok = 2.0 * wl.Hkv * D * D + wl.Hq * (2.0 * D * D + 2.0 * D)
    for j, (name, K, N) in enumerate(maps):
        if K is None:
            f_all, f_kept = la_per_tok * T, la_per_tok * kept
        else:
            f_all, f_kept = 2.0 * T * K * N, 2.0 * kept * K * N
        res_maps[name] = {"K": K, "N": N, "flops_all": f_all, "ms_all": ms_all[j],
                          "ms_kept": ms_kept[j],
                          "TFLOP/s_all": f_all / (ms_all[j] * 1e-3) / 1e12,
                          "TFLOP/s_kept": f_kept / (ms_kept[j] * 1e-3) / 1e12,
                          "frac_all": f_all / (ms_all[j] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    flops_all = oracle.later_layer_flops(T, H, QKV, MLP) + la_per_tok * T
    flops_kept = oracle.later_layer_flops(kept, H, QKV, MLP) + la_per_tok * kept
    dominant = max(res_maps, key=lambda k: res_maps[k]["ms_all"])
    dm = res_maps[dominant]
    res = {
        "metric": "later layer on the kept tokens vs all tokens (ms per layer)",
        "value": wall_kept, "unit": "ms", "higher_is_better": False, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "one Llama-3.1-8B-shaped later linear-attention layer (4096 -> 6144, "
                               "causal linear attention 32/8 heads x 128 in parts of 1024 rows, 4096 -> 4096, SwiGLU "
                               "4096 -> 2 x 14336, 14336 -> 4096) on the packed prefill of "
                               f"{T} tokens, {kept} kept by top-p {pc.p} (block 64)",
                   "rows_all": T, "rows_kept": kept},
        "layer_ms_all": wall_all, "layer_ms_kept": wall_kept,
        "time_saved_frac": 1.0 - wall_kept / wall_all,
        "flops_all": flops_all, "flops_kept": flops_kept,
        "flops_saved_frac": 1.0 - flops_kept / flops_all,
        "maps": res_maps,
        "roofline": {"bound": "mfma", "kernel": "linear_bf16_kernel", "map": dominant,
                     "achieved": dm["TFLOP/s_all"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": dm["frac_all"],
                     "traffic": traffic_from_profile(
                         kernel_code_hash(os.path.join(ROOT, "block_sparse_token_amd", "csrc",
                                                       "linear.hip")),
                         "linear_bf16_later_layer_kernel_stats.md")},
    }
    # reference point, not part of the path: the vendor GEMM library
    # (torch.matmul, hipBLASLt) on the same bf16 operands and all rows; the
    # gated map without the SwiGLU epilogue (its output is twice as wide)
    lib_maps = {"qkv": (x_all, w_qkv), "o": (attn.view(T, H), w_o),
                "gate_up_swiglu": (x_all, w_gu), "down": (hmid, w_down)}
    library = {}
    for name, (inp, w) in lib_maps.items():
        wt = w.t()
        for _ in range(args.warmup):
            torch.matmul(inp, wt)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            torch.matmul(inp, wt)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        library[name] = {"ms_all": ms, "TFLOP/s_all": res_maps[name]["flops_all"] / (ms * 1e-3) / 1e12,
                         "ours_over_library_time": res_maps[name]["ms_all"] / ms}
    res["library_gemm"] = {"what": "torch.matmul (hipBLASLt) on the same operands, all rows; "
                                   "gate/up without the SwiGLU epilogue; reference only",
                           "maps": library}
    if not args.no_cpu_baseline:
        # the oracle's four maps on the first kept rows, float64 on this host
        n = 512
        xs = x_kept[:n].float().cpu().numpy().astype(np.float64)
        ws = {k: v.float().cpu().numpy().astype(np.float64)
              for k, v in (("qkv", w_qkv), ("o", w_o), ("gate", w_gate), ("up", w_up),
                           ("down", w_down))}
        cu_k = [int(c) for c in pc.cu_seqlens_out.cpu().numpy() if c < n] + [n]
        Hq, Hkv = wl.Hq, wl.Hkv
        t0 = time.perf_counter()
        qkv_s = oracle.linear(xs, ws["qkv"])
        att = oracle.linear_attention(qkv_s[:, : Hq * D].reshape(n, Hq, D),
                                      qkv_s[:, Hq * D: (Hq + Hkv) * D].reshape(n, Hkv, D),
                                      qkv_s[:, (Hq + Hkv) * D:].reshape(n, Hkv, D), cu_k)
        oracle.linear(att.reshape(n, Hq * D), ws["o"])
        hs = oracle.swiglu(xs, ws["gate"], ws["up"])
        oracle.linear(hs, ws["down"])
        spent = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": n / spent, "unit": "rows/s", "cores": default_threads(),
                               "kind": "oracle",
                               "sample": f"the first {n} kept rows through the layer (linear "
                                         f"maps, linear attention over their prompts), float64 "
                                         f"NumPy, {spent:.2f} s",
                               "gpu_rows_per_s_kept": kept / (wall_kept * 1e-3)}
    print(json.dumps(res), flush=True)


def _time_one_call(torch, wl, steps, warmup):
    """Stage a one-call workload on the GPU and time its whole step (rotary
    and cache write, attention with block mass, scores, top-p, compaction);
    returns (ms per step, attention kernel ms, visible pairs, kept tokens)."""
    from workloads import device as WD
    from block_sparse_token_amd import binding as B
    from block_sparse_token_amd import step as ST

    call = wl.calls[0]
    kc, vc = WD.make_caches(wl)
    batch = ST.make_batch(call.cu_seqlens, call.ctx_lens, call.positions, call.slot_mapping,
                          call.block_table)
    pc = ST.PrefillCall(batch=batch, q=WD.stored_to_tensor(call.q), k=WD.stored_to_tensor(call.k),
                        v=WD.stored_to_tensor(call.v), k_cache=kc, v_cache=vc,
                        num_blocks=call.num_blocks(wl.block_size),
                        flags=torch.from_numpy(call.flags.astype(np.uint8)).cuda(),
                        block_size=wl.block_size, p=wl.p, rope_theta=wl.theta,
                        rows=WD.row_sources(call))
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        pc.launch()
    torch.cuda.synchronize()
    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)  # creates the underlying event the library records
        return e

    evs = [(ev(), ev()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        B.up_profile_attn_events(a, b)
        pc.launch()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    B.up_profile_attn_events()
    attn = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    pairs = visible_pairs(call.cu_seqlens, call.ctx_lens, call.positions, 0)
    kept = int(pc.num_kept.item())
    del pc, kc, vc
    torch.cuda.empty_cache()
    return wall, attn, pairs, kept


def run_sweep(args):
    """Operator throughput against the number of packed prompts, and the
    padding comparison of the Prepacking summary ("Key design"): the
    headline batch's 16 prompts run (a) packed back to back, the operator's
    own layout, (b) bin-packed by first-fit decreasing into rows of the
    longest prompt's length, each row padded at its end, (c) each prompt
    padded to the longest.  Padding tokens are ordinary tokens to the
    operator (they cost what real ones cost) and are not scored.  Prints one
    JSON line."""
    import torch
    import workloads as W
    from block_sparse_token_amd import packing as PK

    common = dict(Hq=32, Hkv=8, D=128, dtype="bf16", block_size=64, p=0.95, theta=500000.0,
                  hidden_width=4096, scale=1.0 / np.sqrt(128.0))

    def entry(S, T, useful, ms, attn, pairs, kept):
        fl = 4.0 * 128 * 32 * pairs
        return {"prompts": S, "tokens": T, "useful_tokens": useful, "kept_tokens": kept,
                "ms_per_step": ms, "useful_tokens_per_s": useful / (ms * 1e-3),
                "attention_ms": attn, "attention_frac_of_bf16_peak":
                    fl / (attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}

    sweep = []
    for S in (1, 2, 4, 8, 16, 32):
        lengths = [int(x) for x in np.random.default_rng(100 + S).integers(512, 8193, size=S)]
        wl = W.custom(lengths=lengths, seed=100 + S, **common)
        ms, attn, pairs, kept = _time_one_call(torch, wl, args.steps, args.warmup)
        T = int(sum(lengths))
        sweep.append(entry(S, T, T, ms, attn, pairs, kept))
        print(f"sweep prompts={S} tokens={T} ms={ms:.3f}", file=sys.stderr, flush=True)

    head = W.make(WORKLOAD)
    lengths = [s.n for s in head.calls[0].segments]
    T = int(sum(lengths))
    cap = max(lengths)
    layouts = {}
    ms, attn, pairs, kept = _time_one_call(torch, head, args.steps, args.warmup)
    layouts["packed"] = dict(entry(len(lengths), T, T, ms, attn, pairs, kept), pad_tokens=0)
    del head
    segs, pad_flags, pad, nrows = PK.bin_packed_segments(lengths, cap)
    wl = W.custom(lengths=segs, flags=[not f for f in pad_flags], seed=7, **common)
    ms, attn, pairs, kept = _time_one_call(torch, wl, args.steps, args.warmup)
    layouts["bin_packed_rows"] = dict(entry(len(lengths), sum(segs), T, ms, attn, pairs, kept),
                                      pad_tokens=pad, rows=nrows, row_capacity=cap)
    print(f"bin-packed rows={nrows} pad={pad} ms={ms:.3f}", file=sys.stderr, flush=True)
    del wl
    segs, pad = PK.padded_lengths(lengths)
    wl = W.custom(lengths=segs, seed=8, **common)
    ms, attn, pairs, kept = _time_one_call(torch, wl, args.steps, args.warmup)
    layouts["padded"] = dict(entry(len(lengths), sum(segs), T, ms, attn, pairs, kept),
                             pad_tokens=pad)
    print(f"padded pad={pad} ms={ms:.3f}", file=sys.stderr, flush=True)
    res = {"metric": "packed prefill tokens/s vs packed prompts; packed vs bin-packed rows vs "
                     "padded (useful tokens/s)",
           "unit": "tokens/s", "higher_is_better": True, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "prompts with lengths uniform in [512, 8192] (seed 100 + "
                                  "prompts), 32/8 heads x 128, rope 5e5, block 64, top-p 0.95, "
                                  "hidden 4096; padding comparison on the headline batch"},
           "sweep": sweep, "padding": layouts}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the operator is "
              "built and measured for a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return

    if args.propagation:
        run_propagation(args)
        return
    if args.sweep:
        run_sweep(args)
        return
    if args.workload != "all":
        run_one_workload(args)
        return
    run_all(args)


def _generate(names):
    """Generate the workloads on background threads (numpy's bulk draws
    release the interpreter lock), so the GPU measures one while the next is
    drawn."""
    from concurrent.futures import ThreadPoolExecutor
    import workloads as W

    ex = ThreadPoolExecutor(max_workers=3)
    return ex, {n: ex.submit(W.make, n) for n in names}


def run_one_workload(args):
    """One workload (every call, timed as one step), with its oracle sample."""
    import torch

    import workloads as W
    wl = W.make(args.workload)
    if args.whole_prompt and args.workload != "chunked_128k":
        raise SystemExit("--whole-prompt applies to chunked_128k (one prompt in chunks)")
    st = Staged(torch, wl, whole=args.whole_prompt)
    t = time_workload(torch, st, args.steps, args.warmup)
    m = workload_metrics(st, t)
    if args.whole_prompt:
        pc = st.calls[-1][1]
        nbp = int(pc.cu_blocks[-1].item())
        keep = pc.keep[:nbp].cpu().numpy().astype(bool)
        sc = pc.scores[:nbp].cpu().numpy()
        hb = -(-wl.heavy_prefix // wl.block_size)  # blocks holding the heavy-hitter cluster
        m["whole_prompt"] = {
            "prompt_blocks": nbp, "kept_blocks": int(keep.sum()), "cluster_blocks": hb,
            "cluster_blocks_kept": int(keep[:hb].sum()), "other_blocks_kept": int(keep[hb:].sum()),
            "mean_score_cluster": float(sc[:hb].mean()), "mean_score_other": float(sc[hb:].mean()),
            "kept_cached_tokens": int(pc.num_kept_slots.item()),
            "kept_own_tokens": int(pc.num_kept.item())}
    l2p = m["swa_layer"]["pairs"] if "swa_layer" in m else None
    del st
    torch.cuda.empty_cache()
    res = {"metric": METRIC, "value": m["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": m["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
           "data": "synthetic", "config": {"workload": f"{args.workload}: {DESCRIBE[args.workload]}"},
           "roofline": dict(m["attention"], achieved=m["attention"]["TFLOP/s"],
                            unit="TFLOP/s", traffic=None),
           "detail": m}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = oracle_sample(wl, args.cpu_budget_s / 2, l2p)
    print(json.dumps(res), flush=True)


def run_all(args):
    """The default run: the headline packed workload gives the bench line's
    value, roofline and CPU baseline; every other workload is timed the same
    way under ``configs``.  Inputs are generated on background threads while
    the GPU measures; the oracle samples run afterwards on an idle host."""
    import torch
    from block_sparse_token_amd import binding as B

    names = [n for n, *_ in CONFIGS]
    ex, futs = _generate(names)
    stream = torch.cuda.current_stream()
    att = attainable_peaks(torch, B, stream)
    results, wls, l2pairs, copy_cache = {}, {}, {}, {}
    for name, label, cap_steps, cap_warm in CONFIGS:
        wl = futs[name].result()
        wls[name] = wl
        K = args.steps if cap_steps is None else min(args.steps, cap_steps)
        Wm = args.warmup if cap_warm is None else min(args.warmup, cap_warm)
        print(f"measuring {label} {name} ({K} steps)", file=sys.stderr, flush=True)
        st = Staged(torch, wl)
        t = time_workload(torch, st, K, Wm)
        m = workload_metrics(st, t)
        m.update(label=label, workload=DESCRIBE[name], steps=K, warmup=Wm)
        if name == WORKLOAD:
            # the same passes with the Infinity Cache flushed before each step
            flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
            tf = time_workload(torch, st, min(K, 10), 0, flush=flush)
            del flush
            mf = workload_metrics(st, tf)
            m["cache_flushed"] = {"attention_ms": tf["attn_ms"],
                                  "passes": {k: v for k, v in mf["passes"].items()}}
            if args.library:
                call, pc = st.calls[0]
                m["library_attention"] = library_attention(torch, wl, call, pc, min(K, 5))
        l2pairs[name] = m["swa_layer"]["pairs"] if "swa_layer" in m else None
        results[name] = m
        del st
        torch.cuda.empty_cache()
        add_copy_comparison(torch, B, stream, m, copy_cache)
    ex.shutdown(wait=True)
    if not args.no_cpu_baseline:
        for name, label, *_ in CONFIGS:
            budget = args.cpu_budget_s if name == WORKLOAD else args.cpu_budget_s / 2
            print(f"oracle sample {label}", file=sys.stderr, flush=True)
            results[name]["cpu_baseline"] = oracle_sample(wls[name], budget, l2pairs[name])
    h = results[WORKLOAD]
    src_hash = kernel_code_hash(os.path.join(ROOT, "block_sparse_token_amd", "csrc",
                                             "attn_bf16.hip"))
    a = h["attention"]
    res = {
        "metric": METRIC, "value": h["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": h["steps"], "warmup": h["warmup"], "ms_per_step": h["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: {DESCRIBE[WORKLOAD]} ({h['tokens']} tokens)",
                   "tokens": h["tokens"], "kept_tokens": h["kept_tokens"]},
        "roofline": {"bound": "mfma", "achieved": a["TFLOP/s"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": a["frac"],
                     "traffic": traffic_from_profile(src_hash), "kernel": a["kernel"],
                     "avg_ms": a["ms"], "flops_per_launch": a["flops"], "pairs": a["pairs"],
                     "attainable": att["mfma_bf16_TFLOP/s"],
                     "frac_of_attainable": a["TFLOP/s"] / att["mfma_bf16_TFLOP/s"]},
        "passes_hbm": h["passes"],
        "attainable_peaks": att,
        "configs": {results[n]["label"]: results[n] for n in names},
    }
    if "cpu_baseline" in h:
        res["cpu_baseline"] = h["cpu_baseline"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
