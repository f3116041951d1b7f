"""Seeded synthetic inputs for the packed, chunked prefill operator.

This module draws random inputs and lays out batch metadata (segment offsets,
page tables, slot numbers, the chunk schedule).  It holds none of the
operator's arithmetic: no rotary embedding, attention, scoring, selection or
compaction.  Both the CPU oracle's callers and the GPU binding's callers read
the arrays made here.

Conventions
-----------
* ``np.random.default_rng(seed)`` (PCG64).  Draw order: lengths, heavy-hitter
  groups, the heavy direction ``u``, q, k, v, hidden, page permutation, extras.
* bf16 tensors are stored as ``uint16`` bit patterns, the round-to-nearest-even
  rounding of float32 draws.  fp32 tensors are stored as ``float32``.
* "Uniform in [a, b]" means integers with both ends included.
* Heavy-hitter keys: in a seeded fraction of each prompt's 16-token groups the
  keys get ``3 * u`` added (``u`` a unit vector, one per workload) before any
  rotary embedding, so a few key blocks stand out.
* KV pages hold 16 tokens.  Each prompt owns ``ceil(len / 16)`` pages taken
  from a seeded permutation of the page pool, so page ids are scattered.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16
GROUP = 16  # heavy-hitter group size in tokens


# ---------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    The sum stays inside 32 bits for every finite value and for the
    infinities (bit patterns below 0xFFFF8000); the generators draw no NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored tensor."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


# ---------------------------------------------------------------------------
# data classes
# ---------------------------------------------------------------------------
@dataclass
class Segment:
    prompt: int  # prompt / request id
    ctx: int  # tokens already in the KV cache before this segment
    n: int  # new tokens in this call
    flagged: bool  # score and select this segment


@dataclass
class Call:
    """One operator call: a packed batch of segments."""

    segments: list
    q: np.ndarray  # [T, Hq, D]
    k: np.ndarray  # [T, Hkv, D]  (before rotary embedding)
    v: np.ndarray  # [T, Hkv, D]
    hidden: np.ndarray  # [T, W]
    positions: np.ndarray  # [T] int32
    slot_mapping: np.ndarray  # [T] int32
    cu_seqlens: np.ndarray  # [S+1] int32
    ctx_lens: np.ndarray  # [S] int32
    block_table: np.ndarray  # [S, max_pages] int32
    flags: np.ndarray  # [S] uint8
    extra: dict = field(default_factory=dict)  # further row tensors ([T, ...])

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def S(self) -> int:
        return len(self.segments)

    def max_seqlen(self) -> int:
        return int(max(s.n for s in self.segments))

    def max_ctx(self) -> int:
        return int(max(s.ctx for s in self.segments))

    def num_blocks(self, block_size: int, whole_prompt: bool = False) -> int:
        """Blocks of the call; with whole_prompt, a flagged segment's blocks
        cover its cached tokens too (layout only, no arithmetic of the method)."""
        return int(self.cu_blocks(block_size, whole_prompt)[-1])

    def cu_blocks(self, block_size: int, whole_prompt: bool = False) -> np.ndarray:
        nb = [-(-(s.n + (s.ctx if whole_prompt and s.flagged else 0)) // block_size)
              for s in self.segments]
        return np.concatenate([[0], np.cumsum(nb)]).astype(np.int32)


@dataclass
class Workload:
    name: str
    dtype: str  # "f32" | "bf16"
    Hq: int
    Hkv: int
    D: int
    block_size: int
    p: float
    theta: float  # rotary base; <= 0 disables it
    window: int  # <= 0: full causal
    hidden_width: int
    num_pages: int
    prompt_pages: dict  # prompt id -> int32 page ids (logical page order)
    prompt_len: dict  # prompt id -> total tokens the prompt ever holds in the cache
    calls: list
    # KV entries that exist before the first call, taken as already rotated:
    # prompt id -> (K [c, Hkv, D], V [c, Hkv, D]) in storage dtype.
    given_cache: dict = field(default_factory=dict)
    # For very large given caches: drawn on the device from this seed instead
    # (see ``device_cache_spec``); ``given_cache`` then stays empty.
    device_cache_seed: int | None = None
    device_cache_ctx: dict = field(default_factory=dict)  # prompt id -> c
    layer2: dict | None = None  # second (sliding-window) layer settings
    seed: int = 0
    heavy_prefix: int = 0  # tokens of the leading heavy-hitter cluster, if any

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def _uniform_int(rng, a, b, n):
    return rng.integers(a, b + 1, size=n).astype(np.int64)


def _unit(rng, D):
    u = rng.standard_normal(D).astype(np.float64)
    return (u / np.linalg.norm(u)).astype(np.float32)


def _normal32(rng, shape, scale=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _pages_for(rng, prompt_len: dict):
    order = sorted(prompt_len)
    npages = {pid: -(-prompt_len[pid] // PAGE_SIZE) for pid in order}
    total = int(sum(npages.values()))
    perm = rng.permutation(total).astype(np.int32)
    pages, off = {}, 0
    for pid in order:
        pages[pid] = perm[off : off + npages[pid]]
        off += npages[pid]
    return total, pages


def _pack_calls(schedule, prompt_pages, Hq, Hkv, D, W, dtype, rng, scale, heavy_tok, u,
                draw_hidden=True, q_mult=1.0):
    """Draw q, k, v, hidden for every new token of the schedule and pack per call.

    ``schedule``: list of calls, each a list of Segment.  ``heavy_tok``: dict
    prompt -> boolean array over that prompt's token positions.
    """
    tot = sum(s.n for call in schedule for s in call)
    q = _normal32(rng, (tot, Hq, D), scale)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    k = _normal32(rng, (tot, Hkv, D), scale)
    v = _normal32(rng, (tot, Hkv, D), scale)
    # heavy-hitter keys
    row = 0
    for call in schedule:
        for s in call:
            hv = heavy_tok.get(s.prompt)
            if hv is not None:
                m = hv[s.ctx : s.ctx + s.n]
                if m.any():
                    k[row : row + s.n][m] += np.float32(3.0) * u
            row += s.n
    hidden = _normal32(rng, (tot, W)) if draw_hidden else np.zeros((tot, W), np.float32)
    qs, ks, vs, hs = _store(q, dtype), _store(k, dtype), _store(v, dtype), _store(hidden, dtype)
    del q, k, v, hidden
    return qs, ks, vs, hs


def _finish_calls(schedule, qs, ks, vs, hs, prompt_pages):
    calls, row = [], 0
    for segs in schedule:
        T = sum(s.n for s in segs)
        sl = slice(row, row + T)
        row += T
        cu = np.zeros(len(segs) + 1, np.int32)
        cu[1:] = np.cumsum([s.n for s in segs])
        ctx = np.array([s.ctx for s in segs], np.int32)
        pos = np.concatenate([np.arange(s.ctx, s.ctx + s.n) for s in segs]).astype(np.int32)
        maxp = max(len(prompt_pages[s.prompt]) for s in segs)
        bt = np.zeros((len(segs), maxp), np.int32)
        slots = np.empty(T, np.int32)
        for i, s in enumerate(segs):
            pg = prompt_pages[s.prompt]
            bt[i, : len(pg)] = pg
            lp = np.arange(s.ctx, s.ctx + s.n)
            slots[cu[i] : cu[i + 1]] = pg[lp // PAGE_SIZE] * PAGE_SIZE + lp % PAGE_SIZE
        flags = np.array([1 if s.flagged else 0 for s in segs], np.uint8)
        calls.append(
            Call(segments=list(segs), q=qs[sl], k=ks[sl], v=vs[sl], hidden=hs[sl], positions=pos,
                 slot_mapping=slots, cu_seqlens=cu, ctx_lens=ctx, block_table=bt, flags=flags)
        )
    return calls


def _heavy_random(rng, prompt_len: dict, frac: float):
    """Pick round(frac * groups) of all prompts' 16-token groups at random."""
    order = sorted(prompt_len)
    groups = [(pid, g) for pid in order for g in range(-(-prompt_len[pid] // GROUP))]
    nh = int(np.floor(frac * len(groups) + 0.5))
    pick = rng.choice(len(groups), size=nh, replace=False) if nh else np.zeros(0, np.int64)
    heavy = {pid: np.zeros(prompt_len[pid], bool) for pid in order}
    for i in np.sort(pick):
        pid, g = groups[int(i)]
        heavy[pid][g * GROUP : (g + 1) * GROUP] = True
    return heavy


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------
def _chunk_schedule(lengths, chunk, ctx0=None, flag=True):
    """Call c processes chunk c of every prompt that still has tokens."""
    ctx0 = ctx0 or [0] * len(lengths)
    done = list(ctx0)
    calls = []
    while any(done[i] < lengths[i] + ctx0[i] for i in range(len(lengths))):
        segs = []
        for i, L in enumerate(lengths):
            end = ctx0[i] + L
            if done[i] < end:
                n = min(chunk, end - done[i])
                segs.append(Segment(prompt=i, ctx=done[i], n=n, flagged=flag))
                done[i] += n
        calls.append(segs)
    return calls


def config_small_chunked_fp32(seed: int = 1) -> Workload:
    """Tiny packed prefill, fp32: 4 prompts {37,100,64,255}, 2+2 heads x 64,
    block 16, p 0.9, chunk 64 (so later chunks attend their cached KV)."""
    rng = np.random.default_rng(seed)
    lengths = [37, 100, 64, 255]
    plen = {i: L for i, L in enumerate(lengths)}
    heavy = _heavy_random(rng, plen, 0.10)
    u = _unit(rng, 64)
    sched = _chunk_schedule(lengths, 64)
    qs, ks, vs, hs = _pack_calls(sched, None, 2, 2, 64, 128, "f32", rng, 1.0, heavy, u)
    npages, pages = _pages_for(rng, plen)
    calls = _finish_calls(sched, qs, ks, vs, hs, pages)
    return Workload(name="small_chunked_fp32", dtype="f32", Hq=2, Hkv=2, D=64, block_size=16, p=0.9, theta=0.0,
                    window=0, hidden_width=128, num_pages=npages, prompt_pages=pages,
                    prompt_len=plen, calls=calls, seed=seed)


def config_packed_llama8b(seed: int = 2) -> Workload:
    """Llama-3.1-8B-shaped layer, bf16: 16 prompts U{512..8192} packed in one
    call, 32/8 heads x 128, q,k,v ~ N(0,1)/sqrt(128), rotary base 500000,
    block 64, p 0.95, hidden width 4096."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in _uniform_int(rng, 512, 8192, 16)]
    plen = {i: L for i, L in enumerate(lengths)}
    heavy = _heavy_random(rng, plen, 0.10)
    u = _unit(rng, 128)
    sched = [[Segment(prompt=i, ctx=0, n=L, flagged=True) for i, L in enumerate(lengths)]]
    qs, ks, vs, hs = _pack_calls(sched, None, 32, 8, 128, 4096, "bf16", rng, 1.0 / np.sqrt(128.0),
                                 heavy, u)
    npages, pages = _pages_for(rng, plen)
    calls = _finish_calls(sched, qs, ks, vs, hs, pages)
    return Workload(name="packed_llama8b", dtype="bf16", Hq=32, Hkv=8, D=128, block_size=64, p=0.95,
                    theta=500000.0, window=0, hidden_width=4096, num_pages=npages,
                    prompt_pages=pages, prompt_len=plen, calls=calls, seed=seed)


def config_chunked_128k(seed: int = 3, total: int = 131072, chunk: int = 8192) -> Workload:
    """One long prompt in chunks over a paged cache: 131072 tokens, chunk 8192,
    bf16, Llama-3.1-8B heads, block 128, p 0.9.  Heavy-hitter groups are 5% of
    the groups, one contiguous cluster from token 0."""
    rng = np.random.default_rng(seed)
    plen = {0: total}
    ngroups = -(-total // GROUP)
    nh = int(np.floor(0.05 * ngroups + 0.5))
    heavy = {0: np.zeros(total, bool)}
    heavy[0][: nh * GROUP] = True
    u = _unit(rng, 128)
    sched = _chunk_schedule([total], chunk)
    qs, ks, vs, hs = _pack_calls(sched, None, 32, 8, 128, 4096, "bf16", rng, 1.0, heavy, u)
    npages, pages = _pages_for(rng, plen)
    calls = _finish_calls(sched, qs, ks, vs, hs, pages)
    return Workload(name="chunked_128k", dtype="bf16", Hq=32, Hkv=8, D=128, block_size=128, p=0.9,
                    theta=500000.0, window=0, hidden_width=4096, num_pages=npages,
                    prompt_pages=pages, prompt_len=plen, calls=calls, seed=seed,
                    heavy_prefix=nh * GROUP)


def config_mixed_decode_prefill(seed: int = 4, n_decode: int = 256, budget: int = 8192,
              ctx_range=(1024, 32768), wait_range=(4096, 65536), n_wait: int = 6,
              device_cache: bool = True) -> Workload:
    """Continuous-batching step: 256 decodes (1 token, cached context
    U{1024..32768}) then first-come-first-served prefill chunks of 6 waiting
    prompts (U{4096..65536}) up to a token budget of 8192.  Only the prefill
    segments are scored.  The decodes' cached KV (about 17.7 GB at full size)
    is drawn on the device from ``device_cache_seed`` unless ``device_cache``
    is False."""
    rng = np.random.default_rng(seed)
    dec_ctx = [int(x) for x in _uniform_int(rng, ctx_range[0], ctx_range[1], n_decode)]
    wait = [int(x) for x in _uniform_int(rng, wait_range[0], wait_range[1], n_wait)]
    left = budget - n_decode
    segs = [Segment(prompt=i, ctx=c, n=1, flagged=False) for i, c in enumerate(dec_ctx)]
    for j, L in enumerate(wait):
        if left <= 0:
            break
        n = min(L, left)
        segs.append(Segment(prompt=n_decode + j, ctx=0, n=n, flagged=True))
        left -= n
    plen = {i: c + 1 for i, c in enumerate(dec_ctx)}
    for s in segs[n_decode:]:
        plen[s.prompt] = s.n
    prefill_len = {s.prompt: s.n for s in segs[n_decode:]}
    heavy = _heavy_random(rng, prefill_len, 0.10)
    u = _unit(rng, 128)
    qs, ks, vs, hs = _pack_calls([segs], None, 32, 8, 128, 4096, "bf16", rng, 1.0, heavy, u)
    npages, pages = _pages_for(rng, plen)
    calls = _finish_calls([segs], qs, ks, vs, hs, pages)
    wl = Workload(name="mixed_decode_prefill", dtype="bf16", Hq=32, Hkv=8, D=128, block_size=64, p=0.95,
                  theta=500000.0, window=0, hidden_width=4096, num_pages=npages,
                  prompt_pages=pages, prompt_len=plen, calls=calls, seed=seed)
    cache_seed = int(rng.integers(0, 2**31 - 1))
    if device_cache:
        wl.device_cache_seed = cache_seed
        wl.device_cache_ctx = {i: c for i, c in enumerate(dec_ctx)}
    else:
        crng = np.random.default_rng(cache_seed)
        for i, c in enumerate(dec_ctx):
            K = _normal32(crng, (c, 8, 128))
            V = _normal32(crng, (c, 8, 128))
            wl.given_cache[i] = (_store(K, "bf16"), _store(V, "bf16"))
    return wl


def config_swa_after_selection(seed: int = 5, n_prompts: int = 8, len_range=(8192, 32768)) -> Workload:
    """Hybrid-layer propagation: a full-attention layer scores and selects on 8
    prompts U{8192..32768} (block 64, p 0.9); compaction then carries hidden
    states, positions, slots and the second layer's q/k/v; a sliding-window
    (4096) layer runs on the kept tokens at their original positions."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in _uniform_int(rng, len_range[0], len_range[1], n_prompts)]
    plen = {i: L for i, L in enumerate(lengths)}
    heavy = _heavy_random(rng, plen, 0.10)
    u = _unit(rng, 128)
    sched = [[Segment(prompt=i, ctx=0, n=L, flagged=True) for i, L in enumerate(lengths)]]
    qs, ks, vs, hs = _pack_calls(sched, None, 32, 8, 128, 4096, "bf16", rng, 1.0, heavy, u)
    npages, pages = _pages_for(rng, plen)
    calls = _finish_calls(sched, qs, ks, vs, hs, pages)
    T = calls[0].T
    calls[0].extra = {
        "q2": _store(_normal32(rng, (T, 32, 128)), "bf16"),
        "k2": _store(_normal32(rng, (T, 8, 128)), "bf16"),
        "v2": _store(_normal32(rng, (T, 8, 128)), "bf16"),
    }
    return Workload(name="swa_after_selection", dtype="bf16", Hq=32, Hkv=8, D=128, block_size=64, p=0.9,
                    theta=500000.0, window=0, hidden_width=4096, num_pages=npages,
                    prompt_pages=pages, prompt_len=plen, calls=calls,
                    layer2={"window": 4096, "theta": 500000.0}, seed=seed)


CONFIGS = {"small_chunked_fp32": config_small_chunked_fp32, "packed_llama8b": config_packed_llama8b, "chunked_128k": config_chunked_128k, "mixed_decode_prefill": config_mixed_decode_prefill, "swa_after_selection": config_swa_after_selection}


def make(name: str, seed: int | None = None, **kw) -> Workload:
    fn = CONFIGS[name]
    return fn(**kw) if seed is None else fn(seed=seed, **kw)


# ---------------------------------------------------------------------------
# small custom batches (edge cases, random shapes)
# ---------------------------------------------------------------------------
def custom(*, lengths, ctxs=None, flags=None, Hq=2, Hkv=2, D=64, dtype="f32", block_size=16,
           p=0.9, theta=0.0, window=0, hidden_width=64, seed=0, heavy_frac=0.1, scale=1.0,
           extra_rows=False, layer2_window=0, q_mult=1.0) -> Workload:
    """One call with the given segments.  A segment with ctx > 0 has ``ctx``
    cached tokens drawn here (taken as already rotated) and written into its
    pages before the call.  ``q_mult`` multiplies the query draws only (large
    logits without larger values)."""
    rng = np.random.default_rng(seed)
    S = len(lengths)
    ctxs = list(ctxs) if ctxs is not None else [0] * S
    flags = list(flags) if flags is not None else [True] * S
    plen = {i: ctxs[i] + lengths[i] for i in range(S)}
    new_len = {i: lengths[i] for i in range(S)}
    heavy_new = _heavy_random(rng, new_len, heavy_frac)
    heavy = {}
    for i in range(S):
        h = np.zeros(plen[i], bool)
        h[ctxs[i] :] = heavy_new[i]
        heavy[i] = h
    u = _unit(rng, D)
    segs = [Segment(prompt=i, ctx=ctxs[i], n=lengths[i], flagged=bool(flags[i])) for i in range(S)]
    qs, ks, vs, hs = _pack_calls([segs], None, Hq, Hkv, D, hidden_width, dtype, rng, scale, heavy, u,
                                 q_mult=q_mult)
    npages, pages = _pages_for(rng, plen)
    calls = _finish_calls([segs], qs, ks, vs, hs, pages)
    wl = Workload(name="custom", dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size, p=p,
                  theta=theta, window=window, hidden_width=hidden_width, num_pages=npages,
                  prompt_pages=pages, prompt_len=plen, calls=calls, seed=seed)
    for i in range(S):
        if ctxs[i] > 0:
            K = _normal32(rng, (ctxs[i], Hkv, D), scale)
            V = _normal32(rng, (ctxs[i], Hkv, D), scale)
            wl.given_cache[i] = (_store(K, dtype), _store(V, dtype))
    T = calls[0].T
    if extra_rows:
        calls[0].extra = {"x2": _store(_normal32(rng, (T, 3, 8)), dtype)}
    if layer2_window > 0:
        calls[0].extra.update({
            "q2": _store(_normal32(rng, (T, Hq, D), scale), dtype),
            "k2": _store(_normal32(rng, (T, Hkv, D), scale), dtype),
            "v2": _store(_normal32(rng, (T, Hkv, D), scale), dtype),
        })
        wl.layer2 = {"window": layer2_window, "theta": theta}
    return wl


def paged_given_cache(wl: Workload):
    """Lay the given cached KV into page-pool arrays ``[num_pages, Hkv, 16, D]``
    (storage dtype).  Pages nobody writes stay zero."""
    dt = np.uint16 if wl.dtype == "bf16" else np.float32
    kc = np.zeros((wl.num_pages, wl.Hkv, PAGE_SIZE, wl.D), dt)
    vc = np.zeros_like(kc)
    for pid, (K, V) in wl.given_cache.items():
        pg = wl.prompt_pages[pid]
        c = K.shape[0]
        lp = np.arange(c)
        page, off = pg[lp // PAGE_SIZE], lp % PAGE_SIZE
        kc[page, :, off, :] = K
        vc[page, :, off, :] = V
    return kc, vc


def linear_inputs(seed: int, rows: int, k: int, n: int, x_scale: float = 1.0):
    """Activations x [rows, k] ~ N(0, x_scale^2) and weights w [n, k] ~
    N(0, 1/k) (so each output has about x_scale's spread), both bf16 bits."""
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(_normal32(rng, (rows, k), x_scale))
    w = f32_to_bf16_bits(_normal32(rng, (n, k), 1.0 / np.sqrt(k)))
    return x, w


def attention_inputs(seed: int, rows: int, Hq: int, Hkv: int, D: int):
    """q [rows, Hq, D], k and v [rows, Hkv, D] ~ N(0, 1), bf16 bits."""
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(_normal32(rng, (rows, Hq, D)))
    k = f32_to_bf16_bits(_normal32(rng, (rows, Hkv, D)))
    v = f32_to_bf16_bits(_normal32(rng, (rows, Hkv, D)))
    return q, k, v
