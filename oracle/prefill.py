"""CPU oracle for the UniPrefill-style prefill operator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only the tests, the package's smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

It computes, in float64 NumPy on the exact input values, what one operator
call does to a packed batch of prompt segments:

* packing: every segment is its own sequence inside the packed batch; a token
  sees only keys of its own segment, and positions restart per prompt
  (Prepacking summary, "Technical framework" and "Key design": the attention
  mask and the positional encoding are modified so several prompts share one
  sequence);
* chunked prefill: when a prompt is fed in pieces, each piece's queries see
  the prompt's KV record left by the pieces before it together with the
  piece's own keys, masked by position so no query sees a later token; the
  pieces' outputs then coincide with a single pass over the whole prompt
  (Ultralytics glossary "Chunked Prefill", section "How chunked prefill
  works");
* token importance per block and top-p block selection: the input is split
  into token blocks, each block gets an importance, and the fewest blocks
  whose cumulative importance reaches p are kept (UniPrefill review,
  "Key Terms & Definitions" (Top-p Token Selection) and "Method & Key
  Results");
* propagation: the dropped tokens leave the batch for all later layers, so
  the kept tokens' rows are compacted (UniPrefill review, "Method & Key
  Results").

The pages give no formula for the importance; the reading used here is: the
importance of key block b is the softmax probability mass that the rows of
the segment's last query block put on b, summed over heads and those rows and
normalised over the segment's blocks.  The first and last blocks are always
kept and their mass counts toward p.

Where the pages leave a step open the plain reading is taken; each such
reading is stated in the docstring of the function that makes it.

Parity status: every function here is pinned by tests under ``tests/`` against
closed forms, a library routine, brute force, or the chunked-prefill example
printed on the glossary page.  ``block_mass`` is pinned by its closed form at
q = 0 (exact rationals) and by a second formulation through block-wise
log-sum-exps written separately in the tests; what no page fixes is the
choice of that importance definition, which is a reading (stated at
``block_mass``), not something a test can pin.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# --------------------------------------------------------------------------
# rotary position embedding
# --------------------------------------------------------------------------


def rope_frequencies(D: int, theta: float) -> np.ndarray:
    """omega_j = theta ** (-2 j / D) for j in [0, D/2) (float64).

    The pages only say the positional encoding is adjusted per prompt
    (Prepacking summary, "Technical framework"); the rotate-half rotary form
    with base ``theta`` is the reading used for the Llama-shaped workloads.
    """
    j = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / D)


def apply_rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate each head vector of ``x`` [n, H, D] by its token's position.

    Pairs (j, j + D/2): x'_j = x_j cos a - x_{j+D/2} sin a and
    x'_{j+D/2} = x_{j+D/2} cos a + x_j sin a, with a = pos * omega_j.
    ``theta <= 0`` means no rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    if theta <= 0:
        return x.copy()
    D = x.shape[-1]
    h = D // 2
    a = np.asarray(positions, dtype=np.float64)[:, None] * rope_frequencies(D, theta)[None, :]
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------


def visible(q_pos: np.ndarray, k_pos: np.ndarray, window: int) -> np.ndarray:
    """Boolean [n, m]: key j is visible to query t.

    A key is visible when its position does not exceed the query's (for a
    chunk this is the lower-triangular mask moved along by the chunk's
    offset, as the glossary's chunked-prefill section describes).  With
    ``window > 0`` only the last ``window`` positions are
    visible: q_pos - window < k_pos <= q_pos.
    """
    qp = np.asarray(q_pos, dtype=np.int64)[:, None]
    kp = np.asarray(k_pos, dtype=np.int64)[None, :]
    vis = kp <= qp
    if window > 0:
        vis &= kp > qp - window
    return vis


def softmax_probs(q_rot, keys, q_pos, k_pos, window, h, G, scale=None):
    """Exact softmax rows P [n, m] of head ``h`` (float64), masked keys get 0.

    Logits are (q . k) * scale with scale = 1/sqrt(D) unless given.  Rows are
    normalised over their visible keys only (max subtracted, exp, divided by
    the sum).  Also returns the natural-log normaliser lse [n].
    """
    D = q_rot.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    g = h // G
    z = (q_rot[:, h, :] @ keys[:, g, :].T) * scale
    vis = visible(q_pos, k_pos, window)
    z = np.where(vis, z, -np.inf)
    mx = z.max(axis=1, keepdims=True)
    e = np.exp(z - mx)
    ssum = e.sum(axis=1, keepdims=True)
    return e / ssum, (mx + np.log(ssum))[:, 0]


def attention(q_rot, keys, vals, q_pos, k_pos, window=0, scale=None, threads=None,
              row_tile=512):
    """Causal (optionally windowed) attention of one segment.

    q_rot [n, Hq, D] (already rotated), keys/vals [m, Hkv, D] with key
    positions k_pos [m].  Query head h reads KV head h // (Hq / Hkv).
    Returns out [n, Hq, D] and lse [n, Hq].  Rows are processed in groups of
    ``row_tile`` only to bound memory; each row's softmax is whole.
    """
    n, Hq, D = q_rot.shape
    Hkv = keys.shape[1]
    G = Hq // Hkv
    out = np.zeros((n, Hq, D), np.float64)
    lse = np.zeros((n, Hq), np.float64)
    jobs = [(h, r0) for h in range(Hq) for r0 in range(0, n, row_tile)]

    def run(job):
        h, r0 = job
        r1 = min(n, r0 + row_tile)
        # only keys up to the last row's position can be visible
        P, l = softmax_probs(q_rot[r0:r1], keys, q_pos[r0:r1], k_pos, window, h, G, scale)
        out[r0:r1, h, :] = P @ vals[:, h // G, :]
        lse[r0:r1, h] = l

    _parallel(run, jobs, threads)
    return out, lse


def _parallel(fn, jobs, threads=None):
    threads = threads or default_threads()
    if threads <= 1 or len(jobs) <= 1:
        for j in jobs:
            fn(j)
        return
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fn, jobs))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# --------------------------------------------------------------------------
# block importance
# --------------------------------------------------------------------------


def num_blocks(n: int, B: int) -> int:
    """Blocks of B tokens from the segment start; the last one may be short."""
    return -(-n // B)


def block_mass(q_rot, keys, q_pos, k_pos, n_ctx, n, B, window=0, scale=None, scope="segment"):
    """Mass m_k per own block of a segment (float64 [nb]).

    The segment's rows are local [0, n); its keys are ``n_ctx`` cached keys
    followed by its own n keys.  The last query block is local rows
    [(nb-1)B, n) (the whole segment when n <= B).  For every head and every
    row t of that block, the exact softmax probabilities over all visible keys
    (cached ones included, so they take part in the normaliser) are summed
    over the own keys of each block.  Cached keys are not scored.

    Reading (the pages name block importance estimated at a full-attention
    layer, UniPrefill review, "Method & Key Results", but give no formula):
    the importance of a block is this softmax mass, normalised afterwards by
    ``normalise_scores``.

    scope="prompt" (whole-prompt scoring of a prompt's final chunk): the
    blocks are those of the whole prompt, B keys each from its first key,
    over the n_ctx cached keys and the n own ones, so cached blocks are
    scored too; n_ctx must be a multiple of B, which makes the prompt's last
    block the segment's last block (the same query rows).
    """
    Hq = q_rot.shape[1]
    G = Hq // keys.shape[1]
    nb = num_blocks(n, B)
    r0 = (nb - 1) * B
    if scope == "prompt":
        if n_ctx % B:
            raise ValueError("whole-prompt scoring needs the cached length to be a multiple of B")
        nbp = num_blocks(n_ctx + n, B)
        m = np.zeros(nbp, np.float64)
        for h in range(Hq):
            P, _ = softmax_probs(q_rot[r0:n], keys, q_pos[r0:n], k_pos, window, h, G, scale)
            per_key = P.sum(axis=0)  # [n_ctx + n], keys in position order
            for kb in range(nbp):
                m[kb] += per_key[kb * B : min((kb + 1) * B, n_ctx + n)].sum()
        return m
    if scope != "segment":
        raise ValueError(f"unknown scope {scope!r}")
    m = np.zeros(nb, np.float64)
    for h in range(Hq):
        P, _ = softmax_probs(q_rot[r0:n], keys, q_pos[r0:n], k_pos, window, h, G, scale)
        own = P[:, n_ctx:].sum(axis=0)  # [n] mass per own key, summed over rows
        for kb in range(nb):
            m[kb] += own[kb * B : min((kb + 1) * B, n)].sum()
    return m


def normalise_scores(m: np.ndarray) -> np.ndarray:
    """s_k = m_k / sum(m), float64; the emitted value is its float32 rounding."""
    return m / m.sum()


# --------------------------------------------------------------------------
# top-p block selection (exact integer arithmetic)
# --------------------------------------------------------------------------
FX_SCORE_BITS = 40
FX_P_BITS = 22


def score_fixed_point(s32: float) -> int:
    """floor(s * 2**40) of a float32 score, exact (Python integer)."""
    return math.floor(math.ldexp(float(np.float32(s32)), FX_SCORE_BITS))


def p_fixed_point(p: float) -> int:
    """floor(p * 2**22 + 0.5)."""
    return math.floor(math.ldexp(float(p), FX_P_BITS) + 0.5)


def topp_select(scores32: np.ndarray, p: float) -> np.ndarray:
    """Keep mask over one segment's blocks.

    The review's Top-p Token Selection keeps the fewest blocks whose
    cumulative importance reaches p ("Key Terms & Definitions").  Readings:
    the first and last blocks are always kept and their importance counts
    toward p; "reaches" means >=; the remaining blocks are taken in order of
    decreasing score (float32 bit pattern, scores are >= 0), ties to the
    lower index, each added while the running sum is still below the target;
    p >= 1 keeps every block.  The sums are exact integers: q_k =
    floor(s_k 2^40), target = ceil(floor(p 2^22 + 1/2) * sum(q) / 2^22).
    """
    s = np.asarray(scores32, dtype=np.float32)
    nb = len(s)
    keep = np.zeros(nb, bool)
    if nb == 0:
        return keep
    if p >= 1.0:
        keep[:] = True
        return keep
    if not (0.0 <= p):
        raise ValueError("p must be in [0, 1]")
    if np.any(~np.isfinite(s)) or np.any(np.signbit(s)):
        raise ValueError("scores must be finite and non-negative")
    q = [score_fixed_point(x) for x in s]
    Q = sum(q)
    if Q >= 1 << (FX_SCORE_BITS + 1):
        raise ValueError("scores of a segment must sum to less than 2")
    pf = p_fixed_point(p)
    target = -((-pf * Q) >> FX_P_BITS)  # ceil(pf * Q / 2^22)
    forced = sorted({0, nb - 1})
    acc = 0
    for k in forced:
        keep[k] = True
        acc += q[k]
    bits = s.view(np.uint32)
    rest = sorted((k for k in range(nb) if not keep[k]), key=lambda k: (-int(bits[k]), k))
    for k in rest:
        if acc >= target:
            break
        keep[k] = True
        acc += q[k]
    return keep


# --------------------------------------------------------------------------
# compaction
# --------------------------------------------------------------------------


def compact(cu_seqlens, flags, block_size, keep_blocks, rows=None, ctx=None, scope="segment"):
    """Compaction of the kept tokens.

    Token t of segment s is kept when s is not scored, or when its block
    (local index // block_size) is kept.  ``keep_blocks`` lists, per segment,
    the boolean keep mask of its blocks (ignored for unscored segments).
    Returns index_map (ascending original packed indices), cu_seqlens_out
    (per-segment kept counts, prefix-summed) and each row tensor of ``rows``
    gathered by index_map (byte-exact copies).

    scope="prompt": the blocks of a scored segment are those of its whole
    prompt (``ctx[s]`` cached tokens, a multiple of block_size, then its
    own), so own token i is kept when prompt block (ctx[s] + i) //
    block_size is; use ``kept_cache_positions`` for the cached tokens.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    S = len(cu) - 1
    keep_tok = []
    for s in range(S):
        n = int(cu[s + 1] - cu[s])
        if flags[s]:
            kb = np.asarray(keep_blocks[s], bool)
            c0 = int(ctx[s]) if scope == "prompt" else 0
            keep_tok.append(np.repeat(kb, block_size)[c0 : c0 + n])
        else:
            keep_tok.append(np.ones(n, bool))
    kt = np.concatenate(keep_tok) if keep_tok else np.zeros(0, bool)
    index_map = np.nonzero(kt)[0].astype(np.int32)
    counts = [int(x.sum()) for x in keep_tok]
    cu_out = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    out_rows = {}
    for name, r in (rows or {}).items():
        out_rows[name] = np.asarray(r)[index_map]
    return index_map, cu_out, out_rows


def kept_cache_positions(flags, block_size, keep_blocks, ctx):
    """Whole-prompt scoring: per scored segment, the positions of its cached
    tokens whose prompt block is kept (ascending); empty for unscored
    segments.  The later layers attend to these cached keys only."""
    out = []
    for s, f in enumerate(flags):
        if not f:
            out.append(np.zeros(0, np.int64))
            continue
        kb = np.asarray(keep_blocks[s], bool)
        u = np.arange(int(ctx[s]), dtype=np.int64)
        out.append(u[kb[u // block_size]])
    return out


# --------------------------------------------------------------------------
# one operator call over a packed batch
# --------------------------------------------------------------------------


class KVCacheModel:
    """The oracle's own record of each prompt's rotated keys and values,
    indexed by position (what the paged cache holds, without pages)."""

    def __init__(self):
        self.k: dict = {}
        self.v: dict = {}

    def put(self, pid, k_rot, v):
        self.k[pid] = np.asarray(k_rot, np.float64)
        self.v[pid] = np.asarray(v, np.float64)

    def get(self, pid, c, Hkv, D):
        if c == 0:
            z = np.zeros((0, Hkv, D), np.float64)
            return z, z
        K, V = self.k[pid], self.v[pid]
        if K.shape[0] < c:
            raise ValueError(f"prompt {pid}: cache holds {K.shape[0]} < {c} tokens")
        return K[:c], V[:c]

    def append(self, pid, ctx, k_rot, v):
        if ctx == 0 or pid not in self.k:
            if ctx != 0:
                raise ValueError("appending after a gap")
            self.put(pid, k_rot, v)
            return
        if self.k[pid].shape[0] != ctx:
            # keep the first ctx positions, then the new ones
            self.k[pid] = self.k[pid][:ctx]
            self.v[pid] = self.v[pid][:ctx]
        self.k[pid] = np.concatenate([self.k[pid], k_rot])
        self.v[pid] = np.concatenate([self.v[pid], v])


def run_call(*, segments, q, k, v, positions, cu_seqlens, Hq, Hkv, D, theta, window,
             block_size, p, cache: KVCacheModel, rows=None, score=True, select=True,
             threads=None, update_cache=True, scope="segment"):
    """Everything one operator call computes, in order.

    ``segments``: list of (prompt_id, ctx, n, flagged).  q [T, Hq, D],
    k, v [T, Hkv, D] (float64, k before rotation), positions [T].
    Returns a dict with out [T,Hq,D], lse [T,Hq], per flagged segment the
    block masses and float32 scores, the keep masks, and the compaction.
    """
    cu = np.asarray(cu_seqlens, np.int64)
    T = int(cu[-1])
    out = np.zeros((T, Hq, D), np.float64)
    lse = np.zeros((T, Hq), np.float64)
    masses, scores, keeps = [], [], []
    new_kv = []
    for si, (pid, ctx, n, flagged) in enumerate(segments):
        a, b = int(cu[si]), int(cu[si + 1])
        assert b - a == n
        pos = np.asarray(positions[a:b], np.int64)
        q_rot = apply_rope(q[a:b], pos, theta)
        k_rot = apply_rope(k[a:b], pos, theta)
        Kc, Vc = cache.get(pid, ctx, Hkv, D)
        keys = np.concatenate([Kc, k_rot])
        vals = np.concatenate([Vc, np.asarray(v[a:b], np.float64)])
        k_pos = np.concatenate([np.arange(ctx, dtype=np.int64), pos])
        o, l = attention(q_rot, keys, vals, pos, k_pos, window, threads=threads)
        out[a:b], lse[a:b] = o, l
        if flagged and score:
            m = block_mass(q_rot, keys, pos, k_pos, ctx, n, block_size, window, scope=scope)
            s32 = normalise_scores(m).astype(np.float32)
            masses.append(m)
            scores.append(s32)
            keeps.append(topp_select(s32, p) if select else None)
        else:
            masses.append(None)
            scores.append(None)
            keeps.append(None)
        new_kv.append((pid, ctx, k_rot, np.asarray(v[a:b], np.float64)))
    if update_cache:
        for pid, ctx, kr, vv in new_kv:
            cache.append(pid, ctx, kr, vv)
    res = {"out": out, "lse": lse, "mass": masses, "scores": scores, "keep": keeps}
    if score and select:
        flags = [bool(sg[3]) for sg in segments]
        ctxs = [int(sg[1]) for sg in segments]
        im, cu_out, rows_out = compact(cu, flags, block_size, keeps, rows, ctx=ctxs, scope=scope)
        res.update(index_map=im, cu_seqlens_out=cu_out, rows_out=rows_out)
        if scope == "prompt":
            res["kept_cache_positions"] = kept_cache_positions(flags, block_size, keeps, ctxs)
    return res
