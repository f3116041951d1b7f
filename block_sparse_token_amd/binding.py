"""ctypes binding of libuniprefill.so (include/uniprefill.h).

Argument marshalling only: every function passes torch tensors' device
pointers and the current HIP stream to the C entry point of the same name and
raises ``UniprefillError`` with the library's message on a non-OK status.
torch is imported first so the library binds to the HIP runtime torch has
already loaded (both carry the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# UNIPREFILL_LIB selects another build of the library (the tests load the
# host-sanitized one this way); by default the in-tree build.
LIB_PATH = os.environ.get("UNIPREFILL_LIB") or os.path.join(HERE, "libuniprefill.so")

UP_F32, UP_BF16 = 0, 1
UP_SCOPE_SEGMENT, UP_SCOPE_PROMPT = 0, 1
_DT = {torch.float32: UP_F32, torch.bfloat16: UP_BF16}

c_i32, c_size, c_vp, c_f32, c_f64 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, ctypes.c_double


class UniprefillError(RuntimeError):
    pass


class UpBatch(ctypes.Structure):
    _fields_ = [
        ("num_seqs", c_i32),
        ("num_tokens", c_i32),
        ("cu_seqlens", c_vp),
        ("ctx_lens", c_vp),
        ("positions", c_vp),
        ("slot_mapping", c_vp),
        ("block_table", c_vp),
        ("max_pages", c_i32),
        ("page_size", c_i32),
    ]


class UpRows(ctypes.Structure):
    _fields_ = [("src", c_vp), ("dst", c_vp), ("row_bytes", ctypes.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise UniprefillError(
                f"{LIB_PATH} is missing; build it with `python -m block_sparse_token_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        bp = ctypes.POINTER(UpBatch)
        sig = {
            "up_last_error": (ctypes.c_char_p, []),
            "up_version": (ctypes.c_char_p, []),
            "up_block_offsets": (c_i32, [bp, c_i32, c_vp, c_i32, c_vp, c_vp]),
            "up_attn_workspace_bytes": (c_size, [bp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
            "up_prefill_attn": (c_i32, [bp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_f32, c_i32, c_f32, c_vp, c_i32, c_i32, c_vp, c_vp,
                                        c_vp, c_vp, c_vp, c_size, c_vp]),
            "up_prefill_attn_noalloc": (c_i32, [bp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                                c_vp, c_vp, c_f32, c_i32, c_f32, c_vp, c_i32,
                                                c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
            "up_block_scores": (c_i32, [bp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
            "up_topp_select": (c_i32, [bp, c_i32, c_vp, c_vp, c_f64, c_vp, c_vp, c_vp, c_vp]),
            "up_score_select": (c_i32, [bp, c_i32, c_i32, c_vp, c_vp, c_f64, c_vp, c_vp, c_vp,
                                        c_vp, c_vp]),
            "up_profile_rope_events": (c_i32, [c_vp, c_vp]),
            "up_compact_workspace_bytes": (c_size, [c_i32, c_i32]),
            "up_profile_attn_events": (c_i32, [c_vp, c_vp]),
            "up_check_batch": (c_i32, [bp, c_i32, c_vp, c_vp]),
            "up_peak_mfma_bf16": (c_i32, [c_i32, c_i32, c_vp, c_vp]),
            "up_peak_copy": (c_i32, [c_vp, c_vp, c_size, c_vp]),
            "up_linear_attn_bf16": (c_i32, [c_vp, c_i32, c_vp, ctypes.c_int64, c_vp,
                                            ctypes.c_int64, c_vp, ctypes.c_int64, c_i32, c_i32,
                                            c_i32, c_vp, c_vp]),
            "up_linear_attn_workspace_bytes": (c_size, [c_i32, c_i32, c_i32]),
            "up_linear_attn_bf16_parts": (c_i32, [c_vp, c_i32, c_i32, c_vp, ctypes.c_int64, c_vp,
                                                  ctypes.c_int64, c_vp, ctypes.c_int64, c_i32,
                                                  c_i32, c_i32, c_vp, c_vp, c_size, c_vp]),
            "up_linear_bf16": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i32, c_i32, c_vp]),
            "up_compact": (c_i32, [bp, c_i32, c_vp, c_vp, c_i32, c_vp, c_i32, c_i32,
                                   ctypes.POINTER(UpRows), c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
            "up_kept_cache_slots": (c_i32, [bp, c_i32, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_vp,
                                            c_vp, c_vp, c_size, c_vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


EXPORTED = ["up_last_error", "up_version", "up_block_offsets", "up_attn_workspace_bytes",
            "up_prefill_attn", "up_block_scores", "up_topp_select", "up_compact_workspace_bytes",
            "up_compact", "up_profile_attn_events", "up_check_batch", "up_peak_mfma_bf16",
            "up_peak_copy", "up_linear_bf16", "up_linear_attn_bf16", "up_kept_cache_slots",
            "up_linear_attn_workspace_bytes", "up_linear_attn_bf16_parts", "up_score_select",
            "up_profile_rope_events", "up_prefill_attn_noalloc"]
UP_NOALLOC_SCRATCH_BYTES = 64 << 20


def _check(st: int, what: str):
    if st != 0:
        msg = lib().up_last_error().decode()
        raise UniprefillError(f"{what} failed (status {st}): {msg}")


def _p(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if t.device.type != "cuda":
        raise UniprefillError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise UniprefillError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class Batch:
    """Device metadata of one packed batch (see ``up_batch`` in the header)."""

    def __init__(self, cu_seqlens, ctx_lens, positions, slot_mapping, block_table=None,
                 num_tokens=None, page_size=16):
        self.cu_seqlens = cu_seqlens
        self.ctx_lens = ctx_lens
        self.positions = positions
        self.slot_mapping = slot_mapping
        self.block_table = block_table
        self.num_seqs = int(cu_seqlens.numel() - 1)
        self.num_tokens = int(num_tokens if num_tokens is not None else positions.numel())
        self.page_size = page_size
        self.max_pages = int(block_table.shape[1]) if block_table is not None else 0
        self._s = UpBatch(self.num_seqs, self.num_tokens, _p(cu_seqlens).value,
                          _p(ctx_lens).value if ctx_lens is not None else None,
                          _p(positions).value if positions is not None else None,
                          _p(slot_mapping).value if slot_mapping is not None else None,
                          _p(block_table).value if block_table is not None else None,
                          self.max_pages, page_size)

    @property
    def ref(self):
        return ctypes.byref(self._s)


def up_version() -> str:
    return lib().up_version().decode()


def up_block_offsets(batch: Batch, block_size: int, cu_blocks, score_flags=None,
                     score_scope=UP_SCOPE_SEGMENT, stream=None):
    _check(lib().up_block_offsets(batch.ref, block_size, _p(score_flags), int(score_scope),
                                  _p(cu_blocks), _stream(stream)), "up_block_offsets")


def up_attn_workspace_bytes(batch: Batch, dtype, Hq, Hkv, D, block_size=0,
                            score_scope=UP_SCOPE_SEGMENT) -> int:
    """``block_size``: the scoring block size when scores are asked for, else 0."""
    return int(lib().up_attn_workspace_bytes(batch.ref, _DT[dtype], Hq, Hkv, D, int(block_size),
                                             int(score_scope)))


def up_prefill_attn(batch: Batch, q, k, v, k_cache, v_cache, out, workspace, *, rope_theta=0.0,
                    window=0, sm_scale=0.0, score_flags=None, block_size=0,
                    score_scope=UP_SCOPE_SEGMENT, cu_blocks=None, block_mass=None, lse=None,
                    stream=None):
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if q.dtype not in _DT or any(t.dtype != q.dtype for t in (k, v, k_cache, v_cache, out)):
        raise UniprefillError("q, k, v, caches and out must share one dtype (float32 or bfloat16)")
    _check(lib().up_prefill_attn(batch.ref, _DT[q.dtype], Hq, Hkv, D, _p(q), _p(k), _p(v),
                                 _p(k_cache), _p(v_cache), float(rope_theta), int(window),
                                 float(sm_scale), _p(score_flags), int(block_size),
                                 int(score_scope), _p(cu_blocks),
                                 _p(block_mass), _p(out), _p(lse), _p(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "up_prefill_attn")


def up_prefill_attn_noalloc(batch: Batch, q, k, v, k_cache, v_cache, out, *, rope_theta=0.0,
                            window=0, sm_scale=0.0, score_flags=None, block_size=0,
                            score_scope=UP_SCOPE_SEGMENT, cu_blocks=None, block_mass=None,
                            lse=None, stream=None):
    """up_prefill_attn without a workspace: the library's per-GPU scratch
    array serves instead (calls that overlap on one GPU race)."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if q.dtype not in _DT or any(t.dtype != q.dtype for t in (k, v, k_cache, v_cache, out)):
        raise UniprefillError("q, k, v, caches and out must share one dtype (float32 or bfloat16)")
    _check(lib().up_prefill_attn_noalloc(batch.ref, _DT[q.dtype], Hq, Hkv, D, _p(q), _p(k),
                                         _p(v), _p(k_cache), _p(v_cache), float(rope_theta),
                                         int(window), float(sm_scale), _p(score_flags),
                                         int(block_size), int(score_scope), _p(cu_blocks),
                                         _p(block_mass), _p(out), _p(lse), _stream(stream)),
           "up_prefill_attn_noalloc")


def up_block_scores(batch: Batch, Hq, block_size, cu_blocks, score_flags, block_mass, scores,
                    stream=None):
    _check(lib().up_block_scores(batch.ref, Hq, block_size, _p(cu_blocks), _p(score_flags),
                                 _p(block_mass), _p(scores), _stream(stream)), "up_block_scores")


def up_score_select(batch: Batch, Hq, block_size, cu_blocks, score_flags, p, block_mass, scores,
                    keep, kept_blocks=None, stream=None):
    """Block scores and top-p selection in one launch."""
    _check(lib().up_score_select(batch.ref, Hq, block_size, _p(cu_blocks), _p(score_flags),
                                 float(p), _p(block_mass), _p(scores), _p(keep), _p(kept_blocks),
                                 _stream(stream)), "up_score_select")


def up_profile_rope_events(start=None, stop=None):
    """Record torch.cuda.Event ``start``/``stop`` around the rotary/cache-write
    kernel of later up_prefill_attn calls on this thread; no arguments turns
    it off."""
    hs = ctypes.c_void_p(start.cuda_event) if start is not None else None
    he = ctypes.c_void_p(stop.cuda_event) if stop is not None else None
    _check(lib().up_profile_rope_events(hs, he), "up_profile_rope_events")


def up_topp_select(batch: Batch, block_size, cu_blocks, score_flags, p, scores, keep,
                   kept_blocks=None, stream=None):
    _check(lib().up_topp_select(batch.ref, block_size, _p(cu_blocks), _p(score_flags), float(p),
                                _p(scores), _p(keep), _p(kept_blocks), _stream(stream)),
           "up_topp_select")


def up_compact_workspace_bytes(num_seqs, num_blocks) -> int:
    return int(lib().up_compact_workspace_bytes(num_seqs, num_blocks))


def up_compact(batch: Batch, block_size, cu_blocks, keep, num_blocks, rows, index_map,
               cu_seqlens_out, num_kept, workspace, score_flags=None,
               score_scope=UP_SCOPE_SEGMENT, stream=None):
    """``rows``: list of (src, dst) tensors whose first dimension is the token."""
    arr = (UpRows * max(1, len(rows)))()
    for i, (src, dst) in enumerate(rows):
        rb = src[0].numel() * src.element_size() if src.dim() > 1 else src.element_size()
        arr[i] = UpRows(_p(src).value, _p(dst).value, rb)
    _check(lib().up_compact(batch.ref, block_size, _p(cu_blocks), _p(score_flags),
                            int(score_scope), _p(keep), int(num_blocks), len(rows), arr, _p(index_map), _p(cu_seqlens_out), _p(num_kept),
                            _p(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream)), "up_compact")


def up_profile_attn_events(start=None, stop=None):
    """Record torch.cuda.Event ``start``/``stop`` around the attention kernel
    of later up_prefill_attn calls on this thread; no arguments turns it off."""
    hs = ctypes.c_void_p(start.cuda_event) if start is not None else None
    he = ctypes.c_void_p(stop.cuda_event) if stop is not None else None
    _check(lib().up_profile_attn_events(hs, he), "up_profile_attn_events")


def up_check_batch(batch: Batch, num_pages: int, err_word, stream=None):
    """Check the batch's device-side preconditions (synchronises the stream);
    raises UniprefillError naming every violated condition."""
    _check(lib().up_check_batch(batch.ref, int(num_pages), _p(err_word), _stream(stream)),
           "up_check_batch")


def up_peak_mfma_bf16(workgroups: int, iters: int, sink, stream=None):
    """bf16 matrix-core loop: workgroups * 4 * iters * 4 * 32768 flops."""
    if sink.numel() * sink.element_size() < workgroups * 256 * 4:
        raise UniprefillError("sink must hold workgroups * 256 floats")
    _check(lib().up_peak_mfma_bf16(int(workgroups), int(iters), _p(sink), _stream(stream)),
           "up_peak_mfma_bf16")


def up_peak_copy(src, dst, stream=None):
    """Copy src to dst (same byte size) with the library's streaming copy."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise UniprefillError("dst is smaller than src")
    _check(lib().up_peak_copy(_p(src), _p(dst), n, _stream(stream)), "up_peak_copy")


UP_ACT_NONE, UP_ACT_SWIGLU = 0, 1


def up_linear_bf16(x, w, y, rows_in_use=None, act=UP_ACT_NONE, stream=None):
    """y = x w^T over the rows in use (``rows_in_use``: a one-element int32
    device tensor, e.g. the kept count of up_compact; None = all rows of x),
    or the SwiGLU-gated product with ``act=UP_ACT_SWIGLU`` (w's gate and up
    rows interleaved in groups of 32).  x [rows, K], w [N, K], y [rows, N]
    or [rows, N / 2], all bfloat16."""
    for name, t in (("x", x), ("w", w), ("y", y)):
        if t.dtype != torch.bfloat16 or t.dim() != 2:
            raise UniprefillError(f"{name} must be a 2-D bfloat16 tensor")
    rows, K = x.shape
    N = w.shape[0]
    out_cols = N // 2 if act == UP_ACT_SWIGLU else N
    if w.shape[1] != K or y.shape[0] < rows or y.shape[1] != out_cols:
        raise UniprefillError(f"shapes do not match: x {tuple(x.shape)}, w {tuple(w.shape)}, "
                              f"y {tuple(y.shape)}")
    if rows_in_use is not None and (rows_in_use.dtype != torch.int32 or rows_in_use.numel() < 1):
        raise UniprefillError("rows_in_use must be an int32 device tensor")
    _check(lib().up_linear_bf16(_p(x), _p(w), _p(y), rows, _p(rows_in_use), N, K, act,
                                _stream(stream)), "up_linear_bf16")


def interleave_gate_up(w_gate, w_up):
    """The weight layout UP_ACT_SWIGLU reads: gate and up rows ([F, K] each,
    F a multiple of 128) interleaved in groups of 32 rows -> [2F, K]."""
    F, K = w_gate.shape
    if w_up.shape != (F, K) or F % 128:
        raise UniprefillError("gate and up weights must share a shape [F, K], F a multiple of 128")
    return torch.stack([w_gate.reshape(F // 32, 32, K), w_up.reshape(F // 32, 32, K)],
                       dim=1).reshape(2 * F, K).contiguous()


def up_linear_attn_workspace_bytes(rows, num_seqs, Hq):
    return int(lib().up_linear_attn_workspace_bytes(int(rows), int(num_seqs), int(Hq)))


def up_linear_attn_bf16(cu_seqlens, q, k, v, out, workspace=None, stream=None):
    """Causal linear attention (phi = elu + 1) over each segment of
    ``cu_seqlens``.  q [rows, Hq, D] and k, v [rows, Hkv, D] bfloat16 views
    whose rows may be strided (e.g. column ranges of one projection output,
    ``qkv[:, :Hq*D].view(rows, Hq, D)``); out [rows, Hq, D] contiguous.
    With ``workspace`` (a uint8 GPU tensor of up_linear_attn_workspace_bytes
    bytes) the chunk-parallel entry point runs instead."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.device.type != "cuda":
            raise UniprefillError(f"{name} must be a 3-D bfloat16 GPU tensor")
        if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise UniprefillError(f"{name}: heads must be contiguous within a row")
    if not out.is_contiguous():
        raise UniprefillError("out must be contiguous")
    rows, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape != v.shape or k.shape[0] != rows or out.shape != q.shape:
        raise UniprefillError("q, k, v and out shapes do not match")
    if workspace is not None:
        _check(lib().up_linear_attn_bf16_parts(
            _p(cu_seqlens), cu_seqlens.numel() - 1, rows, ctypes.c_void_p(q.data_ptr()),
            q.stride(0), ctypes.c_void_p(k.data_ptr()), k.stride(0),
            ctypes.c_void_p(v.data_ptr()), v.stride(0), Hq, Hkv, D, _p(out), _p(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)),
            "up_linear_attn_bf16_parts")
        return
    _check(lib().up_linear_attn_bf16(_p(cu_seqlens), cu_seqlens.numel() - 1,
                                     ctypes.c_void_p(q.data_ptr()), q.stride(0),
                                     ctypes.c_void_p(k.data_ptr()), k.stride(0),
                                     ctypes.c_void_p(v.data_ptr()), v.stride(0), Hq, Hkv, D,
                                     _p(out), _stream(stream)), "up_linear_attn_bf16")


def up_kept_cache_slots(batch: Batch, block_size, cu_blocks, score_flags, keep, num_blocks, slots,
                        cu_slots_out, num_slots, workspace, stream=None):
    """KV slots of the kept cached tokens under whole-prompt scoring
    (``slots``: int32 tensor whose length is the capacity)."""
    _check(lib().up_kept_cache_slots(batch.ref, block_size, _p(cu_blocks), _p(score_flags),
                                     _p(keep), int(num_blocks), _p(slots), slots.numel(),
                                     _p(cu_slots_out), _p(num_slots), _p(workspace),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream)), "up_kept_cache_slots")
