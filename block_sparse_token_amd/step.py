"""One prefill operator call on the device: buffers plus the call sequence.

``PrefillCall`` allocates (once) every output and workspace a call needs and
``launch()`` issues the library's entry points in order on the current
stream: block offsets, attention (with rotary positions, KV-cache write and
fused block mass), block scores with top-p selection (one launch) and
compaction.  No
arithmetic of the method happens here; torch only provides memory.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import binding as B


def _i32(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def _u8(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def stored_to_tensor(arr: np.ndarray, device="cuda") -> torch.Tensor:
    """Host array in storage form (bf16 as uint16 bits, or float32) -> device tensor."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def tensor_to_stored(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array in storage form (bf16 bits as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def make_batch(cu_seqlens, ctx_lens, positions, slot_mapping, block_table=None, num_tokens=None,
               device="cuda") -> B.Batch:
    bt = _i32(block_table, device) if block_table is not None else None
    return B.Batch(_i32(cu_seqlens, device), _i32(ctx_lens, device), _i32(positions, device),
                   _i32(slot_mapping, device), bt, num_tokens=num_tokens)


@dataclass
class PrefillCall:
    batch: B.Batch
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    num_blocks: int  # capacity >= cu_blocks[S]
    flags: torch.Tensor | None  # [S] u8 or None
    block_size: int
    p: float
    rope_theta: float = 0.0
    window: int = 0
    rows: list = field(default_factory=list)  # [(name, src tensor)] to compact
    with_lse: bool = False
    compact: bool = True
    score_scope: int = B.UP_SCOPE_SEGMENT  # UP_SCOPE_PROMPT: whole-prompt scoring

    def __post_init__(self):
        dev = self.q.device
        T, Hq, D = self.q.shape
        S = self.batch.num_seqs
        NB = max(1, self.num_blocks)
        self.Hq = Hq
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((T, Hq), dtype=torch.float32, device=dev) if self.with_lse else None
        self.cu_blocks = torch.empty(S + 1, dtype=torch.int32, device=dev)
        scoring = self.flags is not None
        self.block_mass = torch.empty(NB * Hq, dtype=torch.float32, device=dev) if scoring else None
        nbytes = B.up_attn_workspace_bytes(self.batch, self.q.dtype, Hq, self.k.shape[1], D,
                                           self.block_size if scoring else 0, self.score_scope)
        self.attn_ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.scores = torch.empty(NB, dtype=torch.float32, device=dev)
        self.keep = torch.empty(NB, dtype=torch.uint8, device=dev)
        self.kept_blocks = torch.empty(S, dtype=torch.int32, device=dev)
        self.index_map = torch.empty(T, dtype=torch.int32, device=dev)
        self.cu_seqlens_out = torch.empty(S + 1, dtype=torch.int32, device=dev)
        self.num_kept = torch.empty(1, dtype=torch.int32, device=dev)
        self.compact_ws = torch.empty(B.up_compact_workspace_bytes(S, NB), dtype=torch.uint8,
                                      device=dev)
        self.rows_out = {name: torch.empty_like(src) for name, src in self.rows}
        if self.score_scope == B.UP_SCOPE_PROMPT:
            # KV slots of the kept cached tokens (at most every cached token)
            cap = S * self.batch.max_pages * self.batch.page_size
            self.kept_slots = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
            self.cu_kept_slots = torch.empty(S + 1, dtype=torch.int32, device=dev)
            self.num_kept_slots = torch.empty(1, dtype=torch.int32, device=dev)

    # individual stages (each one library call, or two for scoring)
    def attention(self, stream=None):
        B.up_block_offsets(self.batch, self.block_size if self.block_size else 16, self.cu_blocks,
                           score_flags=self.flags, score_scope=self.score_scope, stream=stream)
        B.up_prefill_attn(self.batch, self.q, self.k, self.v, self.k_cache, self.v_cache, self.out,
                          self.attn_ws, rope_theta=self.rope_theta, window=self.window,
                          score_flags=self.flags, block_size=self.block_size,
                          score_scope=self.score_scope,
                          cu_blocks=self.cu_blocks if self.flags is not None else None,
                          block_mass=self.block_mass, lse=self.lse, stream=stream)

    def scores_stage(self, stream=None):
        B.up_block_scores(self.batch, self.Hq, self.block_size, self.cu_blocks, self.flags,
                          self.block_mass, self.scores, stream)

    def select_stage(self, stream=None):
        B.up_topp_select(self.batch, self.block_size, self.cu_blocks, self.flags, self.p,
                         self.scores, self.keep, self.kept_blocks, stream)

    def score_select_stage(self, stream=None):
        """Scores and selection in one launch (same results as the two stages)."""
        B.up_score_select(self.batch, self.Hq, self.block_size, self.cu_blocks, self.flags, self.p,
                          self.block_mass, self.scores, self.keep, self.kept_blocks, stream)

    def compact_stage(self, stream=None):
        rows = [(src, self.rows_out[name]) for name, src in self.rows]
        B.up_compact(self.batch, self.block_size, self.cu_blocks, self.keep, self.num_blocks, rows,
                     self.index_map, self.cu_seqlens_out, self.num_kept, self.compact_ws,
                     score_flags=self.flags, score_scope=self.score_scope, stream=stream)
        if self.score_scope == B.UP_SCOPE_PROMPT:
            B.up_kept_cache_slots(self.batch, self.block_size, self.cu_blocks, self.flags, self.keep,
                                  self.num_blocks, self.kept_slots, self.cu_kept_slots,
                                  self.num_kept_slots, self.compact_ws, stream)

    def launch(self, stream=None):
        self.attention(stream)
        if self.flags is not None:
            self.score_select_stage(stream)
            if self.compact:
                self.compact_stage(stream)
