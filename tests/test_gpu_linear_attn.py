"""Parity of the later linear-attention layer on the GPU
(up_linear_attn_bf16) with the float64 oracle (oracle.linear_attention, the
recurrent form).

Tolerance: the bf16 output bounds of the attention tests (``parity_checks``):
|gpu - oracle| <= 2e-2 per element, and <= 2^-6 of the row's largest
|oracle| (a row: one token and head) plus 1e-6.  The outputs are weighted
means of values, so along a long segment they shrink like 1/sqrt(rows) and
the absolute bound alone loses its power; the GPU's own error is relative
to them: phi(q), phi(k) and the chunk's weights in bf16 (2^-9 each), the
running state as a bf16 pair (about 2^-17).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from block_sparse_token_amd import binding as Bd
from block_sparse_token_amd import step as ST

from gpu_harness import check_bf16_values, log

pytestmark = pytest.mark.gpu

SENTINEL = -12288.0


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _workspace(rows, S, Hq):
    # NaN bytes: what the workspace holds on entry must not matter
    n = Bd.up_linear_attn_workspace_bytes(rows, S, Hq)
    return torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")


def _run(lengths, Hq, Hkv, seed, lead=0, tail=0, strided=False, parts=False):
    D = 128
    cu = np.concatenate([[lead], lead + np.cumsum(lengths)]).astype(np.int32)
    rows = int(cu[-1]) + tail
    log(f"linear attention lengths={lengths} Hq={Hq} Hkv={Hkv} lead={lead} tail={tail} "
        f"strided={strided} parts={parts}")
    qb, kb, vb = W.attention_inputs(seed, rows, Hq, Hkv, D)
    q, k, v = (ST.stored_to_tensor(x) for x in (qb, kb, vb))
    if strided:  # q, k, v as column ranges of one projection output
        qkv = torch.cat([q.reshape(rows, -1), k.reshape(rows, -1), v.reshape(rows, -1)], dim=1)
        q = qkv[:, : Hq * D].view(rows, Hq, D)
        k = qkv[:, Hq * D: (Hq + Hkv) * D].view(rows, Hkv, D)
        v = qkv[:, (Hq + Hkv) * D:].view(rows, Hkv, D)
    out = torch.full((rows, Hq, D), SENTINEL, dtype=torch.bfloat16, device="cuda")
    cu_t = torch.from_numpy(cu).cuda()
    Bd.up_linear_attn_bf16(cu_t, q, k, v, out,
                           workspace=_workspace(rows, len(lengths), Hq) if parts else None)
    torch.cuda.synchronize()
    got = _f64(out)
    a, b = int(cu[0]), int(cu[-1])
    ref = oracle.linear_attention(W.to_f64(qb[a:b], "bf16"), W.to_f64(kb[a:b], "bf16"),
                                  W.to_f64(vb[a:b], "bf16"), cu - a)
    err = np.abs(got[a:b] - ref)
    ratio = check_bf16_values(got[a:b], ref, "linear attention")
    log(f"  max abs err {err.max():.3e}, rms out {np.sqrt(np.mean(ref ** 2)):.3e}, "
        f"worst / row-relative bound {ratio:.3f}")
    assert np.all(got[:a] == SENTINEL) and np.all(got[b:] == SENTINEL)


def test_gpu_linear_attention_ragged_segments():
    _run([1, 63, 64, 65, 200], Hq=8, Hkv=2, seed=21)


def test_gpu_linear_attention_empty_segments_and_single_head_groups():
    # segments of no tokens, and one query head per KV head
    _run([0, 70, 0, 1, 129, 0], Hq=2, Hkv=2, seed=24)


def test_gpu_linear_attention_strided_projection_rows():
    _run([700, 303], Hq=4, Hkv=1, seed=22, lead=5, tail=7, strided=True)


def test_gpu_linear_attention_llama_heads_long_segment():
    _run([4100, 130], Hq=32, Hkv=8, seed=23, strided=True)


def test_gpu_linear_attention_parts_ragged():
    # parts of 1024 rows: single rows, exact multiples, ragged tails, empty
    # segments, a segment of many parts, rows outside the segments
    _run([1, 1023, 1024, 1025, 0, 3000, 2049, 5], Hq=8, Hkv=2, seed=25, lead=3, tail=5,
         strided=True, parts=True)


def test_gpu_linear_attention_parts_llama_heads():
    _run([4100, 130, 2100], Hq=32, Hkv=8, seed=26, parts=True)


@pytest.mark.parametrize("parts", [False, True])
def test_gpu_linear_attention_headline_batch_sampled_segments(parts):
    """The launch the propagation benchmark times: 16 segments of lengths
    uniform in [512, 8192], 32 / 8 heads, q, k, v as column ranges of one
    projection output (drawn on the device with torch's seeded generator).
    The oracle recomputes three whole segments (the longest among them)."""
    Hq, Hkv, D = 32, 8, 128
    lengths = [int(x) for x in np.random.default_rng(2).integers(512, 8193, size=16)]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rows = int(cu[-1])
    log(f"linear attention headline-size batch rows={rows} segments={len(lengths)} "
        f"parts={parts}")
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    qkv = torch.randn((rows, (Hq + 2 * Hkv) * D), generator=g, device="cuda").to(torch.bfloat16)
    q = qkv[:, : Hq * D].view(rows, Hq, D)
    k = qkv[:, Hq * D: (Hq + Hkv) * D].view(rows, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].view(rows, Hkv, D)
    out = torch.full((rows, Hq, D), SENTINEL, dtype=torch.bfloat16, device="cuda")
    Bd.up_linear_attn_bf16(torch.from_numpy(cu).cuda(), q, k, v, out,
                           workspace=_workspace(rows, len(lengths), Hq) if parts else None)
    torch.cuda.synchronize()
    longest = int(np.argmax(lengths))
    for s in sorted({0, longest, len(lengths) - 1}):
        a, b = int(cu[s]), int(cu[s + 1])
        ref = oracle.linear_attention(_f64(q[a:b]), _f64(k[a:b]), _f64(v[a:b]), [0, b - a])
        got = _f64(out[a:b])
        err = float(np.abs(got - ref).max())
        ratio = check_bf16_values(got, ref, f"segment {s}")
        log(f"  segment {s} ({b - a} tokens): max abs err {err:.3e}, worst / row-relative "
            f"bound {ratio:.3f}")
    assert not bool((out == SENTINEL).any()), "a row inside the segments was not written"


def test_gpu_linear_attention_parts_one_long_segment():
    """One segment of 117,888 rows (the kept rows of the 128K-token prompt
    under whole-prompt scoring: 110,720 cached + 7,168 own), 32 / 8 heads,
    in the chunk-parallel form: 116 parts per head.  The oracle recomputes
    query head 0 (KV head 0) over the whole segment; every row of every
    head must be written."""
    Hq, Hkv, D, rows = 32, 8, 128, 117888
    log(f"linear attention parts, one segment of {rows} rows")
    g = torch.Generator(device="cuda")
    g.manual_seed(32)
    qkv = torch.randn((rows, (Hq + 2 * Hkv) * D), generator=g, device="cuda").to(torch.bfloat16)
    q = qkv[:, : Hq * D].view(rows, Hq, D)
    k = qkv[:, Hq * D: (Hq + Hkv) * D].view(rows, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].view(rows, Hkv, D)
    out = torch.full((rows, Hq, D), SENTINEL, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, rows], dtype=torch.int32, device="cuda")
    Bd.up_linear_attn_bf16(cu, q, k, v, out, workspace=_workspace(rows, 1, Hq))
    torch.cuda.synchronize()
    ref = oracle.linear_attention(_f64(q[:, :1]), _f64(k[:, :1]), _f64(v[:, :1]), [0, rows])
    got = _f64(out[:, :1])
    err = np.abs(got - ref)
    ratio = check_bf16_values(got, ref, "head 0")
    log(f"  head 0: max abs err {err.max():.3e} (worst row {int(err.max(axis=(1, 2)).argmax())}), "
        f"worst / row-relative bound {ratio:.3f}")
    assert not bool((out == SENTINEL).any()), "a row was not written"
