"""The C-ABI library on the CPU: it loads without a GPU, exports every entry
point the header declares, and rejects bad arguments on the host before any
launch (no GPU call is made by these tests: every call below fails
validation)."""
import ctypes
import math
import os
import re
import subprocess

import pytest
import torch  # noqa: F401  (binds the library to torch's HIP runtime)

import block_sparse_token_amd as bst
from block_sparse_token_amd import binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uniprefill.h")

UP_OK, UP_ERR_INVALID, UP_ERR_UNSUPPORTED, UP_ERR_WORKSPACE, UP_ERR_DEVICE = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(up_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(Bd.LIB_PATH):
        pytest.skip("library not built")
    return Bd.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"up_prefill_attn", "up_block_scores", "up_topp_select", "up_compact"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", Bd.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (up_[a-z_0-9]+)", out))
    assert set(names) <= exported, set(names) - exported
    for n in names:
        getattr(L, n)
    assert set(Bd.EXPORTED) == set(names)
    assert "gfx950" in bst.up_version()


def _batch(S=2, T=10, page_size=16, with_ptrs=True):
    b = Bd.UpBatch()
    b.num_seqs, b.num_tokens = S, T
    if with_ptrs:
        b.cu_seqlens = b.ctx_lens = b.positions = b.slot_mapping = b.block_table = FAKE.value
    b.max_pages, b.page_size = 4, page_size
    return b


def _attn(L, b, *, dtype=1, Hq=8, Hkv=2, D=128, ws_bytes=1 << 20, flags=None, block=64,
          theta=1e4, scale=0.0, scope=0):
    return L.up_prefill_attn(ctypes.byref(b) if b is not None else None, dtype, Hq, Hkv, D,
                             FAKE, FAKE, FAKE, FAKE, FAKE, theta, 0, scale, flags, block, scope,
                             FAKE, FAKE, FAKE, None, FAKE, ws_bytes, None)


def test_attention_argument_validation(L):
    b = _batch()
    assert _attn(L, None) == UP_ERR_INVALID
    assert _attn(L, b, Hq=6, Hkv=4) == UP_ERR_INVALID
    assert _attn(L, b, Hq=66, Hkv=2) == UP_ERR_UNSUPPORTED  # G = 33
    assert _attn(L, b, Hq=256, Hkv=256) == UP_ERR_UNSUPPORTED  # cache rows use 24-bit products
    assert _attn(L, b, D=96) == UP_ERR_UNSUPPORTED
    assert _attn(L, b, dtype=7) == UP_ERR_UNSUPPORTED
    assert _attn(L, _batch(page_size=8)) == UP_ERR_UNSUPPORTED
    assert _attn(L, _batch(S=0)) == UP_ERR_INVALID
    assert _attn(L, _batch(S=5, T=3)) == UP_ERR_INVALID
    assert _attn(L, _batch(S=4097, T=5000)) == UP_ERR_UNSUPPORTED  # work planner limit
    assert "4096" in L.up_last_error().decode()
    # block sizes: multiples of 16 in [16, 256]
    for bad in (0, 8, 24, 100, 272, 512):
        assert _attn(L, b, flags=FAKE, block=bad) == UP_ERR_UNSUPPORTED, bad
    assert b"multiple of 16" in L.up_last_error()
    assert _attn(L, b, theta=float("nan")) == UP_ERR_INVALID
    # whole-prompt scoring: bf16 only, needs a block table; unknown scopes refused
    assert _attn(L, b, flags=FAKE, scope=1, dtype=0, Hq=2, Hkv=2, D=64) == UP_ERR_UNSUPPORTED
    assert _attn(L, b, flags=FAKE, scope=3) == UP_ERR_INVALID
    nbt = _batch()
    nbt.block_table = None
    assert _attn(L, nbt, flags=FAKE, scope=1) == UP_ERR_INVALID
    assert b"block table" in L.up_last_error()
    need = L.up_attn_workspace_bytes(ctypes.byref(b), 1, 8, 2, 128, 0, 0)
    assert need > 16
    assert _attn(L, b, ws_bytes=need - 1) == UP_ERR_WORKSPACE
    assert b"workspace" in L.up_last_error()
    # 16-byte alignment of the row arrays
    odd = ctypes.c_void_p(FAKE.value + 8)
    for i in range(6):
        ptrs = [FAKE] * 6
        ptrs[i] = odd
        assert L.up_prefill_attn(ctypes.byref(b), 1, 8, 2, 128, *ptrs[:5], 0.0, 0, 0.0, None, 0,
                                 0, None, None, ptrs[5], None, FAKE, 1 << 30, None) == UP_ERR_INVALID
        assert b"16-byte aligned" in L.up_last_error()
    nb = _batch(with_ptrs=False)
    assert _attn(L, nb) == UP_ERR_INVALID
    assert b"NULL" in L.up_last_error()


def test_noalloc_entry_refuses_before_any_device_call(L):
    """The no-allocation attention entry validates like up_prefill_attn and
    refuses a call needing more than its scratch array, all on the host
    (this container has no GPU: a device call would report UP_ERR_DEVICE)."""
    def na(b, **k):
        return L.up_prefill_attn_noalloc(ctypes.byref(b), 1, 32, 8, 128, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, 1e4, 0, 0.0, k.get("flags", FAKE), 64, 0, FAKE,
                                         FAKE, FAKE, None, None)
    b = _batch(S=2, T=600000)
    assert L.up_attn_workspace_bytes(ctypes.byref(b), 1, 32, 8, 128, 64, 0) > Bd.UP_NOALLOC_SCRATCH_BYTES
    assert na(b) == UP_ERR_WORKSPACE
    msg = L.up_last_error().decode()
    assert "bytes of scratch" in msg and str(Bd.UP_NOALLOC_SCRATCH_BYTES) in msg
    assert na(_batch(S=0)) == UP_ERR_INVALID
    bad = _batch(S=2, T=100)
    assert L.up_prefill_attn_noalloc(ctypes.byref(bad), 1, 6, 4, 128, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     1e4, 0, 0.0, None, 0, 0, None, None, FAKE, None,
                                     None) == UP_ERR_INVALID
    # a call that fits gets past validation and only then needs the device
    assert na(_batch(S=2, T=100)) == UP_ERR_DEVICE


def test_workspace_size_arithmetic(L):
    b = _batch(S=16, T=70000)
    # bf16: 256 packed rows per tile -> 64 positions at GQA 4; one int2 per item
    need = L.up_attn_workspace_bytes(ctypes.byref(b), 1, 32, 8, 128, 0, 0)
    items = 16 + 8 * (math.ceil(70000 / 64) + 2 * 16 + 1)
    assert need == items
    assert L.up_attn_workspace_bytes(ctypes.byref(b), 1, 32, 7, 128, 0, 0) == 0
    # scoring in bf16 adds, from a 256-byte boundary, one float per (run of
    # keys, last-block row, head) for every possible block, and one per
    # (segment, last-block row, head); a run is 64, 32 or 16 keys, the
    # largest of those dividing the block
    base = -(-items // 256) * 256
    run_len = {16: 16, 48: 16, 64: 64, 96: 32, 128: 64, 144: 16, 192: 64, 256: 64}
    for B, rl in run_len.items():
        runs = (math.ceil(70000 / B) + 16) * (B // rl)
        want = base + 4 * runs * B * 32 + 4 * 16 * B * 32
        assert L.up_attn_workspace_bytes(ctypes.byref(b), 1, 32, 8, 128, B, 0) == want, B
    for bad in (40, 264):
        assert L.up_attn_workspace_bytes(ctypes.byref(b), 1, 32, 8, 128, bad, 0) == 0
    # float32 scores in its own items: no extra space
    assert (L.up_attn_workspace_bytes(ctypes.byref(b), 0, 2, 2, 64, 16, 0)
            == L.up_attn_workspace_bytes(ctypes.byref(b), 0, 2, 2, 64, 0, 0))
    # whole-prompt scoring: the run bound also counts max_pages * 16 cached
    # tokens per segment (the block table's width)
    b.max_pages = 10
    B = 64
    runs = (math.ceil((70000 + 16 * 10 * 16) / B) + 16) * 1
    want = base + 4 * runs * B * 32 + 4 * 16 * B * 32
    assert L.up_attn_workspace_bytes(ctypes.byref(b), 1, 32, 8, 128, B, 1) == want
    assert L.up_compact_workspace_bytes(16, 1100) == 8 * (1100 + 4)
    assert L.up_compact_workspace_bytes(16, 0) == 0


def test_select_scores_compact_validation(L):
    b = _batch()
    bp = ctypes.byref(b)
    assert L.up_topp_select(bp, 64, FAKE, FAKE, 1.5, FAKE, FAKE, None, None) == UP_ERR_INVALID
    assert L.up_topp_select(bp, 64, FAKE, FAKE, -0.1, FAKE, FAKE, None, None) == UP_ERR_INVALID
    assert L.up_topp_select(bp, 64, FAKE, FAKE, float("nan"), FAKE, FAKE, None, None) == UP_ERR_INVALID
    assert L.up_topp_select(bp, 24, FAKE, FAKE, 0.5, FAKE, FAKE, None, None) == UP_ERR_UNSUPPORTED
    assert L.up_topp_select(bp, 64, None, FAKE, 0.5, FAKE, FAKE, None, None) == UP_ERR_INVALID
    assert L.up_block_scores(bp, 0, 64, FAKE, FAKE, FAKE, FAKE, None) == UP_ERR_INVALID
    assert L.up_block_scores(bp, 8, 64, FAKE, FAKE, None, FAKE, None) == UP_ERR_INVALID
    # the fused score + select entry validates like the two it replaces
    ss = lambda **k: L.up_score_select(bp, k.get("Hq", 8), k.get("B", 64), k.get("cb", FAKE),
                                       FAKE, k.get("p", 0.5), k.get("mass", FAKE), FAKE,
                                       k.get("keep", FAKE), None, None)
    assert ss(p=1.5) == UP_ERR_INVALID
    assert ss(p=float("nan")) == UP_ERR_INVALID
    assert ss(Hq=0) == UP_ERR_INVALID
    assert ss(B=24) == UP_ERR_UNSUPPORTED
    assert ss(cb=None) == UP_ERR_INVALID
    assert ss(mass=None) == UP_ERR_INVALID
    assert ss(keep=None) == UP_ERR_INVALID
    assert L.up_profile_rope_events(FAKE, None) == UP_ERR_INVALID
    assert L.up_profile_rope_events(None, None) == UP_OK
    assert L.up_block_offsets(bp, 100, None, 0, FAKE, None) == UP_ERR_UNSUPPORTED
    assert L.up_block_offsets(bp, 64, FAKE, 2, FAKE, None) == UP_ERR_INVALID  # unknown scope
    rows = (Bd.UpRows * 1)(Bd.UpRows(FAKE.value, FAKE.value, 0))
    assert L.up_compact(bp, 64, FAKE, None, 0, FAKE, 4, 1, rows, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                        None) == UP_ERR_INVALID  # row_bytes 0
    rows = (Bd.UpRows * 1)(Bd.UpRows(FAKE.value, FAKE.value, 8))
    assert L.up_compact(bp, 64, FAKE, None, 0, FAKE, 1, 1, rows, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                        None) == UP_ERR_INVALID  # fewer blocks than segments
    assert L.up_compact(bp, 64, FAKE, None, 0, FAKE, 4, 1, rows, FAKE, FAKE, FAKE, FAKE, 8,
                        None) == UP_ERR_WORKSPACE
    assert L.up_compact(bp, 64, FAKE, None, 0, FAKE, 4, 99, rows, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                        None) == UP_ERR_UNSUPPORTED
    assert L.up_profile_attn_events(FAKE, None) == UP_ERR_INVALID
    assert L.up_profile_attn_events(None, None) == UP_OK


def test_binding_refuses_host_tensors():
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(Bd.UniprefillError):
        Bd.Batch(t, t, t, t)


def test_batch_check_argument_validation(L):
    b = _batch()
    assert L.up_check_batch(None, 0, FAKE, None) == UP_ERR_INVALID
    assert L.up_check_batch(ctypes.byref(b), 0, None, None) == UP_ERR_INVALID
    assert "err_word" in L.up_last_error().decode()
    assert L.up_check_batch(ctypes.byref(b), -1, FAKE, None) == UP_ERR_INVALID
    assert L.up_check_batch(ctypes.byref(_batch(page_size=8)), 0, FAKE, None) == UP_ERR_UNSUPPORTED
    nopos = _batch()
    nopos.positions = None
    assert L.up_check_batch(ctypes.byref(nopos), 0, FAKE, None) == UP_ERR_INVALID


def test_peak_probe_argument_validation(L):
    assert L.up_peak_mfma_bf16(0, 10, FAKE, None) == UP_ERR_INVALID
    assert L.up_peak_mfma_bf16(4, 0, FAKE, None) == UP_ERR_INVALID
    assert L.up_peak_mfma_bf16(4, 10, None, None) == UP_ERR_INVALID
    assert L.up_peak_copy(FAKE, None, 16, None) == UP_ERR_INVALID
    assert L.up_peak_copy(FAKE, FAKE, 24, None) == UP_ERR_INVALID
    assert L.up_peak_copy(ctypes.c_void_p(0x1008), FAKE, 16, None) == UP_ERR_INVALID


def test_linear_argument_validation(L):
    def lin(x=FAKE, w=FAKE, y=FAKE, rows=100, n=512, k=256, act=0):
        return L.up_linear_bf16(x, w, y, rows, None, n, k, act, None)

    assert lin(x=None) == UP_ERR_INVALID
    assert lin(y=None) == UP_ERR_INVALID
    assert lin(rows=-1) == UP_ERR_INVALID
    assert lin(n=300) == UP_ERR_UNSUPPORTED
    assert lin(n=0) == UP_ERR_UNSUPPORTED
    assert lin(k=100) == UP_ERR_UNSUPPORTED
    assert lin(act=2) == UP_ERR_INVALID
    assert lin(x=ctypes.c_void_p(0x1008)) == UP_ERR_INVALID  # not 16-byte aligned
    assert lin(y=ctypes.c_void_p(0x1004)) == UP_ERR_INVALID  # not 8-byte aligned
    assert lin(rows=1 << 20, k=4096) == UP_ERR_UNSUPPORTED  # x of 8 GiB: 32-bit offsets
    assert "4 GiB" in L.up_last_error().decode()
    # each operand under 4 GiB, but more output tiles than one launch takes
    assert lin(rows=(1 << 25) - 1, n=(1 << 25) - 256, k=64) == UP_ERR_UNSUPPORTED
    assert "tiles" in L.up_last_error().decode()


def test_linear_attention_argument_validation(L):
    def la(cu=FAKE, S=2, q=FAKE, qs=4096, k=FAKE, ks=1024, v=FAKE, vs=1024, Hq=32, Hkv=8, D=128,
           out=FAKE):
        return L.up_linear_attn_bf16(cu, S, q, qs, k, ks, v, vs, Hq, Hkv, D, out, None)

    assert la(cu=None) == UP_ERR_INVALID
    assert la(out=None) == UP_ERR_INVALID
    assert la(S=0) == UP_ERR_INVALID
    assert la(S=65536) == UP_ERR_INVALID
    assert la(Hq=30) == UP_ERR_INVALID
    assert la(D=64) == UP_ERR_UNSUPPORTED
    assert la(qs=4000) == UP_ERR_INVALID  # cannot hold 32 heads of 128
    assert la(ks=1028) == UP_ERR_INVALID  # not a multiple of 8
    assert la(q=ctypes.c_void_p(0x1008)) == UP_ERR_INVALID
    assert la(out=ctypes.c_void_p(0x1001)) == UP_ERR_INVALID


def test_linear_attention_parts_validation(L):
    need = L.up_linear_attn_workspace_bytes(5000, 3, 32)
    # slots 5000 // 1024 + 3 + 1 = 8, each 32 heads x (128 x 128 + 128) floats
    assert need == 8 * 32 * (128 * 128 + 128) * 4
    assert L.up_linear_attn_workspace_bytes(-1, 3, 32) == 0

    def lp(rows=5000, ws=FAKE, wsb=need, S=3, D=128, cu=FAKE):
        return L.up_linear_attn_bf16_parts(cu, S, rows, FAKE, 4096, FAKE, 1024, FAKE, 1024, 32, 8,
                                           D, FAKE, ws, wsb, None)

    assert lp(ws=None) == UP_ERR_INVALID
    assert lp(ws=ctypes.c_void_p(0x1008)) == UP_ERR_INVALID  # not 16-byte aligned
    assert lp(wsb=need - 1) == UP_ERR_WORKSPACE
    assert lp(rows=-1) == UP_ERR_INVALID
    assert lp(rows=1 << 26) == UP_ERR_UNSUPPORTED  # more part slots than one grid dimension
    assert lp(cu=None) == UP_ERR_INVALID  # shared checks of up_linear_attn_bf16
    assert lp(D=64) == UP_ERR_UNSUPPORTED


def test_kept_cache_slots_validation(L):
    b = _batch()
    bp = ctypes.byref(b)

    def kc(bt=True, cu=FAKE, flags=FAKE, keep=FAKE, nb=4, slots=FAKE, cap=64, ws=1 << 20):
        bb = _batch()
        if not bt:
            bb.block_table = None
        return L.up_kept_cache_slots(ctypes.byref(bb), 64, cu, flags, keep, nb, slots, cap, FAKE,
                                     FAKE, FAKE, ws, None)

    assert kc(bt=False) == UP_ERR_INVALID
    assert kc(flags=None) == UP_ERR_INVALID
    assert kc(nb=1) == UP_ERR_INVALID
    assert kc(cap=-1) == UP_ERR_INVALID
    assert kc(ws=8) == UP_ERR_WORKSPACE
    assert L.up_kept_cache_slots(bp, 40, FAKE, FAKE, FAKE, 4, FAKE, 64, FAKE, FAKE, FAKE,
                                 1 << 20, None) == UP_ERR_UNSUPPORTED
