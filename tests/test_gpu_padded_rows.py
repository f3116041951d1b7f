"""Row capacity above the tokens in use: ``num_tokens`` = T + pad with
cu_seqlens[S] = T.  The padding rows carry large q/k/v values, position 0
and the slots of real tokens, so any use of them would change the KV cache
or the results.  A padded call must give bit-identical results to the
unpadded one for every real row (outputs, log-sum-exp, block scores,
selection, compaction, caches) and leave the padding rows of every output
untouched."""
import numpy as np
import pytest
import torch

import workloads as W
from block_sparse_token_amd import step as ST

pytestmark = pytest.mark.gpu

PAD = 37
CASES = {
    "bf16": dict(lengths=[130, 47, 200], ctxs=[0, 40, 17], Hq=8, Hkv=2, D=128, dtype="bf16",
                 block_size=32, p=0.9, theta=500000.0),
    "f32": dict(lengths=[70, 1, 33], ctxs=[16, 9, 0], Hq=4, Hkv=2, D=64, dtype="f32",
                block_size=16, p=0.8, theta=10000.0, window=40),
}


def _pad(t, fill):
    extra = torch.full((PAD,) + tuple(t.shape[1:]), fill, dtype=t.dtype, device=t.device)
    return torch.cat([t, extra]).contiguous()


@pytest.mark.parametrize("name", sorted(CASES))
def test_gpu_padded_row_capacity(name):
    import gpu_harness as H
    wl = W.custom(seed=77, hidden_width=64, **CASES[name])
    call = wl.calls[0]
    T = call.T
    H.log(f"padded rows: {name} T={T} pad={PAD}")
    kc, vc = H.make_caches(wl)
    kc_ref, vc_ref = kc.clone(), vc.clone()
    ref = H.launch_call(wl, call, kc_ref, vc_ref)
    r = H.gpu_result(ref)

    dev = "cuda"
    pos = np.concatenate([call.positions, np.zeros(PAD, np.int32)])
    slots = np.concatenate([call.slot_mapping, call.slot_mapping[:PAD]])
    batch = ST.make_batch(call.cu_seqlens, call.ctx_lens, pos, slots, call.block_table,
                          device=dev)
    assert batch.num_tokens == T + PAD
    rows = [(n, _pad(t, 3)) for n, t in H.row_sources(call, dev)]
    kc_p, vc_p = kc.clone(), vc.clone()
    pc = ST.PrefillCall(batch=batch, q=_pad(ST.stored_to_tensor(call.q, dev), 100.0),
                        k=_pad(ST.stored_to_tensor(call.k, dev), 1000.0),
                        v=_pad(ST.stored_to_tensor(call.v, dev), -1000.0), k_cache=kc_p,
                        v_cache=vc_p, num_blocks=call.num_blocks(wl.block_size),
                        flags=torch.from_numpy(call.flags.astype(np.uint8)).to(dev),
                        block_size=wl.block_size, p=wl.p, rope_theta=wl.theta, window=wl.window,
                        rows=rows, with_lse=True)
    pc.out.fill_(7.0)
    pc.lse.fill_(-5.0)
    pc.index_map.fill_(-9)
    pc.launch()
    torch.cuda.synchronize()

    out = ST.tensor_to_stored(pc.out)
    assert np.array_equal(out[:T].view(np.uint8), r["out"].view(np.uint8))
    assert (pc.out[T:] == 7.0).all()
    lse = pc.lse.cpu().numpy()
    assert np.array_equal(lse[:T].view(np.uint32), r["lse"].view(np.uint32))
    assert (lse[T:] == -5.0).all()
    assert np.array_equal(pc.cu_blocks.cpu().numpy(), r["cu_blocks"])
    nb = int(r["cu_blocks"][-1])  # blocks in use; the rest of the arrays is capacity
    assert np.array_equal(pc.scores[:nb].cpu().numpy().view(np.uint32),
                          r["scores"][:nb].view(np.uint32))
    assert np.array_equal(pc.keep[:nb].cpu().numpy(), r["keep"][:nb])
    nk = int(pc.num_kept.item())
    assert nk == int(ref.num_kept.item())
    assert np.array_equal(pc.index_map[:nk].cpu().numpy(), ref.index_map[:nk].cpu().numpy())
    assert (pc.index_map[nk:] == -9).all()
    assert torch.equal(pc.cu_seqlens_out, ref.cu_seqlens_out)
    for n, _ in rows:
        assert torch.equal(pc.rows_out[n][:nk], ref.rows_out[n][:nk]), n
    assert torch.equal(kc_p, kc_ref) and torch.equal(vc_p, vc_ref)
    H.log(f"padded rows: {name} ok")
