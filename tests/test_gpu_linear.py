"""Parity of the later-layer linear maps on the GPU (up_linear_bf16) with the
float64 oracle (oracle/layers.py).

Tolerance, element-wise: the GPU sums exact products of the bf16 inputs in
float32 and rounds each result to bf16 once.  That rounding moves a value by
at most 2^-8 of itself; the float32 sums differ from the exact ones by about
1e-6 of the outputs' spread at these sizes.  So |gpu - oracle| <= 2^-8
|oracle| + 1e-4 rms(oracle).

The small cases draw their inputs with the seeded NumPy generators; the
full-size cases (the row counts of the Llama-3.1-8B-shaped packed batch:
68645 tokens, 65701 of them kept) draw them on the device with torch's
seeded generator (input construction) and hand the oracle the sampled rows
and the weights read back from the device.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from block_sparse_token_amd import binding as Bd
from block_sparse_token_amd import step as ST

from gpu_harness import log

pytestmark = pytest.mark.gpu

REL = 2.0 ** -8
ABS_RMS = 1e-4
SENTINEL = -12288.0  # -3 * 2^12, exactly representable in bf16


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    bound = REL * np.abs(ref) + ABS_RMS * rms
    worst = float(np.max(err - bound))
    assert worst <= 0, f"{what}: max excess {worst:.3e} (max err {float(err.max()):.3e}, rms {rms:.3f})"


def _dev_rows(n):
    return torch.tensor([n], dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("rows_cap,in_use,N,K", [(300, 283, 512, 192), (300, 1000, 256, 64),
                                                 (257, 257, 768, 320), (64, 0, 256, 64)])
def test_gpu_linear_ragged_rows(rows_cap, in_use, N, K):
    log(f"linear rows_cap={rows_cap} in_use={in_use} N={N} K={K}")
    x_bits, w_bits = W.linear_inputs(seed=rows_cap + N + K, rows=rows_cap, k=K, n=N)
    x = ST.stored_to_tensor(x_bits)
    w = ST.stored_to_tensor(w_bits)
    y = torch.full((rows_cap, N), SENTINEL, dtype=torch.bfloat16, device="cuda")
    Bd.up_linear_bf16(x, w, y, rows_in_use=_dev_rows(in_use))
    torch.cuda.synchronize()
    used = min(in_use, rows_cap)
    got = _f64(y)
    ref = oracle.linear(W.to_f64(x_bits[:used], "bf16"), W.to_f64(w_bits, "bf16"))
    if used:
        _check(got[:used], ref, "y")
    assert np.all(got[used:] == SENTINEL), "rows past the rows in use were written"


def test_gpu_linear_all_rows_without_device_count():
    log("linear rows_in_use=None rows=130 N=256 K=128")
    x_bits, w_bits = W.linear_inputs(seed=7, rows=130, k=128, n=256)
    y = torch.empty((130, 256), dtype=torch.bfloat16, device="cuda")
    Bd.up_linear_bf16(ST.stored_to_tensor(x_bits), ST.stored_to_tensor(w_bits), y)
    torch.cuda.synchronize()
    _check(_f64(y), oracle.linear(W.to_f64(x_bits, "bf16"), W.to_f64(w_bits, "bf16")), "y")


@pytest.mark.parametrize("rows_cap,in_use,F,K", [(300, 271, 256, 128), (40, 40, 128, 64)])
def test_gpu_linear_swiglu(rows_cap, in_use, F, K):
    log(f"swiglu rows_cap={rows_cap} in_use={in_use} F={F} K={K}")
    x_bits, wg_bits = W.linear_inputs(seed=11 + F, rows=rows_cap, k=K, n=F)
    _, wu_bits = W.linear_inputs(seed=13 + F, rows=1, k=K, n=F)
    wg, wu = ST.stored_to_tensor(wg_bits), ST.stored_to_tensor(wu_bits)
    w = Bd.interleave_gate_up(wg, wu)
    y = torch.full((rows_cap, F), SENTINEL, dtype=torch.bfloat16, device="cuda")
    Bd.up_linear_bf16(ST.stored_to_tensor(x_bits), w, y, rows_in_use=_dev_rows(in_use),
                      act=Bd.UP_ACT_SWIGLU)
    torch.cuda.synchronize()
    got = _f64(y)
    ref = oracle.swiglu(W.to_f64(x_bits[:in_use], "bf16"), W.to_f64(wg_bits, "bf16"),
                        W.to_f64(wu_bits, "bf16"))
    _check(got[:in_use], ref, "swiglu")
    assert np.all(got[in_use:] == SENTINEL)


# the four maps of one later layer, at the headline workload's row counts
LLAMA_MAPS = [("qkv", 4096, 6144, False), ("o", 4096, 4096, False),
              ("gate_up", 4096, 14336, True), ("down", 14336, 4096, False)]


@pytest.mark.parametrize("name,K,N,gated", LLAMA_MAPS)
def test_gpu_linear_llama_shapes_sampled_rows(name, K, N, gated):
    rows_cap, in_use = 68645, 65701
    log(f"linear {name} rows_cap={rows_cap} in_use={in_use} K={K} N={N} gated={gated}")
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + K + N)
    x = torch.randn((rows_cap, K), generator=g, device="cuda").to(torch.bfloat16)
    s = 1.0 / np.sqrt(K)
    wa = (torch.randn((N, K), generator=g, device="cuda") * s).to(torch.bfloat16)
    if gated:
        wb = (torch.randn((N, K), generator=g, device="cuda") * s).to(torch.bfloat16)
        w = Bd.interleave_gate_up(wa, wb)
        out_cols = N
    else:
        w = wa
        out_cols = N
    y = torch.full((rows_cap, out_cols), SENTINEL, dtype=torch.bfloat16, device="cuda")
    Bd.up_linear_bf16(x, w, y, rows_in_use=_dev_rows(in_use),
                      act=Bd.UP_ACT_SWIGLU if gated else Bd.UP_ACT_NONE)
    torch.cuda.synchronize()
    rng = np.random.default_rng(K + N)
    rows = np.unique(np.concatenate([[0, 255, 256, in_use - 1],
                                     rng.integers(0, in_use, size=28)]))
    idx = torch.from_numpy(rows).cuda()
    xs = _f64(x.index_select(0, idx))
    if gated:
        ref = oracle.swiglu(xs, _f64(wa), _f64(wb))
    else:
        ref = oracle.linear(xs, _f64(wa))
    _check(_f64(y.index_select(0, idx)), ref, name)
    tail = y[in_use:]
    assert bool((tail == SENTINEL).all()), "rows past the kept count were written"
