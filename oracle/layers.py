"""CPU oracle of the later-layer linear maps that run on the kept tokens.

TEST INFRASTRUCTURE ONLY: used by the tests and the benchmark's CPU-baseline
leg, never by the product path; it shares no code with the HIP library.

Why these maps (UniPrefill review, "Method & Key Results"; UniPrefill paper
entry, abstract): after block selection the dropped tokens skip every later
sublayer, so each later layer's matrix products run on the compacted rows
only, which is where the method saves its work.  The layer shapes are those
of Llama-3.1-8B named for the workloads (hidden width 4096, 32 query and 8
KV heads of 128, so the query/key/value projection maps 4096 to 6144 and
the output projection 4096 to 4096; MLP width 14336).  The pages do not
describe the MLP; Llama's is the SwiGLU-gated one (Shazeer, "GLU Variants
Improve Transformer", 2020): silu(x Wg^T) * (x Wu^T), then the down
projection.  Weights are in the [out, in] layout of a linear layer.

Everything is float64 on the exact stored input values.
"""
from __future__ import annotations

import numpy as np


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * w[n, k] (a linear layer without bias)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.shape[1] != w.shape[1]:
        raise ValueError(f"inner sizes differ: x {x.shape}, w {w.shape}")
    return x @ w.T


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z), written so that no
    intermediate overflows: for z < 0, z * e^z / (1 + e^z)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, z / (1.0 + e), z * e / (1.0 + e))


def swiglu(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """The gated half of a SwiGLU MLP: silu(x Wg^T) * (x Wu^T)."""
    return silu(linear(x, w_gate)) * linear(x, w_up)


def later_layer_flops(rows: int, hidden: int = 4096, qkv_out: int = 6144,
                      mlp: int = 14336) -> int:
    """Matrix-product flops (2 per multiply-add) of one later layer's linear
    maps on `rows` tokens: query/key/value and output projections, the gate
    and up projections and the down projection."""
    per_row = hidden * qkv_out + hidden * hidden + 2 * hidden * mlp + mlp * hidden
    return 2 * rows * per_row


def feature_map(x: np.ndarray) -> np.ndarray:
    """phi(x) = elu(x) + 1: x + 1 for x > 0, e^x otherwise (always > 0)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens) -> np.ndarray:
    """Causal linear attention over each segment of a packed batch, in the
    recurrent form of Katharopoulos et al. ("Transformers are RNNs", 2020):
    per head, with g the KV head of query head h,
        S_t = S_{t-1} + phi(k_t) v_t^T,   z_t = z_{t-1} + phi(k_t),
        o_t = phi(q_t)^T S_t / (phi(q_t) . z_t),
    S and z starting at zero at every segment start (segments are the kept
    tokens of one prompt in their original order; the hybrid models the
    pages name interleave such layers with full attention, UniPrefill paper
    entry, abstract).  q [T, Hq, D], k and v [T, Hkv, D]; returns float64
    [T, Hq, D]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D), np.float64)
    cu = [int(x) for x in cu_seqlens]
    for s in range(len(cu) - 1):
        S = np.zeros((Hkv, D, D))
        z = np.zeros((Hkv, D))
        for t in range(cu[s], cu[s + 1]):
            fk = feature_map(k[t])                       # [Hkv, D]
            S += fk[:, :, None] * v[t][:, None, :]
            z += fk
            fq = feature_map(q[t]).reshape(Hkv, G, D)    # query heads of each group
            num = np.einsum("gjd,gde->gje", fq, S)
            den = np.einsum("gjd,gd->gj", fq, z)
            out[t] = (num / den[:, :, None]).reshape(Hq, D)
    return out
