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
