"""fp64 oracle of the GatedDeltaNet recurrent-state update -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the GPU library.

What it computes.  The linear-attention layers of the pages' model (45 of its
60 layers are GatedDeltaNet) keep, per head, a 128 x 128 state matrix, 64 heads
per layer; per decoded token the engine updates that state with three BLAS
routines, a scaling, matrix-vector products and a rank-one update
("48GB内存运行397B模型：Flash-Moe的极端量化与SSD流式加载实践", section "Metal
GPU管线：手写Kernel与FMA优化", paragraph on linear attention (GatedDeltaNet), and
section "可落地参数清单": 64 heads, state dimension 128; flash-moe README
translation, section "Kỹ thuật chính": BLAS for the linear attention).  The
pages give the routines, not the formula.  The reading taken here is the gated
delta rule as its authors define it (Yang, Kautz and Hatamizadeh, "Gated Delta
Networks: Improving Mamba2 with Delta Rule", 2024), with the state S of a
head a d_v x d_k matrix (row i holds value coordinate i):

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t

evaluated as the sequence of routines the pages name, in this order:

    S <- alpha S                     (the scaling: decay of the state by the gate)
    u <- S k                         (matrix-vector product: what the state recalls at key k)
    w <- beta (v - u)                (the delta-rule correction)
    S <- S + w k^T                   (rank-one update)
    o <- S q                         (matrix-vector product: the head's output)

alpha in (0, 1] is the head's gate for the token, beta in [0, 1] its write
strength.  q and k enter as given: the projections, the short convolution and
the normalisation of q and k that precede this step in the model are outside
it (the pages name only the state update).

Parity status: pinned in ``tests/test_gdn_oracle.py`` by a hand-worked 2 x 2
step and 4 x 4 steps (``tests/golden/gdn_worked.txt``), the matrix form of the
recurrence above, the delta rule's exact recall of v at a unit key, decay
alone at beta = 0, brute-force element loops on small states, and the
equivalence of one multi-token call with single-token calls.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def gdn_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: float,
             beta: float) -> Tuple[np.ndarray, np.ndarray]:
    """One token for one head: returns (new state [d_v][d_k], output [d_v]).
    The routines in the order the pages name them (scale, gemv, ger), fp64."""
    S = np.array(S, dtype=np.float64)           # the caller's state is not modified
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S *= float(alpha)                           # scale
    u = S @ k                                   # gemv
    w = float(beta) * (v - u)
    S += np.outer(w, k)                         # ger (rank-one update)
    o = S @ q                                   # gemv
    return S, o


def gdn_layer(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: np.ndarray,
              beta: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """n_tokens tokens, in order, for every head of a layer.
    S [heads][d_v][d_k]; q, k [tokens][heads][d_k]; v [tokens][heads][d_v];
    alpha, beta [tokens][heads].  Returns (final state, outputs [tokens][heads][d_v])."""
    S = np.array(S, dtype=np.float64)
    T, Hh = np.asarray(alpha).shape
    d_v = S.shape[1]
    out = np.empty((T, Hh, d_v), dtype=np.float64)
    for t in range(T):
        for h in range(Hh):
            S[h], out[t, h] = gdn_step(S[h], q[t, h], k[t, h], v[t, h], alpha[t, h], beta[t, h])
    return S, out
