"""Dense-matrix form of the KDA decode update, in fp64 (NumPy).

TEST INFRASTRUCTURE ONLY.  This is the second, independent formulation that
pins the loop oracle: instead of the element loop it writes one token's
update as matrix algebra,

    S1 = (I - beta kn kn^T) diag(a) S0 + beta kn v^T,     o = scale S1^T qn

which is the delta-rule correction u = v - S'^T kn, S1 = S' + beta kn u^T
with S' = diag(a) S0 expanded.  Matrix products come from NumPy; there is no
loop over state elements here.  Same sources as the loop oracle:
ROCm/ATOM PR #2130 (What: in-kernel L2 normalisation, fp32 accumulation)
and ROCm/ATOM PR #2945 (Limitations: unit k, beta in (0, 1), decay <= 1).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def l2_normalise(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.dot(x, x) + EPS)


def dense_token(S0: np.ndarray, q, k, v, g, b, scale: float):
    """One token on one head: S0 [K, V] fp64 -> (S1 [K, V], o [V])."""
    S0 = np.asarray(S0, dtype=np.float64)
    K, V = S0.shape
    qn = l2_normalise(q)
    kn = l2_normalise(k)
    a = np.exp(np.asarray(g, dtype=np.float64))
    beta = 1.0 / (1.0 + np.exp(-float(b)))
    M = np.eye(K) - beta * np.outer(kn, kn)
    S1 = M @ (np.diag(a) @ S0) + beta * np.outer(kn, np.asarray(v, dtype=np.float64))
    o = scale * (S1.T @ qn)
    return S1, o


def dense_launch(pool: np.ndarray, slot_ids, q, k, v, g, b, n_rows: int = 1,
                 scale: float | None = None, init_slot_ids=None) -> np.ndarray:
    """A whole launch on an fp64 pool [n_slots, H, K, V], updated in place:
    request r chains its n_rows tokens starting from slot init_slot_ids[r]
    (default slot_ids[r*n_rows]) and writes token t's state to slot
    slot_ids[r*n_rows + t]."""
    n_slots, H, K, V = pool.shape
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    slot_ids = np.asarray(slot_ids).reshape(-1)
    R = slot_ids.size
    out = np.zeros((R, H, V), dtype=np.float64)
    for r in range(R // n_rows):
        for h in range(H):
            s0 = slot_ids[r * n_rows] if init_slot_ids is None else init_slot_ids[r]
            S = pool[s0, h].astype(np.float64).copy()
            for t in range(n_rows):
                rho = r * n_rows + t
                S, out[rho, h] = dense_token(S, q[rho, h], k[rho, h], v[rho, h],
                                             g[rho, h], b[rho, h], scale)
                pool[slot_ids[rho], h] = S
    return out
