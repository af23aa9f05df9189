"""Brute-force quadratic form of the SSD map -- TEST INFRASTRUCTURE ONLY.

"Engineering hybrid state-space models" (innvotechnologies blog), section 2,
states the duality: the sequence map equals Y = (M o (C B^T)) X with the
1-semiseparable mask M[j,k] = prod_{i=k+1}^{j} a_i (empty product = 1 on the
diagonal, 0 above it).  With a_i = exp(dt_i * A_h) and the input scaled by
dt_k (the Euler input term dt*B*x), the output of head h at token j is

    y_j = sum_{k<=j} M[j,k] * (C_j . B_k) * dt_k * x_k          (intra-sequence)
        + (prod_{i=0}^{j} a_i) * (h0 C_j)                        (initial state)
        + D_h * x_j                                              (skip term)

and the final state is h_L = sum_k (prod_{i=k+1}^{L-1} a_i) dt_k x_k (x) B_k
+ (prod_{i=0}^{L-1} a_i) h0.  Every decay factor is formed as an explicit
product of the per-token a_i, O(L^3) work: only for tiny inputs.  This is an
independent route to the same numbers as the sequential recurrence.
"""
from __future__ import annotations

import numpy as np


def _decay_products(a: np.ndarray) -> np.ndarray:
    """M[j,k] = prod_{i=k+1}^{j} a_i for k <= j, else 0 (explicit products)."""
    L = a.shape[0]
    M = np.zeros((L, L), dtype=np.float64)
    for j in range(L):
        for k in range(j + 1):
            M[j, k] = np.prod(a[k + 1:j + 1])  # empty product (k == j) is 1
    return M


def quadratic_scan_sequence(x, dt, A, B, C, D, init=None):
    """One sequence.  x [L,H,P], dt [L,H], B/C [L,G,N], init [H,P,N] or None.

    Returns (y [L,H,P], final [H,P,N]) in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    L, H, P = x.shape
    G, N = B.shape[1:]
    h0 = np.zeros((H, P, N)) if init is None else np.asarray(init, dtype=np.float64)
    y = np.zeros((L, H, P))
    final = np.zeros((H, P, N))
    for h in range(H):
        g = h // (H // G)
        a = np.exp(dt[:, h] * A[h])
        M = _decay_products(a)
        CB = C[:, g, :] @ B[:, g, :].T                    # [j,k] = C_j . B_k
        X = dt[:, h, None] * x[:, h, :]                   # dt_k * x_k
        y_intra = (M * CB) @ X
        lead = np.array([np.prod(a[:j + 1]) for j in range(L)])
        y_init = lead[:, None] * (C[:, g, :] @ h0[h].T)   # (h0 C_j) per token
        y[:, h, :] = y_intra + y_init + D[h] * x[:, h, :]
        tail = np.array([np.prod(a[k + 1:]) for k in range(L)])
        final[h] = np.einsum("k,kp,kn->pn", tail, X, B[:, g, :]) + np.prod(a) * h0[h]
    return y, final
