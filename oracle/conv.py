"""Causal depthwise conv1d + SiLU, fp64 -- TEST INFRASTRUCTURE ONLY.

The step before the recurrence in the Mamba-2 block ("Engineering Hybrid
State-Space Models", section 3, architecture figure: a width-4 1D convolution
followed by SiLU) with its cache (same page, section 4: a per-layer conv
state of dConv - 1 past inputs per channel).

Readings (the pages name the operation, not its conventions):
  * depthwise: channel c of the output sees only channel c of the input;
  * causal, with tap K-1 on the current token:
        y[t, c] = bias[c] + sum_{k<K} w[c, k] * xp[t + k, c]
    over the padded sequence xp = [state (K-1 rows, oldest first); x];
    a missing state is K-1 rows of zeros;
  * the state after a sequence is the last K-1 rows of xp (so a sequence
    shorter than K-1 keeps part of its incoming state);
  * SiLU(v) = v * sigmoid(v) = v / (1 + exp(-v)).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def silu(v) -> np.ndarray:
    """SiLU in fp64: v * sigmoid(v), with sigmoid written to avoid overflow."""
    v = np.asarray(v, dtype=np.float64)
    e = np.exp(-np.abs(v))
    sig = np.where(v >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return v * sig


def causal_conv1d(x, weight, bias=None, state=None, activation: bool = True
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """One sequence: x [L, C], weight [C, K], bias [C] or None, state [K-1, C]
    or None.  Returns (y [L, C], state after the sequence [K-1, C]), fp64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    C, K = w.shape
    L = x.shape[0]
    assert x.shape == (L, C)
    st = np.zeros((K - 1, C)) if state is None else np.asarray(state, dtype=np.float64)
    assert st.shape == (K - 1, C)
    xp = np.concatenate([st, x], axis=0)  # [K-1+L, C]
    y = np.zeros((L, C)) if bias is None else np.broadcast_to(np.asarray(bias, np.float64), (L, C)).copy()
    for k in range(K):
        y += w[:, k][None, :] * xp[k:k + L]
    if activation:
        y = silu(y)
    return y, xp[L:].copy()


def causal_conv1d_batch(x, weight, bias=None, state=None, cu_seqlens=None, activation: bool = True
                        ) -> Tuple[np.ndarray, np.ndarray]:
    """Dense x [b, L, C] or packed x [T, C] with cu_seqlens [b+1]; state
    [b, K-1, C] or None.  Returns (y shaped like x, final states [b, K-1, C])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    K = w.shape[1]
    if cu_seqlens is None:
        b = x.shape[0]
        seqs = [x[i] for i in range(b)]
    else:
        cu = np.asarray(cu_seqlens)
        b = len(cu) - 1
        seqs = [x[cu[i]:cu[i + 1]] for i in range(b)]
    ys, fins = [], np.zeros((b, K - 1, w.shape[0]))
    for i, xs in enumerate(seqs):
        y, fins[i] = causal_conv1d(xs, w, bias, None if state is None else state[i], activation)
        ys.append(y)
    if cu_seqlens is None:
        return np.stack(ys) if b else np.zeros(x.shape), fins
    return (np.concatenate(ys, axis=0) if ys else np.zeros(x.shape)), fins


def conv1d_step(state, x, weight, bias=None, activation: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """One decode token per sequence: state [b, K-1, C], x [b, C].  Returns
    (y [b, C], new state [b, K-1, C]); the input state is not modified."""
    st = np.asarray(state, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    b = x.shape[0]
    y = np.zeros_like(x)
    new = np.zeros_like(st)
    for i in range(b):
        yi, new[i] = causal_conv1d(x[i][None, :], weight, bias, st[i], activation)
        y[i] = yi[0]
    return y, new
