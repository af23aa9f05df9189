"""fp64 chunked regrouping of the SSD scan -- TEST INFRASTRUCTURE ONLY.

"Compiler-First State Space Duality..." (abstract) names fixed-size chunking
as the structure of the SSD prefill, and "Engineering hybrid state-space
models" (innvotechnologies blog), section 2, computes the recurrence over
chunks of Q tokens with semiseparable products inside each chunk.  Splitting
the decay products of the quadratic form at chunk boundaries gives, for chunk
c of a sequence (tokens t0..t0+len-1) and head h:

  cs[t]      = sum_{s=t0}^{t} dt_s * A_h                 decay exponent, restarted per chunk
  S_c[p,n]   = sum_k exp(cs[last] - cs[k]) dt_k x_k[p] B_k[n]       chunk's own state
  prev_0     = h0 ;  prev_{c+1} = exp(cs[last]) prev_c + S_c        state passed on
  y_t        = exp(cs[t]) (prev_c C_t)
             + sum_{k<=t in c} (C_t . B_k) exp(cs[t]-cs[k]) dt_k x_k  + D_h x_t

The final state of the sequence is prev after its last chunk.  A chunk never
straddles two sequences: chunks restart at each sequence start, and the last
chunk of a sequence may be partial.  The result is the same map as the
sequential recurrence (exact up to rounding), which the pins check.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np


def chunked_scan(x, dt, A, B, C, D, chunk: int, init=None, cu_seqlens=None,
                 return_intermediates: bool = False):
    """Same argument convention as ``oracle.scan`` (dense or packed).

    With ``return_intermediates`` also returns a dict with, per chunk in
    sequence order: 'seq', 'start', 'len', 'cs' [len,H], 'state' [H,P,N]
    (S_c) and 'prev' [H,P,N] (state entering the chunk).
    """
    x = np.asarray(x, dtype=np.float64)
    dense = cu_seqlens is None
    if dense:
        b, L, H, P = x.shape
        xs = x.reshape(b * L, H, P)
        dts = np.asarray(dt, dtype=np.float64).reshape(b * L, H)
        Bs = np.asarray(B, dtype=np.float64).reshape(b * L, *np.shape(B)[2:])
        Cs = np.asarray(C, dtype=np.float64).reshape(b * L, *np.shape(C)[2:])
        cu = np.arange(b + 1) * L
    else:
        xs = x
        dts = np.asarray(dt, dtype=np.float64)
        Bs = np.asarray(B, dtype=np.float64)
        Cs = np.asarray(C, dtype=np.float64)
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        H, P = x.shape[1:]
    A = np.asarray(A, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    G, N = Bs.shape[1:]
    hpg = H // G
    nseq = len(cu) - 1
    y = np.zeros_like(xs)
    final = np.zeros((nseq, H, P, N))
    inter: List[Dict] = []
    for s in range(nseq):
        state = np.zeros((H, P, N)) if init is None else np.array(init[s], dtype=np.float64)
        for t0 in range(int(cu[s]), int(cu[s + 1]), chunk):
            t1 = min(t0 + chunk, int(cu[s + 1]))
            cs = np.cumsum(dts[t0:t1] * A[None, :], axis=0)          # [len,H]
            S_c = np.zeros((H, P, N))
            for h in range(H):
                g = h // hpg
                Xk = dts[t0:t1, h, None] * xs[t0:t1, h, :]             # dt_k x_k  [len,P]
                Bk = Bs[t0:t1, g, :]
                Ct = Cs[t0:t1, g, :]
                w_end = np.exp(cs[-1, h] - cs[:, h])                    # decay k -> chunk end
                S_c[h] = (w_end[:, None] * Xk).T @ Bk
                seg = cs[:, h, None] - cs[None, :, h]                   # cs[t]-cs[k]
                causal = np.tril(np.ones((t1 - t0, t1 - t0), dtype=bool))
                Lmask = np.where(causal, np.exp(np.where(causal, seg, 0.0)), 0.0)
                y_intra = (Lmask * (Ct @ Bk.T)) @ Xk
                y_inter = np.exp(cs[:, h])[:, None] * (Ct @ state[h].T)
                y[t0:t1, h, :] = y_intra + y_inter + D[h] * xs[t0:t1, h, :]
            if return_intermediates:
                inter.append(dict(seq=s, start=t0, len=t1 - t0, cs=cs.copy(),
                                  state=S_c.copy(), prev=state.copy()))
            state = np.exp(cs[-1])[:, None, None] * state + S_c
        final[s] = state
    if dense:
        y = y.reshape(x.shape)
    if return_intermediates:
        return y, final, inter
    return y, final
