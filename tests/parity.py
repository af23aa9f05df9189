"""Helpers shared by the GPU parity tests: move seeded host inputs to the GPU,
run the oracle on the same values, and measure errors the way the tolerances
are stated:

  fp32 inputs: max_i |g_i - r_i| / max(|r_i|, rms(r))   <= 1e-4
  bf16 inputs: max_i |g_i - r_i| / rms(r)               <= 2e-2
  (fp32 state and accumulation in both cases; r is the fp64 oracle.)
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref, dtype: str) -> float:
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    if rms == 0.0:
        rms = 1.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    if dtype == "f32":
        den = np.maximum(np.abs(r), rms)
        return float(np.max(np.abs(g - r) / den))
    return float(np.max(np.abs(g - r)) / rms)


def assert_close(got, ref, dtype: str, what: str = ""):
    e = rel_err(got, ref, dtype)
    assert e <= TOL[dtype], "%s: error %.3e > %.1e" % (what, e, TOL[dtype])
    return e


def tdev(a: np.ndarray, dtype: str = "f32"):
    """Host fp32 array -> GPU tensor (bf16 values are already representable)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def to_gpu(inp):
    dt = inp.wl.dtype
    g = dict(x=tdev(inp.x, dt), dt=tdev(inp.dt), A=tdev(inp.A), B=tdev(inp.B, dt), C=tdev(inp.C, dt),
             D=tdev(inp.D), init=None if inp.init is None else tdev(inp.init))
    if inp.cu_seqlens is not None:
        g["cu"] = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    return g


def oracle_scan(inp, heads=None, seqs=None):
    """fp64 oracle on all or a subset of heads / sequences.  Returns (y, final)
    restricted to those heads (and, for dense batches, sequences)."""
    x, dt, A, B, C, D, init = inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init
    H, G = inp.wl.H, inp.wl.G
    cu = inp.cu_seqlens
    if heads is not None:
        heads = np.asarray(heads)
        groups = heads // (H // G)
        x = x[..., heads, :]
        dt = dt[..., heads]
        A = A[heads]
        D = D[heads]
        B = B[..., groups, :]
        C = C[..., groups, :]
        if init is not None:
            init = init[:, heads]
    if seqs is not None and cu is None:
        seqs = np.asarray(seqs)
        x, dt, B, C = x[seqs], dt[seqs], B[seqs], C[seqs]
        if init is not None:
            init = init[seqs]
    return oracle.scan(x, dt, A, B, C, D, init=init, cu_seqlens=cu)
