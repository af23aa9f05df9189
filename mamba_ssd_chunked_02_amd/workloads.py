"""Seeded synthetic workloads for the SSD scan (inputs only, no SSD arithmetic).

Shapes follow Mamba-2 layers of the sizes that "Compiler-First State Space
Duality..." (abstract) evaluates (130M to 2.7B checkpoints): head dim P=64,
state N=128, 24 heads (130M-like) or 80 heads (2.7B-like).  No trained
weights or text are used; every tensor is drawn from the distributions below.

Distributions (v is a variance):
  x ~ N(0,1);  B, C ~ N(0, 1/N);  D ~ N(0,1)
  dt = clamp(softplus(z - 4), 1e-3, 0.1) with z ~ N(0,1)
  A_h = -exp(u) with u ~ U(0, ln 16)          (so A in [-16, -1])
  initial states ~ N(0, 0.1) or zero
Draw order per workload (numpy PCG64, seed = 20260000 + config id unless
given): x, z, u, B, C, D, init, then the decode-step inputs.

x, B and C are rounded to bfloat16 (round to nearest even) when the workload
is bf16; the GPU gets those bits and the oracle gets the same values exactly.
This module is shared by the tests, the benchmark and the oracle's callers; it
contains no part of the scan itself.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

SEED_BASE = 20260000


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16, nearest-even; returns the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values after a round trip through bfloat16."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# ---------------------------------------------------------------- configs
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    P: int
    N: int
    G: int
    dtype: str                     # "f32" or "bf16": dtype of x, B, C, y
    batch: int = 1                 # dense batch (ignored when seqlens is set)
    seqlen: int = 0                # dense L (0 for decode-only)
    seqlens: Optional[Sequence[int]] = None   # packed variable-length batch
    chunk: int = 256
    init_var: float = 0.0          # 0 => zero initial state
    decode_steps: int = 0
    decode_batch: int = 0          # decode-only workloads: number of sequences

    @property
    def varlen(self) -> bool:
        return self.seqlens is not None

    @property
    def nseq(self) -> int:
        if self.varlen:
            return len(self.seqlens)
        return self.batch if self.seqlen else self.decode_batch

    @property
    def tokens(self) -> int:
        if self.varlen:
            return int(sum(self.seqlens))
        return self.batch * self.seqlen


CONFIGS: Dict[int, Workload] = {
    0: Workload("tiny-fp32 b1 L512 H4 P16 N16 G1 Q64", H=4, P=16, N=16, G=1, dtype="f32",
                batch=1, seqlen=512, chunk=64, decode_steps=16),
    1: Workload("mamba2-130m-layer prefill b1 L4096 H24 P64 N128 G1 Q256", H=24, P=64, N=128,
                G=1, dtype="bf16", batch=1, seqlen=4096, chunk=256),
    2: Workload("mamba2-2.7b-layer decode b256 H80 P64 N128 G1", H=80, P=64, N=128, G=1,
                dtype="bf16", decode_batch=256, decode_steps=100, init_var=0.1),
    3: Workload("mamba2-2.7b-layer prefill b8 L8192 H80 P64 N128 G1 Q256", H=80, P=64, N=128,
                G=1, dtype="bf16", batch=8, seqlen=8192, chunk=256, init_var=0.1),
    4: Workload("varlen grouped prefill {1024,4096,12288,32768} H128 P64 N128 G8 Q256", H=128,
                P=64, N=128, G=8, dtype="bf16", seqlens=(1024, 4096, 12288, 32768), chunk=256,
                init_var=0.1, decode_steps=32),
}


# ---------------------------------------------------------------- generation
@dataclasses.dataclass
class Inputs:
    """Host-side inputs.  Float arrays are fp32 holding exactly the values the
    GPU receives (bf16-representable when dtype == 'bf16')."""
    wl: Workload
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: np.ndarray
    init: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    decode: List[Dict[str, np.ndarray]]


def _dt(rng: np.random.Generator, shape) -> np.ndarray:
    z = rng.standard_normal(shape, dtype=np.float32)
    sp = np.logaddexp(np.float32(0.0), z - np.float32(4.0)).astype(np.float32)  # softplus
    return np.clip(sp, np.float32(1e-3), np.float32(0.1)).astype(np.float32)


def _normal(rng, shape, var: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if var != 1.0:
        a *= np.float32(math.sqrt(var))
    return a


def generate(wl: Workload, seed: int, *, A_range=None, A_zero: bool = False,
             A_values: Optional[Sequence[float]] = None, x_zero: bool = False,
             decode_steps: Optional[int] = None, init_var: Optional[float] = None) -> Inputs:
    """Draw one workload.  Variants used by the tests:
    ``A_range=(lo, hi)`` draws A uniformly in [lo, hi] (slow or strong decay),
    ``A_values`` gives A per head (cycled over the heads), ``A_zero`` sets
    A = 0, ``x_zero`` zeroes x (initial-state path only).  ``A_range`` draws
    its values right after u, so the later tensors differ from the plain
    draw's; the other variants leave every other tensor as drawn."""
    rng = np.random.Generator(np.random.PCG64(seed))
    H, P, N, G = wl.H, wl.P, wl.N, wl.G
    if wl.varlen:
        lead = (wl.tokens,)
        cu = np.concatenate([[0], np.cumsum(wl.seqlens)]).astype(np.int32)
    elif wl.seqlen:
        lead = (wl.batch, wl.seqlen)
        cu = None
    else:
        lead = None
        cu = None
    nseq = wl.nseq
    steps = wl.decode_steps if decode_steps is None else decode_steps
    ivar = wl.init_var if init_var is None else init_var

    if lead is not None:
        x = _normal(rng, lead + (H, P), 1.0)
        dt = _dt(rng, lead + (H,))
    else:
        x = np.zeros((0,), np.float32)
        dt = np.zeros((0,), np.float32)
    u = rng.uniform(0.0, math.log(16.0), size=H).astype(np.float32)
    A = (-np.exp(u)).astype(np.float32)
    if A_range is not None:
        A = rng.uniform(A_range[0], A_range[1], size=H).astype(np.float32)
    if A_zero:
        A = np.zeros(H, np.float32)
    if A_values is not None:
        A = np.resize(np.asarray(A_values, np.float32), H).astype(np.float32)
    if lead is not None:
        B = _normal(rng, lead + (G, N), 1.0 / N)
        C = _normal(rng, lead + (G, N), 1.0 / N)
    else:
        B = np.zeros((0,), np.float32)
        C = np.zeros((0,), np.float32)
    D = _normal(rng, (H,), 1.0)
    init = _normal(rng, (nseq, H, P, N), ivar) if ivar > 0 else None
    dec: List[Dict[str, np.ndarray]] = []
    for _ in range(steps):
        dec.append(dict(x=_normal(rng, (nseq, H, P), 1.0), dt=_dt(rng, (nseq, H)),
                        B=_normal(rng, (nseq, G, N), 1.0 / N),
                        C=_normal(rng, (nseq, G, N), 1.0 / N)))
    if x_zero:
        x = np.zeros_like(x)
    if wl.dtype == "bf16":
        x = round_bf16(x)
        B = round_bf16(B)
        C = round_bf16(C)
        for d in dec:
            d["x"] = round_bf16(d["x"])
            d["B"] = round_bf16(d["B"])
            d["C"] = round_bf16(d["C"])
    return Inputs(wl, x, dt, A, B, C, D, init, cu, dec)


def small_workload(*, batch=1, seqlen=0, seqlens=None, H=4, P=16, N=16, G=1, chunk=64,
                   dtype="f32", init_var=0.0, decode_steps=0, decode_batch=0) -> Workload:
    """An ad-hoc workload for tests (same distributions as the named ones)."""
    tag = "seqlens=%s" % (list(seqlens),) if seqlens is not None else "b%d L%d" % (batch, seqlen)
    return Workload("custom %s H%d P%d N%d G%d Q%d %s" % (tag, H, P, N, G, chunk, dtype), H=H,
                    P=P, N=N, G=G, dtype=dtype, batch=batch, seqlen=seqlen,
                    seqlens=None if seqlens is None else tuple(seqlens), chunk=chunk,
                    init_var=init_var, decode_steps=decode_steps, decode_batch=decode_batch)


# ---------------------------------------------------------------- conv1d inputs
@dataclasses.dataclass
class ConvInputs:
    """Host inputs of the causal conv1d (fp32 arrays holding exactly the values
    the GPU receives)."""
    x: np.ndarray                     # [b, L, C] dense or [T, C] packed
    weight: np.ndarray                # [C, K]
    bias: Optional[np.ndarray]        # [C]
    state: Optional[np.ndarray]       # [nseq, K-1, C]
    cu_seqlens: Optional[np.ndarray]  # int32 [nseq+1] when packed


def conv_inputs(seed: int, *, C: int, K: int = 4, batch: int = 1, seqlen: int = 0,
                seqlens: Optional[Sequence[int]] = None, dtype: str = "bf16", bias: bool = True,
                state: bool = True) -> ConvInputs:
    """Draw conv1d inputs.  x and the incoming states ~ N(0,1); weight and
    bias ~ U(-1/sqrt(K), 1/sqrt(K)) (the usual fan-in bound of a depthwise
    conv).  Draw order: x, weight, bias, state.  Dense [batch, seqlen, C]
    unless ``seqlens`` is given (packed [T, C] with cu_seqlens)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if seqlens is not None:
        cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
        lead = (int(cu[-1]),)
        nseq = len(seqlens)
    else:
        cu = None
        lead = (batch, seqlen)
        nseq = batch
    bound = np.float32(1.0 / math.sqrt(K))
    x = _normal(rng, lead + (C,), 1.0)
    w = rng.uniform(-bound, bound, size=(C, K)).astype(np.float32)
    b = rng.uniform(-bound, bound, size=C).astype(np.float32) if bias else None
    st = _normal(rng, (nseq, K - 1, C), 1.0) if state else None
    if dtype == "bf16":
        x = round_bf16(x)
        if st is not None:
            st = round_bf16(st)
    return ConvInputs(x, w, b, st, cu)
