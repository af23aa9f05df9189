"""CPU oracle for the Mamba-2 SSD selective scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it, and it
shares no code with the GPU library (no kernels, headers, helpers or tables).

Contents
--------
``scan`` / ``decode``
    The reference the GPU results are compared with: the plain sequential fp64
    recurrence, written in C (``ssd_oracle.c``) and run with OpenMP over
    (sequence, head) pairs.  It
    follows the per-token recurrence of "Engineering hybrid state-space models"
    (innvotechnologies blog), section 2, with Abar = exp(dt*A) and the input
    term dt*B*x, plus the D skip term of the continuous SSM (lesty.tech Mamba
    explainer, section 2).
``dt_activation``
    The step-size activation that precedes the scan in the Mamba-2 block
    (blog, section 3, architecture figure: Delta = Softplus(Linear(x) +
    bias)), with an optional clamp range, in fp64.
``decode_window``
    The windowed form of the decode step (SketchSSM page, Fig. 3(a), Fig. 4,
    Table 4: read the state of the window start every step, write it once per
    window): output of window token t, and the state after it, from the
    window-start state and the window's tokens.
``conv.causal_conv1d`` / ``conv.causal_conv1d_batch`` / ``conv.conv1d_step``
    The causal depthwise conv1d (width K, optional SiLU) that precedes the
    scan in the Mamba-2 block, with its conv state of K-1 past inputs per
    channel (blog, sections 3 and 4), in fp64: the sum over taps written out.
``quadratic``
    Brute-force quadratic (attention-like) form of the same map, the duality
    statement of the blog's section 2 (Y = (M o CB^T) X with M a 1-semiseparable
    decay mask).  Used only to pin the recurrence on tiny inputs.
``chunked``
    fp64 chunked regrouping (per-chunk decay sums, chunk states, states passed
    between chunks, chunk outputs), the "fixed-size chunking" of
    "Compiler-First State Space Duality..." (abstract) and the blog's section 2
    chunks of Q tokens.  Used to pin chunk-size invariance and to give the
    expected values of intermediate quantities.

Parity pins for every function live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.ssd_oracle_scan.argtypes = [ctypes.c_int64, i64p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, dp, dp, dp, dp, dp, dp,
                                        dp, dp, dp, ctypes.c_int32]
        lib.ssd_oracle_scan.restype = ctypes.c_int
        lib.ssd_oracle_decode.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, dp, dp, dp, dp, dp, dp,
                                          dp, dp, ctypes.c_int32]
        lib.ssd_oracle_decode.restype = ctypes.c_int
        lib.ssd_oracle_threads.argtypes = []
        lib.ssd_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """Number of OpenMP threads the oracle uses by default."""
    return int(_load().ssd_oracle_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def scan(x, dt, A, B, C, D, init=None, cu_seqlens=None, nthreads: int = 0
         ) -> Tuple[np.ndarray, np.ndarray]:
    """Sequential fp64 prefill.

    Dense form: x [b,L,H,P], dt [b,L,H], B/C [b,L,G,N], init [b,H,P,N] or None.
    Packed form (``cu_seqlens`` given, int [nseq+1]): x [T,H,P], dt [T,H],
    B/C [T,G,N], init [nseq,H,P,N] or None.
    Returns (y, final_state) in fp64 with the input's leading layout.
    """
    x = _f64(x)
    dt = _f64(dt)
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    D = _f64(D)
    if cu_seqlens is None:
        b, L, H, P = x.shape
        cu = np.arange(b + 1, dtype=np.int64) * L
        nseq = b
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        nseq = cu.shape[0] - 1
        H, P = x.shape[-2:]
    G, N = B.shape[-2:]
    init64 = None if init is None else _f64(init)
    y = np.zeros(x.shape, dtype=np.float64)
    final = np.zeros((nseq, H, P, N), dtype=np.float64)
    rc = _load().ssd_oracle_scan(nseq, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, P,
                                 N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                 _ptr(init64), _ptr(y), _ptr(final), int(nthreads))
    if rc != 0:
        raise ValueError("oracle scan rejected its arguments")
    return y, final


def dt_activation(dt_raw, dt_bias=None, dt_limit=(0.0, float("inf"))) -> np.ndarray:
    """dt = clamp(softplus(dt_raw + dt_bias), *dt_limit) in fp64.

    softplus(v) = log(1 + exp(v)), evaluated as logaddexp(0, v) so that it
    neither overflows for large v nor loses the tail for very negative v.
    ``dt_bias`` [H] broadcasts over the last axis of ``dt_raw`` [..., H].
    """
    v = _f64(dt_raw)
    if dt_bias is not None:
        v = v + _f64(dt_bias)
    lo, hi = dt_limit
    return np.minimum(np.maximum(np.logaddexp(0.0, v), lo), hi)


def decode(state, x, dt, A, B, C, D, nthreads: int = 0, inplace: bool = False
           ) -> Tuple[np.ndarray, np.ndarray]:
    """One cached decode step: returns (y [b,H,P], new_state [b,H,P,N]) in fp64.

    state [b,H,P,N], x [b,H,P], dt [b,H], B/C [b,G,N].  The input state is not
    modified, unless ``inplace`` is set and it is already a C-contiguous fp64
    array: then it is updated in place and returned (long decode runs over
    large batches avoid a copy of the state per step).
    """
    if inplace and isinstance(state, np.ndarray) and state.dtype == np.float64 and state.flags.c_contiguous:
        st = state
    else:
        st = _f64(state).copy()
    x = _f64(x)
    dt = _f64(dt)
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    D = _f64(D)
    b, H, P, N = st.shape
    G = B.shape[-2]
    y = np.zeros((b, H, P), dtype=np.float64)
    rc = _load().ssd_oracle_decode(b, H, P, N, G, _ptr(st), _ptr(x), _ptr(dt), _ptr(A),
                                   _ptr(B), _ptr(C), _ptr(D), _ptr(y), int(nthreads))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    return y, st


def decode_window(state0, xw, dtw, A, Bw, Cw, D, t: int) -> Tuple[np.ndarray, np.ndarray]:
    """Windowed decode in fp64: (y_t [b,H,P], state after token t [b,H,P,N]).

    state0 [b,H,P,N] is the state at the window start; xw [b,W,H,P], dtw
    [b,W,H], Bw/Cw [b,W,G,N] hold the window's tokens, of which slots 0..t
    are used.  With cs_s = A sum_{u<=s} dt_u over the window,
      y_t   = exp(cs_t) S0 C_t + sum_{s<=t} exp(cs_t - cs_s) dt_s (B_s . C_t) x_s + D x_t
      S_t   = exp(cs_t) S0 + sum_{s<=t} exp(cs_t - cs_s) dt_s x_s (outer) B_s
    (the window treated as one chunk of the regrouping).
    """
    S0 = _f64(state0)
    x = _f64(xw)[:, : t + 1]
    dt = _f64(dtw)[:, : t + 1]
    A = _f64(A)
    D = _f64(D)
    b, H, P, N = S0.shape
    G = Bw.shape[-2]
    grp = np.arange(H) // (H // G)
    Bh = _f64(Bw)[:, : t + 1][:, :, grp]       # [b, s, H, N]
    Ch = _f64(Cw)[:, t][:, grp]                # [b, H, N]
    cs = np.cumsum(dt * A, axis=1)             # [b, s, H]
    dec = np.exp(cs[:, -1:, :] - cs)           # exp(cs_t - cs_s)
    w = dec * dt                               # [b, s, H]
    kern = w * np.einsum("bshn,bhn->bsh", Bh, Ch)
    et = np.exp(cs[:, -1])                     # [b, H]
    y = (et[:, :, None] * np.einsum("bhpn,bhn->bhp", S0, Ch)
         + np.einsum("bsh,bshp->bhp", kern, x) + D[None, :, None] * x[:, -1])
    St = et[:, :, None, None] * S0 + np.einsum("bsh,bshp,bshn->bhpn", w, x, Bh)
    return y, St
