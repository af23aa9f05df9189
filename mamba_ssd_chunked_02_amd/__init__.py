"""MI355X (gfx950) Mamba-2 SSD selective scan: Python binding of libssd_mi355x.so.

The binding only marshals arguments: every step of the scan runs in the HIP
kernels behind the C ABI of ``include/ssd.h``.  PyTorch supplies device
memory and the current stream; nothing here computes on the CPU, and there is
no fallback: if the library is missing or a call fails, an exception says so.

    y, final_state = chunked_scan(x, dt, A, B, C, D, chunk, init_state=None,
                                  cu_seqlens=None)
    y = decode_step(state, x, dt, A, B, C, D)          # state updated in place

Shapes: dense x [b, L, H, P], dt [b, L, H], B/C [b, L, G, N]; packed
(``cu_seqlens`` int32 [nseq+1]) x [T, H, P], dt [T, H], B/C [T, G, N].
A, D [H]; states [nseq, H, P, N] fp32.  x/B/C/y share one dtype (float32 or
bfloat16); dt, A, D and states are float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

__all__ = ["chunked_scan", "chunked_scan_noalloc", "decode_step", "decode_window_step", "causal_conv1d",
           "conv1d_step", "workspace_size", "SsdError", "library_path", "load"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libssd_mi355x.so"
_lib = None

SSD_F32 = 0
SSD_BF16 = 1


class SsdError(RuntimeError):
    """A status other than SSD_OK from the C ABI."""

    def __init__(self, status: int, what: str, detail: str):
        super().__init__("%s failed: %s (%d): %s" % (what, _status_name(status), status, detail))
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int32),
                ("headdim", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("dtype", ctypes.c_int32), ("ydtype", ctypes.c_int32),
                ("path", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p),
                ("cu_seqlens_host", ctypes.c_void_p)]


class _ConvShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("channels", ctypes.c_int32),
                ("width", ctypes.c_int32), ("dtype", ctypes.c_int32), ("ydtype", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p)]


class _ConvOutputs(ctypes.Structure):
    _fields_ = [("nparts", ctypes.c_int32), ("channels", ctypes.c_int32 * 3), ("out", ctypes.c_void_p * 3)]


class _DtAct(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float)]


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError("%s is not built; run `python -m mamba_ssd_chunked_02_amd.build`"
                               % path)
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        sp = ctypes.POINTER(_Shape)
        lib.ssd_chunked_scan_workspace_size.argtypes = [sp, ctypes.c_int32,
                                                        ctypes.POINTER(ctypes.c_size_t)]
        lib.ssd_chunked_scan_workspace_size.restype = ctypes.c_int32
        lib.ssd_chunked_scan.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp, sp, vp,
                                         ctypes.c_size_t, vp]
        lib.ssd_chunked_scan.restype = ctypes.c_int32
        lib.ssd_chunked_scan_profiled.argtypes = lib.ssd_chunked_scan.argtypes + [
            ctypes.POINTER(ctypes.c_float)]
        lib.ssd_chunked_scan_profiled.restype = ctypes.c_int32
        lib.ssd_chunked_scan_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp, sp, vp]
        lib.ssd_chunked_scan_noalloc.restype = ctypes.c_int32
        lib.ssd_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sp, vp]
        lib.ssd_decode_step.restype = ctypes.c_int32
        ap = ctypes.POINTER(_DtAct)
        lib.ssd_chunked_scan_dt_act.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp, ap, sp,
                                                vp, ctypes.c_size_t, vp]
        lib.ssd_chunked_scan_dt_act.restype = ctypes.c_int32
        lib.ssd_decode_step_dt_act.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ap, sp, vp]
        lib.ssd_decode_step_dt_act.restype = ctypes.c_int32
        lib.ssd_decode_window_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, ap, sp, vp]
        lib.ssd_decode_window_step.restype = ctypes.c_int32
        csp = ctypes.POINTER(_ConvShape)
        cop = ctypes.POINTER(_ConvOutputs)
        lib.ssd_causal_conv1d.argtypes = [vp, vp, vp, vp, vp, cop, csp, vp]
        lib.ssd_causal_conv1d.restype = ctypes.c_int32
        lib.ssd_causal_conv1d_step.argtypes = [vp, vp, vp, vp, cop, csp, vp]
        lib.ssd_causal_conv1d_step.restype = ctypes.c_int32
        lib.ssd_status_string.argtypes = [ctypes.c_int32]
        lib.ssd_status_string.restype = ctypes.c_char_p
        lib.ssd_last_error_detail.argtypes = []
        lib.ssd_last_error_detail.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _status_name(st: int) -> str:
    try:
        return load().ssd_status_string(st).decode()
    except Exception:  # pragma: no cover
        return "status"


def _check(st: int, what: str):
    if st != 0:
        raise SsdError(st, what, load().ssd_last_error_detail().decode())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError("x/B/C must be float32 or bfloat16, got %s" % t.dtype)


def _dtype_code_of(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return SSD_F32
    if dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError("y must be float32 or bfloat16, got %s" % dtype)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _expect(t, shape, dtype, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream_handle(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def make_shape(x, B, cu_seqlens=None, cu_seqlens_host=None, nseq: Optional[int] = None,
               y_dtype=None, path: str = "auto") -> Tuple[_Shape, object]:
    """Build the C shape struct from tensors.  Returns (shape, keepalive)."""
    sh = _Shape()
    if path not in PATHS:
        raise ValueError("path must be one of %s" % sorted(PATHS))
    sh.path = PATHS[path]
    keep = None
    if cu_seqlens is None:
        b, L, H, P = x.shape
        sh.batch, sh.seqlen = b, L
    else:
        T, H, P = x.shape
        sh.batch = cu_seqlens.shape[0] - 1 if nseq is None else nseq
        sh.seqlen = T
        sh.cu_seqlens = cu_seqlens.data_ptr()
        if cu_seqlens_host is not None:
            import numpy as np
            keep = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
            sh.cu_seqlens_host = keep.ctypes.data
    sh.nheads, sh.headdim = H, P
    sh.ngroups, sh.dstate = B.shape[-2], B.shape[-1]
    sh.dtype = _dtype_code(x)
    sh.ydtype = SSD_F32 if y_dtype is None else _dtype_code_of(y_dtype)
    return sh, keep


def workspace_size(x, B, chunk: int, cu_seqlens=None, cu_seqlens_host=None, path: str = "auto",
                   y_dtype=None) -> int:
    """Workspace bytes for a chunked_scan call with the same arguments (the
    kernel path, and so the size, can depend on the host copy of the offsets)."""
    sh, keep = make_shape(x, B, cu_seqlens, cu_seqlens_host, y_dtype=y_dtype, path=path)
    n = ctypes.c_size_t(0)
    _check(load().ssd_chunked_scan_workspace_size(ctypes.byref(sh), int(chunk), ctypes.byref(n)),
           "ssd_chunked_scan_workspace_size")
    del keep
    return int(n.value)


STAGES = ("plan", "cumsum", "cb", "chunk_state", "state_passing", "chunk_scan", "scan_walk")

# Kernel paths of the prefill (ssd_path in include/ssd.h); "auto" lets the
# library choose.
PATHS = {"auto": 0, "chunk_parallel": 1, "state_walk": 2, "scan_walk": 3}


def _dt_act(dt_softplus, dt_bias, dt_limit, H):
    """ssd_dt_activation for the *_dt_act entry points, or None."""
    if not dt_softplus:
        if dt_bias is not None or dt_limit is not None:
            raise ValueError("dt_bias / dt_limit need dt_softplus=True")
        return None
    torch = _torch()
    if dt_bias is not None:
        _need_cuda(dt_bias)
        _expect(dt_bias, (H,), torch.float32, "dt_bias")
    lo, hi = (0.0, float("inf")) if dt_limit is None else dt_limit
    act = _DtAct()
    act.dt_bias = _ptr(dt_bias)
    act.dt_min, act.dt_max = float(lo), float(hi)
    return act


def chunked_scan(x, dt, A, B, C, D, chunk: int = 256, init_state=None, cu_seqlens=None, *,
                 y=None, final_state=None, want_final: bool = True, workspace=None,
                 cu_seqlens_host: Optional[Sequence[int]] = None,
                 stage_ms: Optional[list] = None, y_dtype=None,
                 dt_softplus: bool = False, dt_bias=None, dt_limit=None, path: str = "auto"):
    """Chunked prefill.  Returns (y, final_state or None).

    ``path``: one of ``PATHS`` ("auto" by default), the kernels that compute
    the chunk states, their passing and y (the same result up to fp32
    rounding order).

    ``dt_softplus``: ``dt`` holds raw step sizes and the kernels use
    ``clamp(softplus(dt + dt_bias[h]), *dt_limit)`` (``dt_bias`` [H] fp32 or
    None, ``dt_limit`` (lo, hi), default (0, inf)).

    ``cu_seqlens`` (packed batch) may be a GPU int32 tensor or a host sequence;
    a host sequence is copied to the GPU and also validated on the host.
    ``workspace`` (uint8 GPU tensor) is allocated when not given.
    ``stage_ms``: when a list is given, the call goes through the measuring
    entry point (it blocks until the kernels finish) and the list receives the
    duration in ms of each stage named in ``STAGES``.
    ``y_dtype``: torch.float32 (default) or torch.bfloat16.
    """
    torch = _torch()
    _need_cuda(x, dt, A, B, C, D, init_state)
    host_cu = cu_seqlens_host
    if cu_seqlens is not None and not (hasattr(cu_seqlens, "is_cuda") and cu_seqlens.is_cuda):
        host_cu = list(int(v) for v in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist")
                                        else cu_seqlens))
        cu_seqlens = torch.tensor(host_cu, dtype=torch.int32, device=x.device)
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if y_dtype is None:
        y_dtype = torch.float32 if y is None else y.dtype
    sh, keep = make_shape(x, B, cu_seqlens, host_cu, y_dtype=y_dtype, path=path)
    nseq = sh.batch
    H, P, N = sh.nheads, sh.headdim, sh.dstate
    lead = tuple(x.shape[:-2])
    _expect(dt, lead + (H,), torch.float32, "dt")
    _expect(B, lead + (sh.ngroups, N), x.dtype, "B")
    _expect(C, lead + (sh.ngroups, N), x.dtype, "C")
    _expect(A, (H,), torch.float32, "A")
    _expect(D, (H,), torch.float32, "D")
    _expect(init_state, (nseq, H, P, N), torch.float32, "init_state")
    _expect(y, tuple(x.shape), y_dtype, "y")
    _expect(final_state, (nseq, H, P, N), torch.float32, "final_state")
    if cu_seqlens is not None:
        _expect(cu_seqlens, (nseq + 1,), torch.int32, "cu_seqlens")
    if y is None:
        y = torch.empty(tuple(x.shape), dtype=y_dtype, device=x.device)
    if final_state is None and want_final:
        final_state = torch.empty((nseq, H, P, N), dtype=torch.float32, device=x.device)
    lib = load()
    nbytes = ctypes.c_size_t(0)
    _check(lib.ssd_chunked_scan_workspace_size(ctypes.byref(sh), int(chunk), ctypes.byref(nbytes)),
           "ssd_chunked_scan_workspace_size")
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(int(nbytes.value), dtype=torch.uint8, device=x.device)
    act = _dt_act(dt_softplus, dt_bias, dt_limit, H)
    if act is not None:
        if stage_ms is not None:
            raise ValueError("stage_ms is not available with dt_softplus")
        _check(lib.ssd_chunked_scan_dt_act(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), int(chunk),
                                           _ptr(init_state), _ptr(y), _ptr(final_state), ctypes.byref(act),
                                           ctypes.byref(sh), _ptr(workspace), int(workspace.numel()),
                                           _stream_handle(x)), "ssd_chunked_scan_dt_act")
        del keep
        return y, final_state
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), int(chunk), _ptr(init_state),
            _ptr(y), _ptr(final_state), ctypes.byref(sh), _ptr(workspace), int(workspace.numel()),
            _stream_handle(x))
    if stage_ms is None:
        _check(lib.ssd_chunked_scan(*args), "ssd_chunked_scan")
    else:
        out = (ctypes.c_float * len(STAGES))()
        _check(lib.ssd_chunked_scan_profiled(*args, out), "ssd_chunked_scan_profiled")
        stage_ms[:] = [float(v) for v in out]
    del keep
    return y, final_state


NOALLOC_SCRATCH_BYTES = 64 << 20  # SSD_NOALLOC_SCRATCH_BYTES of include/ssd.h


def chunked_scan_noalloc(x, dt, A, B, C, D, chunk: int, y, final_state=None, init_state=None,
                         cu_seqlens=None, cu_seqlens_host: Optional[Sequence[int]] = None, path: str = "auto"):
    """ssd_chunked_scan_noalloc: the chunked prefill with the library's own
    device scratch array as its workspace (no allocation anywhere: ``y`` and,
    when wanted, ``final_state`` are given by the caller).  Same shapes as
    ``chunked_scan``; ``cu_seqlens`` must already be a GPU int32 tensor."""
    torch = _torch()
    _need_cuda(x, dt, A, B, C, D, init_state, y, final_state)
    if cu_seqlens is not None and not (hasattr(cu_seqlens, "is_cuda") and cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be a GPU tensor here (copying it would allocate)")
    sh, keep = make_shape(x, B, cu_seqlens, cu_seqlens_host, y_dtype=y.dtype, path=path)
    H, P, N = sh.nheads, sh.headdim, sh.dstate
    lead = tuple(x.shape[:-2])
    _expect(dt, lead + (H,), torch.float32, "dt")
    _expect(B, lead + (sh.ngroups, N), x.dtype, "B")
    _expect(C, lead + (sh.ngroups, N), x.dtype, "C")
    _expect(A, (H,), torch.float32, "A")
    _expect(D, (H,), torch.float32, "D")
    _expect(init_state, (sh.batch, H, P, N), torch.float32, "init_state")
    _expect(y, tuple(x.shape), y.dtype, "y")
    _expect(final_state, (sh.batch, H, P, N), torch.float32, "final_state")
    _check(load().ssd_chunked_scan_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), int(chunk),
                                           _ptr(init_state), _ptr(y), _ptr(final_state), ctypes.byref(sh),
                                           _stream_handle(x)), "ssd_chunked_scan_noalloc")
    del keep
    return y, final_state


def decode_step(state, x, dt, A, B, C, D, *, y=None, y_dtype=None, dt_softplus: bool = False,
                dt_bias=None, dt_limit=None):
    """One cached decode step; ``state`` [b, H, P, N] fp32 is updated in place.
    ``y_dtype``: torch.float32 (default) or torch.bfloat16.  ``dt_softplus``,
    ``dt_bias``, ``dt_limit``: as for chunked_scan."""
    torch = _torch()
    if y_dtype is None:
        y_dtype = torch.float32 if y is None else y.dtype
    _need_cuda(state, x, dt, A, B, C, D)
    b, H, P = x.shape
    G, N = B.shape[-2], B.shape[-1]
    _expect(state, (b, H, P, N), torch.float32, "state")
    _expect(dt, (b, H), torch.float32, "dt")
    _expect(B, (b, G, N), x.dtype, "B")
    _expect(C, (b, G, N), x.dtype, "C")
    _expect(A, (H,), torch.float32, "A")
    _expect(D, (H,), torch.float32, "D")
    _expect(y, (b, H, P), y_dtype, "y")
    sh = _Shape()
    sh.batch, sh.seqlen = b, 1
    sh.nheads, sh.headdim = H, P
    sh.ngroups, sh.dstate = B.shape[-2], B.shape[-1]
    sh.dtype = _dtype_code(x)
    sh.ydtype = _dtype_code_of(y_dtype)
    if y is None:
        y = torch.empty((b, H, P), dtype=y_dtype, device=x.device)
    act = _dt_act(dt_softplus, dt_bias, dt_limit, H)
    if act is not None:
        st = load().ssd_decode_step_dt_act(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                           _ptr(y), ctypes.byref(act), ctypes.byref(sh), _stream_handle(x))
        _check(st, "ssd_decode_step_dt_act")
        return y
    st = load().ssd_decode_step(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                _ptr(y), ctypes.byref(sh), _stream_handle(x))
    _check(st, "ssd_decode_step")
    return y


def decode_window_step(state, x, dt, A, B, C, D, t: int, flush: bool, *, y=None, y_dtype=None,
                       dt_softplus: bool = False, dt_bias=None, dt_limit=None):
    """Exact windowed decode step: output of the token in window slot ``t``.

    ``state`` [b, H, P, N] fp32 is the state at the window start (rewritten to
    the state after token ``t`` when ``flush``); ``x`` [b, W, H, P], ``dt``
    [b, W, H], ``B``/``C`` [b, W, G, N] hold the window's tokens in slots
    0..t.  W = x.shape[1] <= 16.  Returns y [b, H, P]."""
    torch = _torch()
    if y_dtype is None:
        y_dtype = torch.float32 if y is None else y.dtype
    _need_cuda(state, x, dt, A, B, C, D)
    b, W, H, P = x.shape
    G, N = B.shape[-2], B.shape[-1]
    _expect(state, (b, H, P, N), torch.float32, "state")
    _expect(dt, (b, W, H), torch.float32, "dt")
    _expect(B, (b, W, G, N), x.dtype, "B")
    _expect(C, (b, W, G, N), x.dtype, "C")
    _expect(A, (H,), torch.float32, "A")
    _expect(D, (H,), torch.float32, "D")
    _expect(y, (b, H, P), y_dtype, "y")
    sh = _Shape()
    sh.batch, sh.seqlen = b, 1
    sh.nheads, sh.headdim = H, P
    sh.ngroups, sh.dstate = G, N
    sh.dtype = _dtype_code(x)
    sh.ydtype = _dtype_code_of(y_dtype)
    if y is None:
        y = torch.empty((b, H, P), dtype=y_dtype, device=x.device)
    act = _dt_act(dt_softplus, dt_bias, dt_limit, H)
    st = load().ssd_decode_window_step(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                       _ptr(y), int(W), int(t), 1 if flush else 0,
                                       None if act is None else ctypes.byref(act), ctypes.byref(sh),
                                       _stream_handle(x))
    _check(st, "ssd_decode_window_step")
    return y


def _conv_outputs(lead, C, split, outs, y_dtype, device):
    """The output parts: given tensors, or new ones [*lead, channels_p]."""
    torch = _torch()
    split = [C] if split is None else [int(c) for c in split]
    if sum(split) != C:
        raise ValueError("split %s does not add up to %d channels" % (split, C))
    if outs is None:
        outs = [torch.empty(tuple(lead) + (c,), dtype=y_dtype, device=device) for c in split]
    if len(outs) != len(split):
        raise ValueError("%d output tensors for %d parts" % (len(outs), len(split)))
    co = _ConvOutputs()
    co.nparts = len(split)
    for p, (c, o) in enumerate(zip(split, outs)):
        _expect(o, tuple(lead) + (c,), o.dtype, "output part %d" % p)
        if o.dtype != y_dtype:
            raise TypeError("output part %d has dtype %s, expected %s" % (p, o.dtype, y_dtype))
        co.channels[p] = c
        co.out[p] = _ptr(o)
    return co, outs


def causal_conv1d(x, weight, bias=None, *, cu_seqlens=None, cu_seqlens_host=None, conv_state=None,
                  final_conv_state=None, activation: bool = True, split: Optional[Sequence[int]] = None,
                  outs=None, y_dtype=None):
    """Causal depthwise conv1d (+ SiLU) over whole sequences.

    x: dense [b, L, C] or packed [T, C] with ``cu_seqlens`` int32 [b+1];
    weight [C, K] fp32 (tap K-1 on the current token); bias [C] fp32 or None;
    conv_state [b, K-1, C] (x's dtype) or None; final_conv_state, if given,
    receives the state after each sequence (it may be conv_state itself).
    ``split`` lists channel counts of consecutive output parts (default: one
    part of C channels); returns the list of parts [*x.shape[:-1], c_p]."""
    torch = _torch()
    _need_cuda(x, weight, bias, conv_state, final_conv_state, cu_seqlens)
    C = x.shape[-1]
    K = weight.shape[-1]
    if y_dtype is None:
        y_dtype = x.dtype if outs is None else outs[0].dtype
    _expect(weight, (C, K), torch.float32, "weight")
    _expect(bias, (C,), torch.float32, "bias")
    sh = _ConvShape()
    keep = None
    if cu_seqlens is None:
        if x.dim() != 3:
            raise ValueError("dense x must be [b, L, C]")
        sh.batch, sh.seqlen = x.shape[0], x.shape[1]
    else:
        if x.dim() != 2:
            raise ValueError("packed x must be [T, C]")
        _expect(cu_seqlens, (cu_seqlens.shape[0],), torch.int32, "cu_seqlens")
        sh.batch, sh.seqlen = cu_seqlens.shape[0] - 1, x.shape[0]
        sh.cu_seqlens = cu_seqlens.data_ptr()
        if cu_seqlens_host is not None:
            import numpy as np
            keep = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
            sh.cu_seqlens_host = keep.ctypes.data
    nseq = sh.batch
    _expect(conv_state, (nseq, K - 1, C), x.dtype, "conv_state")
    _expect(final_conv_state, (nseq, K - 1, C), x.dtype, "final_conv_state")
    sh.channels, sh.width = C, K
    sh.dtype = _dtype_code(x)
    sh.ydtype = _dtype_code_of(y_dtype)
    sh.activation = 1 if activation else 0
    co, outs = _conv_outputs(x.shape[:-1], C, split, outs, y_dtype, x.device)
    st = load().ssd_causal_conv1d(_ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state), _ptr(final_conv_state),
                                  ctypes.byref(co), ctypes.byref(sh), _stream_handle(x))
    del keep
    _check(st, "ssd_causal_conv1d")
    return outs


def conv1d_step(conv_state, x, weight, bias=None, *, activation: bool = True,
                split: Optional[Sequence[int]] = None, outs=None, y_dtype=None):
    """One decode token per sequence: x [b, C]; conv_state [b, K-1, C] is
    shifted in place (oldest row out, x in).  Returns the output parts [b, c_p]."""
    torch = _torch()
    _need_cuda(conv_state, x, weight, bias)
    b, C = x.shape
    K = weight.shape[-1]
    if y_dtype is None:
        y_dtype = x.dtype if outs is None else outs[0].dtype
    _expect(weight, (C, K), torch.float32, "weight")
    _expect(bias, (C,), torch.float32, "bias")
    _expect(conv_state, (b, K - 1, C), x.dtype, "conv_state")
    sh = _ConvShape()
    sh.batch, sh.seqlen = b, 1
    sh.channels, sh.width = C, K
    sh.dtype = _dtype_code(x)
    sh.ydtype = _dtype_code_of(y_dtype)
    sh.activation = 1 if activation else 0
    co, outs = _conv_outputs((b,), C, split, outs, y_dtype, x.device)
    st = load().ssd_causal_conv1d_step(_ptr(conv_state), _ptr(x), _ptr(weight), _ptr(bias), ctypes.byref(co),
                                       ctypes.byref(sh), _stream_handle(x))
    _check(st, "ssd_causal_conv1d_step")
    return outs
