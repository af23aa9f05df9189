"""Exact windowed decode on the GPU against the oracle: a decode session of
several windows, every token's output and the state after every flush,
compared with the sequential fp64 recurrence."""
import sys

import numpy as np
import pytest
import torch

import oracle
import mamba_ssd_chunked_02_amd as ssd
from mamba_ssd_chunked_02_amd import workloads as W
from parity import assert_close, host, tdev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,P,N,G,window,act", [
    ("bf16", 64, 128, 1, 16, False),
    ("f32", 32, 64, 2, 5, False),
    ("bf16", 24, 40, 3, 1, False),
    ("f32", 64, 128, 2, 16, True),
    ("bf16", 128, 256, 1, 16, False),
])
def test_window_session_matches_sequential_decode(dtype, P, N, G, window, act):
    steps = 2 * window + 3 if window > 1 else 4  # two full windows and a partial one
    b, H = 3, 6
    wl = W.small_workload(batch=b, seqlen=0, H=H, P=P, N=N, G=G, dtype=dtype, init_var=0.1,
                          decode_steps=steps, decode_batch=b)
    inp = W.generate(wl, 60 + window)
    say("case: window session", dtype, P, N, G, window, act)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(window)
    bias = rng.normal(0.0, 0.5, size=H).astype(np.float32)
    state = tdev(inp.init)
    xw = torch.zeros((b, window, H, P), dtype=tdt, device="cuda")
    dtw = torch.zeros((b, window, H), device="cuda")
    Bw = torch.zeros((b, window, G, N), dtype=tdt, device="cuda")
    Cw = torch.zeros((b, window, G, N), dtype=tdt, device="cuda")
    A, D = tdev(inp.A), tdev(inp.D)
    ref = inp.init.astype(np.float64)
    kw = dict(dt_softplus=True, dt_bias=tdev(bias), dt_limit=(0.0, 0.2)) if act else {}
    t = 0
    for k, d in enumerate(inp.decode):
        raw = rng.normal(-4.0, 1.0, size=d["dt"].shape).astype(np.float32) if act else d["dt"]
        xw[:, t].copy_(tdev(d["x"], dtype))
        dtw[:, t].copy_(tdev(raw))
        Bw[:, t].copy_(tdev(d["B"], dtype))
        Cw[:, t].copy_(tdev(d["C"], dtype))
        flush = t == window - 1 or k == steps - 1
        y = ssd.decode_window_step(state, xw, dtw, A, Bw, Cw, D, t, flush, **kw)
        dt_used = oracle.dt_activation(raw, bias, (0.0, 0.2)) if act else d["dt"]
        yr, ref = oracle.decode(ref, d["x"], dt_used, inp.A, d["B"], d["C"], inp.D)
        torch.cuda.synchronize()
        assert_close(host(y), yr, dtype, "y token %d (slot %d)" % (k, t))
        if flush:
            assert_close(host(state), ref, dtype, "state after token %d" % k)
            t = 0
        else:
            t += 1


def test_window_step_without_flush_leaves_state_unchanged():
    wl = W.small_workload(batch=2, seqlen=0, H=4, P=32, N=64, G=1, dtype="f32", init_var=0.1,
                          decode_steps=1, decode_batch=2)
    inp = W.generate(wl, 70)
    state = tdev(inp.init)
    before = state.clone()
    d = inp.decode[0]
    xw = tdev(d["x"][:, None])
    y = ssd.decode_window_step(state, xw, tdev(d["dt"][:, None]), tdev(inp.A), tdev(d["B"][:, None]),
                               tdev(d["C"][:, None]), tdev(inp.D), 0, False)
    torch.cuda.synchronize()
    assert torch.equal(state, before)
    y1 = ssd.decode_step(state, tdev(d["x"]), tdev(d["dt"]), tdev(inp.A), tdev(d["B"]), tdev(d["C"]),
                         tdev(inp.D))
    torch.cuda.synchronize()
    assert_close(host(y), host(y1).astype(np.float64), "f32", "window of one vs decode step")


def test_window_step_bf16_output_is_the_rounded_fp32_output():
    """y in bf16 is the same kernel's fp32 y rounded to nearest even, for a
    read-only and a flush step."""
    wl = W.small_workload(batch=3, seqlen=0, H=4, P=64, N=128, G=1, dtype="bf16", init_var=0.1,
                          decode_steps=4, decode_batch=3)
    inp = W.generate(wl, 71)
    W_ = 4
    xw = torch.stack([tdev(d["x"], "bf16") for d in inp.decode], dim=1).contiguous()
    dtw = torch.stack([tdev(d["dt"]) for d in inp.decode], dim=1).contiguous()
    Bw = torch.stack([tdev(d["B"], "bf16") for d in inp.decode], dim=1).contiguous()
    Cw = torch.stack([tdev(d["C"], "bf16") for d in inp.decode], dim=1).contiguous()
    A, D = tdev(inp.A), tdev(inp.D)
    for t, flush in ((1, False), (W_ - 1, True)):
        s32 = tdev(inp.init)
        s16 = tdev(inp.init)
        y32 = ssd.decode_window_step(s32, xw, dtw, A, Bw, Cw, D, t, flush)
        y16 = ssd.decode_window_step(s16, xw, dtw, A, Bw, Cw, D, t, flush, y_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert y16.dtype == torch.bfloat16
        assert torch.equal(y16, y32.to(torch.bfloat16)), (t, flush)
        assert torch.equal(s16, s32)
