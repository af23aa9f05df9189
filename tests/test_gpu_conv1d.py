"""Causal conv1d + SiLU on the GPU against the fp64 oracle (oracle.conv):
dense and packed batches with ragged lengths (empty, shorter than the
window, several token blocks plus a tail), incoming and final conv states
(also updated in place), split outputs, the decode step, and the 2.7B-layer
channel count on sampled channels."""
import sys

import numpy as np
import pytest
import torch

from oracle import conv as oconv
import mamba_ssd_chunked_02_amd as ssd
from mamba_ssd_chunked_02_amd import workloads as W
from parity import assert_close, host, tdev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_inputs(ci, dtype):
    g = dict(x=tdev(ci.x, dtype), weight=tdev(ci.weight),
             bias=None if ci.bias is None else tdev(ci.bias),
             state=None if ci.state is None else tdev(ci.state, dtype))
    if ci.cu_seqlens is not None:
        g["cu"] = torch.from_numpy(ci.cu_seqlens).cuda()
    return g


def check_y(run, yr, dtype, ydtype, what="y"):
    """Parity of the arithmetic on the fp32 output (the stated tolerance for
    the input dtype); a bf16 output must be exactly that output rounded to
    nearest even (the same kernel, narrowed at the store)."""
    y32 = run(torch.float32)
    torch.cuda.synchronize()
    assert_close(host(y32), yr, dtype, what)
    if ydtype == "bf16":
        y16 = run(torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(y16, y32.to(torch.bfloat16)), what + ": bf16 output is not the rounded fp32 output"


DENSE = [
    # b, L, C, K, dtype, ydtype, silu, bias, state
    (2, 100, 64, 4, "bf16", "bf16", True, True, True),
    (3, 1, 8, 4, "f32", "f32", True, True, True),
    (1, 2, 24, 3, "f32", "f32", False, False, True),
    (2, 130, 520, 4, "f32", "f32", True, True, False),
    (1, 200, 1040, 2, "bf16", "f32", True, True, True),
    (4, 64, 512, 4, "bf16", "bf16", False, True, True),
]


@pytest.mark.parametrize("b,L,C,K,dtype,ydtype,silu,bias,state", DENSE)
def test_conv1d_dense(b, L, C, K, dtype, ydtype, silu, bias, state):
    say("case: conv dense", b, L, C, K, dtype, ydtype, silu, bias, state)
    ci = W.conv_inputs(300 + L + C, C=C, K=K, batch=b, seqlen=L, dtype=dtype, bias=bias, state=state)
    g = gpu_inputs(ci, dtype)
    fin = torch.empty((b, K - 1, C), dtype=g["x"].dtype, device="cuda")

    def run(ydt):
        return ssd.causal_conv1d(g["x"], g["weight"], g["bias"], conv_state=g["state"], final_conv_state=fin,
                                 activation=silu, y_dtype=ydt)[0]
    yr, fr = oconv.causal_conv1d_batch(ci.x, ci.weight, ci.bias, ci.state, activation=silu)
    check_y(run, yr, dtype, ydtype)
    assert np.array_equal(host(fin), fr), "final conv state (exact copies of inputs)"


PACKED = [
    # lens, C, K, dtype, state
    ([5, 0, 1, 70, 2, 130, 0], 64, 4, "bf16", True),
    ([0, 0, 3], 16, 4, "f32", True),
    ([64, 64, 1, 63, 65], 136, 4, "f32", False),
    ([200, 3, 0, 129], 32, 3, "bf16", True),
]


@pytest.mark.parametrize("lens,C,K,dtype,state", PACKED)
def test_conv1d_packed(lens, C, K, dtype, state):
    say("case: conv packed", lens, C, K, dtype, state)
    ci = W.conv_inputs(400 + C, C=C, K=K, seqlens=lens, dtype=dtype, state=state)
    g = gpu_inputs(ci, dtype)
    n = len(lens)
    fin = torch.empty((n, K - 1, C), dtype=g["x"].dtype, device="cuda")
    (y,) = ssd.causal_conv1d(g["x"], g["weight"], g["bias"], cu_seqlens=g["cu"], cu_seqlens_host=ci.cu_seqlens,
                             conv_state=g["state"], final_conv_state=fin, y_dtype=torch.float32)
    yr, fr = oconv.causal_conv1d_batch(ci.x, ci.weight, ci.bias, ci.state, cu_seqlens=ci.cu_seqlens)
    torch.cuda.synchronize()
    assert_close(host(y), yr, dtype, "y")
    assert np.array_equal(host(fin), fr), "final conv state"


def test_conv1d_state_in_place_and_split_outputs():
    say("case: conv in place + split")
    b, L, K = 3, 77, 4
    parts = [256, 16, 16]
    C = sum(parts)
    ci = W.conv_inputs(501, C=C, K=K, batch=b, seqlen=L, dtype="bf16")
    g = gpu_inputs(ci, "bf16")
    (whole,) = ssd.causal_conv1d(g["x"], g["weight"], g["bias"], conv_state=g["state"])
    st = g["state"].clone()
    xs, bs, cs = ssd.causal_conv1d(g["x"], g["weight"], g["bias"], conv_state=st, final_conv_state=st,
                                   split=parts)
    _, fr = oconv.causal_conv1d_batch(ci.x, ci.weight, ci.bias, ci.state)
    torch.cuda.synchronize()
    assert xs.shape == (b, L, 256) and bs.shape == (b, L, 16)
    assert torch.equal(torch.cat([xs, bs, cs], dim=-1), whole)
    assert np.array_equal(host(st), fr)


def test_conv1d_steps_continue_the_prefill():
    say("case: conv prefill + decode steps")
    b, L, C, K, steps = 4, 37, 96, 4, 9
    ci = W.conv_inputs(502, C=C, K=K, batch=b, seqlen=L + steps, dtype="bf16")
    g = gpu_inputs(ci, "bf16")
    st = g["state"].clone()
    (y0,) = ssd.causal_conv1d(g["x"][:, :L].contiguous(), g["weight"], g["bias"], conv_state=st,
                              final_conv_state=st, y_dtype=torch.float32)
    ys = [y0]
    for t in range(steps):
        (yt,) = ssd.conv1d_step(st, g["x"][:, L + t].contiguous(), g["weight"], g["bias"], y_dtype=torch.float32)
        ys.append(yt[:, None])
    yr, fr = oconv.causal_conv1d_batch(ci.x, ci.weight, ci.bias, ci.state)
    torch.cuda.synchronize()
    assert_close(host(torch.cat(ys, dim=1)), yr, "bf16", "prefill then steps")
    assert np.array_equal(host(st), fr)
    # the step in fp32, against the oracle step
    ci2 = W.conv_inputs(503, C=C, K=3, batch=5, seqlen=1, dtype="f32")
    g2 = gpu_inputs(ci2, "f32")
    st2 = g2["state"].clone()
    (y2,) = ssd.conv1d_step(st2, g2["x"][:, 0].contiguous(), g2["weight"], g2["bias"], activation=False)
    yr2, sr2 = oconv.conv1d_step(ci2.state, ci2.x[:, 0], ci2.weight, ci2.bias, activation=False)
    torch.cuda.synchronize()
    assert_close(host(y2), yr2, "f32", "step y")
    assert np.array_equal(host(st2), sr2)


def test_conv1d_2p7b_layer_channels_sampled():
    """xBC of a 2.7B-shaped layer: C = H*P + 2*G*N = 5120 + 256, split into the
    scan's x, B and C; b2 L2048 on 384 sampled channels."""
    say("case: conv 2.7B channels")
    b, L, K = 2, 2048, 4
    parts = [5120, 128, 128]
    C = sum(parts)
    ci = W.conv_inputs(504, C=C, K=K, batch=b, seqlen=L, dtype="bf16")
    g = gpu_inputs(ci, "bf16")
    fin = torch.empty((b, K - 1, C), dtype=torch.bfloat16, device="cuda")
    outs = ssd.causal_conv1d(g["x"], g["weight"], g["bias"], conv_state=g["state"], final_conv_state=fin,
                             split=parts)
    y16 = torch.cat(outs, dim=-1)
    y32 = torch.cat(ssd.causal_conv1d(g["x"], g["weight"], g["bias"], conv_state=g["state"], split=parts,
                                      y_dtype=torch.float32), dim=-1)
    rng = np.random.default_rng(5)
    cols = np.sort(np.concatenate([rng.choice(C, 376, replace=False), [0, 5119, 5120, 5247, 5248, C - 1]]))
    cols = np.unique(cols)
    st = ci.state[:, :, cols]
    yr, fr = oconv.causal_conv1d_batch(ci.x[:, :, cols], ci.weight[cols], ci.bias[cols], st)
    torch.cuda.synchronize()
    assert_close(host(y32)[:, :, cols], yr, "bf16", "y sampled")
    assert torch.equal(y16, y32.to(torch.bfloat16))
    assert np.array_equal(host(fin)[:, :, cols], fr)
