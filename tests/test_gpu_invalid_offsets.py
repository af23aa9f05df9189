"""Device-side sequence offsets that are not a valid offset list (no host
copy to validate them): a sequence whose end precedes its start is empty and
passes its incoming state through; sequences stay inside [0, T]; every
access stays in bounds.  Overlapping sequences write overlapping rows, so y
is checked only on rows one sequence owns."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import conv as oconv
import mamba_ssd_chunked_02_amd as ssd
from mamba_ssd_chunked_02_amd import workloads as W
from parity import assert_close, host, tdev

pytestmark = pytest.mark.gpu

CU = np.array([0, 100, 50, 300], dtype=np.int32)  # sequence 1 decreases: empty; sequence 2 overlaps 0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_prefill_with_decreasing_device_offsets():
    say("case: prefill, device offsets", CU.tolist())
    T, H, P, N = 300, 2, 16, 16
    wl = W.small_workload(seqlens=(100, 0, 200), H=H, P=P, N=N, G=1, chunk=64, dtype="f32", init_var=0.1)
    inp = W.generate(wl, 950)  # inputs for T = 300 rows and 3 sequences
    assert inp.x.shape[0] == T
    cu_dev = torch.from_numpy(CU).cuda()
    y, fin = ssd.chunked_scan(tdev(inp.x), tdev(inp.dt), tdev(inp.A), tdev(inp.B), tdev(inp.C), tdev(inp.D), 64,
                              init_state=tdev(inp.init), cu_seqlens=cu_dev)
    torch.cuda.synchronize()
    fin_h = host(fin)
    assert np.array_equal(fin_h[1], inp.init[1]), "empty sequence keeps its initial state"
    for s, (a, b) in ((0, (0, 100)), (2, (50, 300))):
        yr, fr = oracle.scan(inp.x[None, a:b], inp.dt[None, a:b], inp.A, inp.B[None, a:b], inp.C[None, a:b],
                             inp.D, init=inp.init[s:s + 1])
        assert_close(fin_h[s], fr[0], "f32", "final state of sequence %d" % s)
        if s == 0:
            assert_close(host(y)[0:50], yr[0, 0:50], "f32", "y rows only sequence 0 covers")
        else:
            assert_close(host(y)[100:300], yr[0, 50:250], "f32", "y rows only sequence 2 covers")


def test_conv1d_with_decreasing_device_offsets():
    say("case: conv1d, device offsets", CU.tolist())
    C, K = 16, 4
    ci = W.conv_inputs(951, C=C, K=K, seqlens=(100, 0, 200), dtype="f32")
    cu_dev = torch.from_numpy(CU).cuda()
    fin = torch.empty((3, K - 1, C), device="cuda")
    (y,) = ssd.causal_conv1d(tdev(ci.x), tdev(ci.weight), tdev(ci.bias), cu_seqlens=cu_dev,
                             conv_state=tdev(ci.state), final_conv_state=fin)
    torch.cuda.synchronize()
    yh, fh = host(y), host(fin)
    assert np.all(np.isfinite(yh))
    assert np.array_equal(fh[1], ci.state[1]), "empty sequence keeps its conv state"
    _, f0 = oconv.causal_conv1d(ci.x[0:100], ci.weight, ci.bias, ci.state[0])
    _, f2 = oconv.causal_conv1d(ci.x[50:300], ci.weight, ci.bias, ci.state[2])
    assert np.array_equal(fh[0], f0) and np.array_equal(fh[2], f2)
    y0, _ = oconv.causal_conv1d(ci.x[0:100], ci.weight, ci.bias, ci.state[0])
    assert_close(yh[0:100], y0, "f32", "rows of sequence 0")
