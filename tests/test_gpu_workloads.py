"""GPU parity at the full sizes of the named workloads, in the launch
configuration the benchmark uses (library-chosen segmentation).  Where the
fp64 oracle would take too long on every element, it recomputes sampled
(sequence, head) pairs exactly and those are compared element by element."""
import sys

import numpy as np
import pytest
import torch

import oracle
import mamba_ssd_chunked_02_amd as ssd
from mamba_ssd_chunked_02_amd import workloads as W
from parity import assert_close, host, oracle_scan, tdev, to_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_scan(inp):
    g = to_gpu(inp)
    y, fin = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], inp.wl.chunk,
                              init_state=g["init"], cu_seqlens=g.get("cu"))
    torch.cuda.synchronize()
    return g, y, fin


def test_mamba2_130m_prefill_full():
    wl = W.CONFIGS[1]
    say("case:", wl.name)
    inp = W.generate(wl, W.SEED_BASE + 1)
    _, y, fin = gpu_scan(inp)
    yr, fr = oracle_scan(inp)
    say("  y err %.3e" % assert_close(host(y), yr, "bf16", "y"))
    say("  final err %.3e" % assert_close(host(fin), fr, "bf16", "final"))


def test_mamba2_2p7b_prefill_sampled():
    wl = W.CONFIGS[3]
    say("case:", wl.name)
    inp = W.generate(wl, W.SEED_BASE + 3)
    _, y, fin = gpu_scan(inp)
    heads = [0, 41, 79]
    seqs = [0, 5]
    yr, fr = oracle_scan(inp, heads=heads, seqs=seqs)
    yg = y[seqs][:, :, heads]
    fg = fin[seqs][:, heads]
    say("  y err %.3e" % assert_close(host(yg), yr, "bf16", "y"))
    say("  final err %.3e" % assert_close(host(fg), fr, "bf16", "final"))


def test_varlen_grouped_prefill_and_decode_sampled():
    wl = W.CONFIGS[4]
    say("case:", wl.name)
    inp = W.generate(wl, W.SEED_BASE + 4)
    g, y, fin = gpu_scan(inp)
    heads = np.array([0, 17, 64, 127])  # groups 0, 1, 4, 7
    yr, fr = oracle_scan(inp, heads=heads)
    say("  y err %.3e" % assert_close(host(y[:, heads]), yr, "bf16", "y"))
    say("  final err %.3e" % assert_close(host(fin[:, heads]), fr, "bf16", "final"))
    # 32 decode steps per sequence, continuing from the prefill's final states
    state = fin
    ref = fr
    groups = heads // (wl.H // wl.G)
    for k, d in enumerate(inp.decode):
        yd = ssd.decode_step(state, tdev(d["x"], "bf16"), tdev(d["dt"]), g["A"], tdev(d["B"], "bf16"),
                             tdev(d["C"], "bf16"), g["D"])
        yref, ref = oracle.decode(ref, d["x"][:, heads], d["dt"][:, heads], inp.A[heads],
                                  d["B"][:, groups], d["C"][:, groups], inp.D[heads])
        assert_close(host(yd[:, heads]), yref, "bf16", "decode y %d" % k)
    torch.cuda.synchronize()
    say("  decode state err %.3e" % assert_close(host(state[:, heads]), ref, "bf16", "decode state"))


def test_mamba2_2p7b_decode_100_steps_sampled():
    wl = W.CONFIGS[2]
    say("case:", wl.name)
    inp = W.generate(wl, W.SEED_BASE + 2)
    state = tdev(inp.init)
    A, D = tdev(inp.A), tdev(inp.D)
    seqs = np.array([0, 77, 255])
    ref = inp.init[seqs].astype(np.float64)
    worst = 0.0
    for k, d in enumerate(inp.decode):
        y = ssd.decode_step(state, tdev(d["x"], "bf16"), tdev(d["dt"]), A, tdev(d["B"], "bf16"),
                            tdev(d["C"], "bf16"), D)
        yr, ref = oracle.decode(ref, d["x"][seqs], d["dt"][seqs], inp.A, d["B"][seqs], d["C"][seqs],
                                inp.D)
        worst = max(worst, assert_close(host(y[seqs]), yr, "bf16", "decode y %d" % k))
    torch.cuda.synchronize()
    say("  worst y err %.3e" % worst)
    say("  state err %.3e" % assert_close(host(state[seqs]), ref, "bf16", "state after 100 steps"))
