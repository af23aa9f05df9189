"""GPU parity at the full sizes of the five named workloads, in the launch
configuration the benchmark uses (the library's own choice of kernels), every
output element against the fp64 oracle:

  tiny fp32 b1 L512 H4 P16 N16 (+16 decode steps)      tests/test_gpu_parity.py
  130M-shaped layer b1 L4096 H24                        y and final state
  2.7B-shaped decode b256 H80, 100 steps                every step's y, state after steps 1, 50, 100
  2.7B-shaped layer b8 L8192 H80                        y and final states (all 640 sequence-head pairs)
  packed {1024,4096,12288,32768} H128 G8 (+32 steps)    y, final states, every decode step
"""
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
    st = []
    y, fin = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], inp.wl.chunk,
                              init_state=g["init"], cu_seqlens=g.get("cu"), stage_ms=st)
    torch.cuda.synchronize()
    say("  stages (ms)", dict(zip(ssd.STAGES, ["%.3f" % v for v in st])))
    return g, y, fin


def test_mamba2_130m_prefill_full():
    wl = W.CONFIGS[1]
    say("case:", wl.name)
    inp = W.generate(wl, W.SEED_BASE + 1)
    _, y, fin = gpu_scan(inp)
    yr, fr = oracle_scan(inp)
    say("  y err %.3e" % assert_close(host(y), yr, "bf16", "y"))
    say("  final err %.3e" % assert_close(host(fin), fr, "bf16", "final"))


def test_mamba2_2p7b_prefill_full():
    wl = W.CONFIGS[3]
    say("case:", wl.name)
    inp = W.generate(wl, W.SEED_BASE + 3)
    _, y, fin = gpu_scan(inp)
    yg, fg = host(y), host(fin)
    del y, fin
    yr, fr = oracle_scan(inp)
    say("  y err %.3e" % assert_close(yg, yr, "bf16", "y"))
    say("  final err %.3e" % assert_close(fg, fr, "bf16", "final"))
    # per sequence too: a fault confined to one sequence's walk cannot hide
    # behind the whole tensor's RMS
    worst = max(assert_close(yg[s], yr[s], "bf16", "y seq %d" % s) for s in range(wl.batch))
    say("  worst per-sequence y err %.3e" % worst)


def test_varlen_grouped_prefill_and_decode_full():
    wl = W.CONFIGS[4]
    say("case:", wl.name)
    inp = W.generate(wl, W.SEED_BASE + 4)
    g, y, fin = gpu_scan(inp)
    yr, fr = oracle_scan(inp)
    yg = host(y)
    say("  y err %.3e" % assert_close(yg, yr, "bf16", "y"))
    say("  final err %.3e" % assert_close(host(fin), fr, "bf16", "final"))
    cu = inp.cu_seqlens
    for s in range(len(wl.seqlens)):
        assert_close(yg[cu[s]:cu[s + 1]], yr[cu[s]:cu[s + 1]], "bf16", "y seq %d" % s)
    # 32 decode steps per sequence on every head, continuing from the prefill's final states
    state = fin
    ref = np.ascontiguousarray(fr, dtype=np.float64)
    worst = 0.0
    for k, d in enumerate(inp.decode):
        yd = ssd.decode_step(state, tdev(d["x"], "bf16"), tdev(d["dt"]), g["A"], tdev(d["B"], "bf16"),
                             tdev(d["C"], "bf16"), g["D"])
        yref, ref = oracle.decode(ref, d["x"], d["dt"], inp.A, d["B"], d["C"], inp.D, inplace=True)
        worst = max(worst, assert_close(host(yd), yref, "bf16", "decode y %d" % k))
    torch.cuda.synchronize()
    say("  worst decode y err %.3e" % worst)
    say("  decode state err %.3e" % assert_close(host(state), ref, "bf16", "decode state"))


def test_mamba2_2p7b_decode_100_steps_full():
    wl = W.CONFIGS[2]
    say("case:", wl.name)
    inp = W.generate(wl, W.SEED_BASE + 2)
    state = tdev(inp.init)
    A, D = tdev(inp.A), tdev(inp.D)
    ref = np.ascontiguousarray(inp.init, dtype=np.float64)
    worst = 0.0
    for k, d in enumerate(inp.decode):
        y = ssd.decode_step(state, tdev(d["x"], "bf16"), tdev(d["dt"]), A, tdev(d["B"], "bf16"),
                            tdev(d["C"], "bf16"), D)
        yr, ref = oracle.decode(ref, d["x"], d["dt"], inp.A, d["B"], d["C"], inp.D, inplace=True)
        worst = max(worst, assert_close(host(y), yr, "bf16", "decode y %d" % k))
        if k in (0, 49, len(inp.decode) - 1):
            torch.cuda.synchronize()
            say("  step %d: state err %.3e" % (k + 1, assert_close(host(state), ref, "bf16",
                                                                    "state after step %d" % (k + 1))))
    say("  worst y err over %d steps %.3e" % (len(inp.decode), worst))
