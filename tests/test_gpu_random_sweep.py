"""GPU parity over a seeded random sweep of shapes: every output element of a
prefill, then one decode step continuing from its final state, against the
fp64 oracle at the tolerance of the input dtype.

Each case draws the dtype, chunk length, heads and groups, head dim and
dstate (multiples of 8 across the supported ranges), a dense or packed batch
(empty and one-token sequences included), the initial state, the decay
regime, and the prefill path: the library's choice, or one of the three
paths forced where it applies.  The hand-picked shapes elsewhere cover the
named configurations and the limits; this sweep covers the combinations
between them.  A draw whose dstate and chunk need more LDS than the kernels
have is rejected by the library with SSD_ERR_SHAPE, and the sweep checks
that rejection instead.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import mamba_ssd_chunked_02_amd as ssd
from mamba_ssd_chunked_02_amd import workloads as W
from parity import assert_close, host, oracle_scan, tdev, to_gpu

pytestmark = pytest.mark.gpu

SSD_ERR_SHAPE = -2
NCASES = 48


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draw(k):
    """Case k of the sweep (numpy PCG64, seed 9100 + k)."""
    rng = np.random.Generator(np.random.PCG64(9100 + k))
    path = str(rng.choice(["auto", "auto", "chunk_parallel", "state_walk", "scan_walk"]))
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    chunk = int(rng.choice([32, 64, 128, 256]))
    G = int(rng.choice([1, 2, 4]))
    H = G * int(rng.choice([1, 2, 3, 4, 8]))
    P = int(rng.choice([8, 16, 24, 32, 40, 64, 72, 96, 128]))
    N = int(rng.choice([8, 16, 32, 48, 64, 72, 96, 128, 136, 256]))
    if path == "scan_walk":
        # the shapes that path covers: bf16, 256-token chunks, dstate in (64, 128]
        dtype, chunk, N = "bf16", 256, int(rng.choice([72, 96, 128]))
    if rng.random() < 0.3:
        lens = [int(v) for v in rng.integers(0, 700, size=int(rng.integers(1, 6)))]
        lens[int(rng.integers(0, len(lens)))] = int(rng.choice([0, 1, chunk, chunk + 1]))
        batch, L = 0, 0
    else:
        lens = None
        batch = int(rng.integers(1, 5))
        L = int(rng.choice([1, chunk - 1, chunk + 1, int(rng.integers(2, 900)), int(rng.integers(2, 900))]))
    init_var = 0.1 if rng.random() < 0.6 else 0.0
    regime = str(rng.choice(["default", "default", "slow", "strong", "zero"]))
    wl = W.small_workload(batch=batch, seqlen=L, seqlens=lens, H=H, P=P, N=N, G=G, chunk=chunk, dtype=dtype,
                          init_var=init_var, decode_steps=1)
    kw = dict(slow=dict(A_range=(-0.05, -0.001)), strong=dict(A_range=(-200.0, -20.0)),
              zero=dict(A_zero=True)).get(regime, {})
    return wl, W.generate(wl, 9200 + k, **kw), regime, path


@pytest.mark.parametrize("k", range(NCASES))
def test_random_shape(k):
    wl, inp, regime, path = draw(k)
    dt = wl.dtype
    say("case %d:" % k, wl.name, regime, path)
    g = to_gpu(inp)
    try:
        y, fin = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], wl.chunk,
                                  init_state=g["init"], cu_seqlens=g.get("cu"), path=path)
    except ssd.SsdError as e:
        # the only rejection a draw can meet: dstate and chunk beyond the LDS
        assert e.status == SSD_ERR_SHAPE and "LDS" in str(e), str(e)
        say("  rejected as expected:", e)
        return
    torch.cuda.synchronize()
    yr, fr = oracle_scan(inp)
    ey = assert_close(host(y), yr, dt, "y")
    ef = assert_close(host(fin), fr, dt, "final")
    # one decode step per sequence from the final state
    d = inp.decode[0]
    state = fin.clone()
    yd = ssd.decode_step(state, tdev(d["x"], dt), tdev(d["dt"]), g["A"], tdev(d["B"], dt), tdev(d["C"], dt),
                         g["D"])
    torch.cuda.synchronize()
    ydr, sr = oracle.decode(fr, d["x"], d["dt"], inp.A, d["B"], d["C"], inp.D)
    ed = assert_close(host(yd), ydr, dt, "decode y")
    es = assert_close(host(state), sr, dt, "decode state")
    say("  y %.2e  final %.2e  decode y %.2e  state %.2e" % (ey, ef, ed, es))
