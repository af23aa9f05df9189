"""GPU parity of the scan walk's longest-first schedule on packed batches.

The plan kernel orders the sequences by chunk count, longest first (ties in
index order), and the walk's workgroups start in that order, in runs of
consecutive (pair, slice) items dealt to the XCDs in turn.  With the host
copy of the offsets, the host picks the units per workgroup from a
longest-first time estimate and, for the library's choice, whether to walk at
all.  The order only schedules: every case compares each output element with
the fp64 oracle at the bf16 tolerance, with the order built from the device
offsets even where the host copy disagrees with them.
"""
import sys

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_02_amd as ssd
from mamba_ssd_chunked_02_amd import workloads as W
from parity import assert_close, host, oracle_scan, to_gpu

pytestmark = pytest.mark.gpu

S = ssd.STAGES


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(inp, path, cu_host):
    g = to_gpu(inp)
    st = []
    y, fin = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], inp.wl.chunk,
                              init_state=g["init"], cu_seqlens=g["cu"], cu_seqlens_host=cu_host, path=path,
                              stage_ms=st)
    torch.cuda.synchronize()
    return y, fin, st


def walked(st):
    return st[S.index("scan_walk")] > 0 and st[S.index("chunk_scan")] == 0


def check(inp, what, path="scan_walk", cu_host=None, expect_walk=None):
    say("case:", inp.wl.name, what, path)
    cu_host = [int(v) for v in inp.cu_seqlens] if cu_host is None else cu_host
    y, fin, st = run(inp, path, cu_host)
    say("  stages", ["%.3f" % v for v in st])
    if expect_walk is not None:
        assert walked(st) == expect_walk, st
    yr, fr = oracle_scan(inp)
    ey = assert_close(host(y), yr, "bf16", "y " + what)
    ef = assert_close(host(fin), fr, "bf16", "final " + what)
    say("  y err %.3e  final err %.3e" % (ey, ef))


@pytest.mark.parametrize("lens", [
    (0, 9000, 300, 9000, 0, 4000, 256, 1),   # ties, empty and one-token sequences
    (5000, 37, 5000, 12000, 700),
    (256, 512, 768, 1024, 1280, 1536, 1792, 2048, 2304, 7000),
])
def test_longest_first_walk_forced(lens):
    wl = W.small_workload(seqlens=lens, H=16, P=64, N=128, G=2, chunk=256, dtype="bf16", init_var=0.1)
    check(W.generate(wl, 211 + sum(lens)), "lens=%s" % (lens,), expect_walk=True)


@pytest.mark.parametrize("lens,H,G", [((1024, 4096, 12288, 16384), 32, 4), ((2048, 8192, 8192, 6000), 16, 1)])
def test_library_choice_with_the_host_copy(lens, H, G):
    """Uneven packed batches through the library's choice (the longest-first
    estimate decides between the walk and the chunk-parallel kernels)."""
    wl = W.small_workload(seqlens=lens, H=H, P=64, N=128, G=G, chunk=256, dtype="bf16", init_var=0.1)
    check(W.generate(wl, 223 + sum(lens)), "lens=%s H%d G%d" % (lens, H, G), path="auto")


def test_more_sequences_than_are_ordered():
    """Past kOrderMaxSeq sequences the plan kernel keeps their index order."""
    rng = np.random.default_rng(227)
    lens = tuple(int(v) for v in rng.integers(0, 700, size=300))
    wl = W.small_workload(seqlens=lens, H=8, P=64, N=128, G=1, chunk=256, dtype="bf16", init_var=0.1)
    check(W.generate(wl, 229), "300 sequences", expect_walk=True)


@pytest.mark.parametrize("dev_lens,host_lens", [((9000, 300, 4000), (300, 4000, 9000)),
                                                ((4646, 4654, 4000), (9000, 300, 4000))])
def test_host_copy_that_disagrees_with_the_device_offsets(dev_lens, host_lens):
    """The host copy only sizes and schedules; the order and every output
    follow the device offsets."""
    wl = W.small_workload(seqlens=dev_lens, H=16, P=64, N=128, G=1, chunk=256, dtype="bf16", init_var=0.1)
    inp = W.generate(wl, 233)
    cu_host = [0] + [int(v) for v in np.cumsum(host_lens)]
    assert cu_host[-1] == int(inp.cu_seqlens[-1])
    check(inp, "host copy %s" % (host_lens,), cu_host=cu_host, expect_walk=True)
