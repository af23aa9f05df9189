"""GPU parity of the scan walk: the prefill path in which one kernel walks a
sequence's chunks for a slice of (head, 32-column tile) units, keeping each
unit's state in MFMA accumulators and writing y chunk by chunk, so the state
entering a chunk never reaches memory.  Every case forces the path and
compares each output element with the fp64 oracle at the bf16 tolerance
(max |err| / RMS <= 2e-2), and some also with the other two paths.

The path covers bf16 inputs, 256-token chunks and dstate in (64, 128].  The
cases span:
  * 1 to 6 units per workgroup (the unit count follows the batch size);
  * ragged sequence lengths (partial chunks and partial 32-token blocks),
    single-token and empty sequences, packed batches;
  * head dims that are not a multiple of 32 (a partial column tile);
  * dstate 72, 96 and 128; one group or several;
  * zero and nonzero initial states, a final state aliasing the initial one;
  * fp32 and bf16 y;
  * slow decay, strong decay past the fast-path bound, and the flush limit;
  * chunks on both sides of the whole-chunk decay bound of the single
    reference form.
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(inp, path="scan_walk", y_dtype=None, want_stages=True):
    g = to_gpu(inp)
    st = [] if want_stages else None
    y, fin = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], inp.wl.chunk,
                              init_state=g["init"], cu_seqlens=g.get("cu"), path=path, y_dtype=y_dtype,
                              stage_ms=st)
    torch.cuda.synchronize()
    if want_stages and path == "scan_walk":
        # the walk replaces the three separate stages
        names = ssd.STAGES
        assert st[names.index("chunk_state")] == 0.0 and st[names.index("chunk_scan")] == 0.0, st
        assert st[names.index("scan_walk")] > 0.0, st
    return y, fin


def check(inp, what="", **kw):
    say("case:", inp.wl.name, what)
    y, fin = run(inp, **kw)
    yr, fr = oracle_scan(inp)
    ey = assert_close(host(y), yr, "bf16", "y " + what)
    ef = assert_close(host(fin), fr, "bf16", "final " + what)
    say("  y err %.3e  final err %.3e" % (ey, ef))
    return y, fin


SHAPES = [
    # (batch, L, H, P, N, G, init): units = batch * H * ceil(P/32) set the units per workgroup
    (1, 700, 4, 64, 128, 1, 0.1),       # 8 units: one per workgroup
    (2, 300, 4, 64, 128, 2, 0.0),       # zero initial state, two groups
    (8, 300, 32, 64, 128, 1, 0.1),      # 512 units: 2 per workgroup
    (8, 257, 48, 64, 128, 1, 0.1),      # 768 units: 3
    (8, 260, 64, 64, 128, 4, 0.1),      # 1024 units: 4, four groups
    (8, 300, 80, 64, 128, 1, 0.1),      # 1280 units: 5 (the 2.7B-shaped layer's split)
    (8, 200, 96, 64, 128, 2, 0.1),      # 1536 units: 6
    (2, 300, 80, 64, 128, 1, 0.1),      # 320 units: 2 (160 workgroups in one round, not 320 in two)
    (4, 300, 80, 64, 128, 1, 0.1),      # 640 units: 3 (216 workgroups, the last slice of each group short)
    (2, 513, 8, 40, 96, 2, 0.1),        # partial column tile, dstate 96
    (2, 300, 6, 128, 72, 3, 0.1),       # four column tiles, dstate 72, three groups
    (3, 33, 8, 64, 128, 1, 0.1),        # one partial chunk of one full and one partial block
    (4, 1, 8, 64, 128, 1, 0.1),         # single-token sequences
    (1, 2048, 8, 64, 128, 1, 0.1),      # eight chunks
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "b%d-L%d-H%d-P%d-N%d-G%d-init%g" % c)
def test_scan_walk_shapes(case):
    b, L, H, P, N, G, iv = case
    wl = W.small_workload(batch=b, seqlen=L, H=H, P=P, N=N, G=G, chunk=256, dtype="bf16", init_var=iv)
    check(W.generate(wl, 500 + L + H + P + N), what=str(case))


@pytest.mark.parametrize("variant", ["slow", "A0", "x0", "strong", "mixed", "flush"])
def test_scan_walk_decay_regimes(variant):
    """Slow decay and A = 0 make the passed state matter in every chunk; x = 0
    leaves only the initial state's path; strong decay and the flush limit
    take the exact per-element path of blocks decaying past the fast bound."""
    wl = W.small_workload(batch=4, seqlen=900, H=16, P=64, N=128, G=2, chunk=256, dtype="bf16",
                          init_var=0.1)
    kw = dict(slow=dict(A_range=(-0.05, -0.001)), A0=dict(A_zero=True), x0=dict(x_zero=True),
              strong=dict(A_range=(-1e3, -60.0)), mixed=dict(A_values=(-10.0, -300.0)),
              flush=dict(A_range=(-1e6, -1e6)))[variant]
    check(W.generate(wl, 21, **kw), what=variant)


def test_scan_walk_chunks_on_both_sides_of_the_single_reference_bound():
    """A chunk whose whole decay stays below 60 takes its weights to the
    chunk's end (one scaling of the state, unscaled sums); others take the
    per-block Horner scheme.  Here each (sequence, chunk, head) gets its own
    total decay, drawn from U(35, 85), so the two forms alternate along one
    head's walk and between the heads of one step, over full and ragged
    chunks (1000 tokens: three full chunks and one of 232)."""
    wl = W.small_workload(batch=4, seqlen=1000, H=16, P=64, N=128, G=2, chunk=256, dtype="bf16",
                          init_var=0.1)
    inp = W.generate(wl, 91)
    rng = np.random.default_rng(92)
    b, L, H = inp.dt.shape
    dt = np.empty_like(inp.dt)
    decay = []
    for c0 in range(0, L, 256):
        c1 = min(c0 + 256, L)
        r = rng.uniform(0.5, 1.5, size=(b, c1 - c0, H))
        total = rng.uniform(35.0, 85.0, size=(b, 1, H))
        dt[:, c0:c1] = (r / r.sum(axis=1, keepdims=True) * total / -inp.A[None, None, :]).astype(np.float32)
        decay.append(-(dt[:, c0:c1].astype(np.float64) * inp.A).sum(axis=1))
    decay = np.concatenate(decay)
    assert (decay < 58).sum() > 50 and (decay > 62).sum() > 50, "both forms must occur"
    inp.dt = dt
    check(inp, what="decay U(35, 85) per chunk")


def test_scan_walk_bf16_y_is_rounded_fp32_y():
    wl = W.small_workload(batch=2, seqlen=500, H=8, P=64, N=128, G=2, chunk=256, dtype="bf16", init_var=0.1)
    inp = W.generate(wl, 77)
    y32, f32 = run(inp)
    y16, f16 = run(inp, y_dtype=torch.bfloat16)
    assert y16.dtype == torch.bfloat16
    assert torch.equal(y16, y32.to(torch.bfloat16)) and torch.equal(f16, f32)


@pytest.mark.parametrize("lens", [(100, 0, 513, 1, 256, 700), (0, 0), (300, 280, 310, 290, 2000)])
def test_scan_walk_packed(lens):
    wl = W.small_workload(seqlens=lens, H=16, P=64, N=128, G=4, chunk=256, dtype="bf16", init_var=0.1)
    check(W.generate(wl, 79 + sum(lens)), what="lens=%s" % (lens,))


def test_scan_walk_agrees_with_the_other_paths():
    """The three paths on one input: each within tolerance of the oracle and
    of each other."""
    wl = W.small_workload(batch=8, seqlen=600, H=32, P=64, N=128, G=2, chunk=256, dtype="bf16", init_var=0.1)
    inp = W.generate(wl, 83, A_range=(-0.5, -0.01))
    yr, fr = oracle_scan(inp)
    outs = {}
    for path in ("chunk_parallel", "state_walk", "scan_walk"):
        y, fin = run(inp, path=path)
        outs[path] = (host(y), host(fin))
        assert_close(outs[path][0], yr, "bf16", "y " + path)
        assert_close(outs[path][1], fr, "bf16", "final " + path)
    for path in ("chunk_parallel", "state_walk"):
        assert_close(outs["scan_walk"][0], outs[path][0].astype(np.float64), "bf16", "y vs " + path)
        assert_close(outs["scan_walk"][1], outs[path][1].astype(np.float64), "bf16", "final vs " + path)


def test_scan_walk_final_may_alias_initial_and_continues_with_decode():
    wl = W.small_workload(batch=4, seqlen=400, H=16, P=64, N=128, G=1, chunk=256, dtype="bf16", init_var=0.1,
                          decode_steps=3, decode_batch=4)
    inp = W.generate(wl, 87)
    g = to_gpu(inp)
    st = g["init"].clone()
    y, _ = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 256, init_state=st, final_state=st,
                            path="scan_walk")
    torch.cuda.synchronize()
    yr, fr = oracle_scan(inp)
    assert_close(host(y), yr, "bf16", "y")
    assert_close(host(st), fr, "bf16", "aliased final")
    ref = fr
    for k, d in enumerate(inp.decode):
        yd = ssd.decode_step(st, tdev(d["x"], "bf16"), tdev(d["dt"]), g["A"], tdev(d["B"], "bf16"),
                             tdev(d["C"], "bf16"), g["D"])
        yref, ref = oracle.decode(ref, d["x"], d["dt"], inp.A, d["B"], d["C"], inp.D)
        assert_close(host(yd), yref, "bf16", "decode y %d" % k)
    torch.cuda.synchronize()
    assert_close(host(st), ref, "bf16", "decode state")


def test_scan_walk_deterministic_with_poisoned_buffers_and_graph_replay():
    """NaN-filled workspace and outputs give the same bits as a clean call,
    and a captured call replays bitwise equal (the walk clears nothing and
    allocates nothing)."""
    wl = W.small_workload(batch=8, seqlen=300, H=32, P=64, N=128, G=2, chunk=256, dtype="bf16", init_var=0.1)
    inp = W.generate(wl, 89)
    g = to_gpu(inp)
    nbytes = ssd.workspace_size(g["x"], g["B"], 256, path="scan_walk")
    ws = torch.full((nbytes // 4 + 1,), float("nan"), device="cuda").view(torch.uint8)[:nbytes]
    y = torch.full(tuple(g["x"].shape), float("nan"), device="cuda")
    fin = torch.full_like(g["init"], float("nan"))

    def call():
        ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 256, init_state=g["init"], y=y,
                         final_state=fin, workspace=ws, path="scan_walk")
    call()
    torch.cuda.synchronize()
    y_ref, f_ref = y.clone(), fin.clone()
    y2, f2 = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 256, init_state=g["init"],
                              path="scan_walk")
    torch.cuda.synchronize()
    assert torch.equal(y_ref, y2) and torch.equal(f_ref, f2)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in range(3):
        y.fill_(float("nan"))
        fin.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(fin, f_ref), "replay %d" % k
        _ = (g["x"].float() * 2).sum().item()
