"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Small cases compare every element; full-size workloads
compare sampled (sequence, head) pairs that the oracle recomputes."""
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


def run_gpu(inp, chunk=None, want_final=True, path="auto"):
    g = to_gpu(inp)
    chunk = chunk or inp.wl.chunk
    y, fin = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk,
                              init_state=g["init"], cu_seqlens=g.get("cu"), want_final=want_final, path=path)
    torch.cuda.synchronize()
    return host(y), None if fin is None else host(fin)


def check_scan(inp, chunk=None, what="", path="auto"):
    dt = inp.wl.dtype
    say("case:", inp.wl.name, "chunk", chunk, what, path)
    y, fin = run_gpu(inp, chunk, path=path)
    yr, fr = oracle_scan(inp)
    ey = assert_close(y, yr, dt, "y " + what)
    ef = assert_close(fin, fr, dt, "final " + what)
    return ey, ef


# ------------------------------------------------------------------ tiny fp32 workload
def test_tiny_fp32_prefill_and_decode():
    wl = W.CONFIGS[0]
    inp = W.generate(wl, W.SEED_BASE + 0)
    say("case: tiny fp32 config with 16 decode steps")
    g = to_gpu(inp)
    y, fin = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], wl.chunk,
                              init_state=g["init"])
    yr, fr = oracle.scan(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, init=inp.init)
    assert_close(host(y), yr, "f32", "y")
    assert_close(host(fin), fr, "f32", "final")
    state = fin.clone()
    ref_state = fr
    for k, d in enumerate(inp.decode):
        yd = ssd.decode_step(state, tdev(d["x"]), tdev(d["dt"]), g["A"], tdev(d["B"]), tdev(d["C"]),
                             g["D"])
        yref, ref_state = oracle.decode(ref_state, d["x"], d["dt"], inp.A, d["B"], d["C"], inp.D)
        assert_close(host(yd), yref, "f32", "decode y step %d" % k)
        assert_close(host(state), ref_state, "f32", "decode state step %d" % k)


# ------------------------------------------------------------------ shapes, tiles, ragged tails
SMALL = [
    # (batch, L, H, P, N, G, chunk, dtype, init)
    (1, 64, 4, 16, 16, 1, 64, "f32", 0.0),
    (2, 700, 6, 64, 128, 2, 256, "bf16", 0.1),
    (1, 1000, 4, 64, 128, 1, 128, "bf16", 0.1),
    (3, 333, 4, 32, 64, 4, 64, "bf16", 0.1),
    (2, 257, 4, 64, 64, 2, 32, "f32", 0.1),
    (1, 300, 2, 128, 128, 1, 64, "bf16", 0.1),
    (1, 130, 2, 8, 8, 2, 64, "f32", 0.1),
    (2, 200, 3, 24, 40, 3, 32, "bf16", 0.1),
    (1, 513, 2, 64, 256, 1, 128, "bf16", 0.1),
    (1, 96, 2, 64, 256, 1, 32, "bf16", 0.1),
    (1, 160, 2, 128, 128, 2, 32, "bf16", 0.1),
    (1, 300, 2, 32, 256, 1, 256, "f32", 0.1),
    (2, 290, 2, 64, 256, 1, 256, "bf16", 0.1),
    # 256 or more (chunk, group) pairs: the whole-chunk C.B^T kernel
    (8, 1000, 4, 32, 64, 2, 64, "bf16", 0.1),
    (4, 2000, 8, 16, 32, 4, 128, "f32", 0.1),
    # the largest head (P 128, N 256) at the largest chunk
    (1, 300, 2, 128, 256, 1, 256, "bf16", 0.1),
    (1, 300, 2, 128, 256, 2, 256, "f32", 0.1),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b%d-L%d-H%d-P%d-N%d-G%d-Q%d-%s" % c[:8])
def test_small_shapes(case):
    b, L, H, P, N, G, Q, dt, iv = case
    wl = W.small_workload(batch=b, seqlen=L, H=H, P=P, N=N, G=G, chunk=Q, dtype=dt, init_var=iv)
    check_scan(W.generate(wl, 11 + L), what=str(case))


@pytest.mark.parametrize("variant", ["slow", "A0", "x0"])
def test_decay_variants(variant):
    """Slow decay, A = 0 and x = 0 (initial-state path only) stress the state
    passed between chunks, which strong decay would hide."""
    wl = W.small_workload(batch=2, seqlen=900, H=4, P=64, N=128, G=2, chunk=128, dtype="bf16",
                          init_var=0.1)
    kw = dict(slow=dict(A_range=(-0.05, -0.001)), A0=dict(A_zero=True), x0=dict(x_zero=True))[variant]
    inp = W.generate(wl, 21, **kw)
    check_scan(inp, what=variant)


@pytest.mark.parametrize("chunk", [32, 64, 128, 256])
def test_chunk_sizes_agree(chunk):
    wl = W.small_workload(batch=1, seqlen=777, H=4, P=64, N=64, G=1, chunk=chunk, dtype="f32",
                          init_var=0.1)
    inp = W.generate(wl, 31, A_range=(-0.2, -0.01))
    check_scan(inp, chunk=chunk)


@pytest.mark.parametrize("L", [64 * 7, 64 * 8, 64 * 9 + 5, 4100])
def test_many_chunks_per_sequence(L):
    """State passing walks the chunks in batches of eight: chunk counts below,
    at and past a batch boundary, and a long sequence with slow decay so that
    the passed state matters to the last chunk."""
    wl = W.small_workload(batch=2, seqlen=L, H=3, P=64, N=128, G=1, chunk=64, dtype="bf16",
                          init_var=0.1)
    inp = W.generate(wl, 41 + L, A_range=(-0.02, -0.001))
    check_scan(inp, what="L=%d" % L)


def test_edge_lengths():
    for L in (1, 31, 32, 33, 64, 65):
        wl = W.small_workload(batch=2, seqlen=L, H=2, P=16, N=16, G=1, chunk=32, dtype="f32",
                              init_var=0.1)
        check_scan(W.generate(wl, 50 + L), what="L=%d" % L)


def test_no_initial_state_equals_zero_initial_state():
    wl = W.small_workload(batch=1, seqlen=300, H=2, P=64, N=64, G=1, chunk=64, dtype="bf16")
    inp = W.generate(wl, 60)
    g = to_gpu(inp)
    y0, f0 = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 64)
    z = torch.zeros_like(f0)
    y1, f1 = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 64, init_state=z)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)


@pytest.mark.parametrize("H,walk", [(2, False), (64, True)])
def test_final_state_may_alias_initial_state(H, walk):
    """final_state == init_state on both state paths: 4 and 256 (sequence,
    head, column tile) walks."""
    wl = W.small_workload(batch=2, seqlen=400, H=H, P=64 if walk else 32, N=32, G=1, chunk=64,
                          dtype="f32", init_var=0.1)
    inp = W.generate(wl, 61)
    g = to_gpu(inp)
    st = g["init"].clone()
    stages = []
    y, fin = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 64, init_state=st,
                              final_state=st, stage_ms=stages)
    torch.cuda.synchronize()
    assert (stages[ssd.STAGES.index("state_passing")] == 0.0) == walk, stages
    yr, fr = oracle.scan(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, init=inp.init)
    assert_close(host(st), fr, "f32", "aliased final")
    assert_close(host(y), yr, "f32", "y")


# ------------------------------------------------------------------ packed variable-length batches
@pytest.mark.parametrize("lens,G", [
    ((100, 0, 513, 1, 256), 2),
    ((300, 700, 64, 65), 4),
    ((1024, 3000, 7), 8),
    ((0, 0), 1),
])
def test_packed_batches(lens, G):
    H = 8 if G in (1, 2, 4, 8) else G
    wl = W.small_workload(seqlens=lens, H=H, P=64, N=128, G=G, chunk=256, dtype="bf16", init_var=0.1)
    check_scan(W.generate(wl, 70 + sum(lens)), what="lens=%s" % (lens,))


def test_packed_equals_separate_dense_runs():
    lens = (200, 450, 31)
    wl = W.small_workload(seqlens=lens, H=4, P=64, N=64, G=2, chunk=64, dtype="f32", init_var=0.1)
    inp = W.generate(wl, 80)
    y, fin = run_gpu(inp)
    cu = inp.cu_seqlens
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        g = dict(x=tdev(inp.x[None, a:b]), dt=tdev(inp.dt[None, a:b]), B=tdev(inp.B[None, a:b]),
                 C=tdev(inp.C[None, a:b]))
        ys, fs = ssd.chunked_scan(g["x"], g["dt"], tdev(inp.A), g["B"], g["C"], tdev(inp.D), 64,
                                  init_state=tdev(inp.init[s:s + 1]))
        torch.cuda.synchronize()
        assert_close(y[a:b], host(ys)[0], "f32", "seq %d y" % s)
        assert_close(fin[s], host(fs)[0], "f32", "seq %d final" % s)


# ------------------------------------------------------------------ one walk per (sequence, head, tile)
# With at least 256 (sequence, head, 32-column tile) walks the chunk states
# and the passing between chunks run as one kernel that walks each
# sequence's chunks in order.  Where the scan walk applies (bf16, chunk 256,
# dstate in (64, 128]) the library takes that instead; these tests force the
# state walk so that it keeps its coverage at those shapes too.
FUSED = [
    # (batch, L, H, P, N, G, chunk, dtype, init)
    (4, 300, 32, 64, 128, 2, 64, "bf16", 0.1),
    (8, 130, 32, 32, 64, 4, 32, "f32", 0.1),
    (2, 513, 128, 40, 40, 8, 128, "bf16", 0.1),
    (16, 100, 16, 64, 256, 1, 64, "bf16", 0.0),
    (64, 70, 4, 8, 8, 2, 32, "f32", 0.1),
    (2, 1000, 64, 64, 128, 1, 256, "bf16", 0.1),
    (4, 257, 32, 128, 32, 4, 128, "f32", 0.1),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "b%d-L%d-H%d-P%d-N%d-G%d-Q%d-%s" % c[:8])
def test_fused_state_walk_shapes(case):
    b, L, H, P, N, G, Q, dt, iv = case
    wl = W.small_workload(batch=b, seqlen=L, H=H, P=P, N=N, G=G, chunk=Q, dtype=dt, init_var=iv)
    check_scan(W.generate(wl, 13 + L), what=str(case), path="state_walk")


def test_fused_state_walk_slow_decay_long_sequences():
    wl = W.small_workload(batch=4, seqlen=2300, H=32, P=64, N=128, G=1, chunk=128, dtype="bf16",
                          init_var=0.1)
    check_scan(W.generate(wl, 23, A_range=(-0.02, -0.001)), what="slow decay", path="state_walk")


@pytest.mark.parametrize("path", ["state_walk", "auto"])
def test_fused_state_walk_packed_with_empty_sequences(path):
    lens = (100, 0, 513, 1, 256, 0, 700, 64, 65, 300, 0, 7, 1024, 33, 0, 250)
    wl = W.small_workload(seqlens=lens, H=8, P=64, N=128, G=2, chunk=256, dtype="bf16", init_var=0.1)
    check_scan(W.generate(wl, 71), what="packed, %d sequences" % len(lens), path=path)


def test_fused_walk_equals_separate_runs():
    """A packed batch of 40 sequences takes the one-kernel walk; each sequence
    alone (16 walks) takes the chunk-parallel kernels.  Both must agree."""
    rng = np.random.default_rng(5)
    lens = tuple(int(v) for v in rng.integers(0, 600, size=40))
    wl = W.small_workload(seqlens=lens, H=8, P=64, N=64, G=2, chunk=64, dtype="f32", init_var=0.1)
    inp = W.generate(wl, 81)
    y, fin = run_gpu(inp)
    cu = inp.cu_seqlens
    for s in range(0, len(lens), 7):
        a, b = cu[s], cu[s + 1]
        if b == a:
            assert_close(fin[s], inp.init[s], "f32", "empty seq %d final" % s)
            continue
        g = dict(x=tdev(inp.x[None, a:b]), dt=tdev(inp.dt[None, a:b]), B=tdev(inp.B[None, a:b]),
                 C=tdev(inp.C[None, a:b]))
        ys, fs = ssd.chunked_scan(g["x"], g["dt"], tdev(inp.A), g["B"], g["C"], tdev(inp.D), 64,
                                  init_state=tdev(inp.init[s:s + 1]))
        torch.cuda.synchronize()
        assert_close(y[a:b], host(ys)[0], "f32", "seq %d y" % s)
        assert_close(fin[s], host(fs)[0], "f32", "seq %d final" % s)


@pytest.mark.parametrize("lens,walk", [((300, 280, 310, 290), True), ((64, 64, 64, 1000), False)],
                         ids=["balanced", "one-long-sequence"])
def test_state_path_follows_sequence_balance(lens, walk):
    """With the host copy of the offsets, a packed batch takes the walk only
    when no sequence has more than 1.5x the mean chunk count (the walk lasts
    as long as the longest sequence); both choices match the oracle."""
    wl = W.small_workload(seqlens=lens, H=32, P=64, N=64, G=2, chunk=64, dtype="bf16", init_var=0.1)
    inp = W.generate(wl, 91)
    say("case: state path for", lens)
    g = to_gpu(inp)
    st = []
    y, fin = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 64, init_state=g["init"],
                              cu_seqlens=[int(v) for v in inp.cu_seqlens], stage_ms=st)
    torch.cuda.synchronize()
    took_walk = st[ssd.STAGES.index("state_passing")] == 0.0
    assert took_walk == walk, st
    yr, fr = oracle_scan(inp)
    assert_close(host(y), yr, "bf16", "y")
    assert_close(host(fin), fr, "bf16", "final")


# ------------------------------------------------------------------ fused dt activation
# Raw step sizes (softplus argument) with a per-head bias; the kernels apply
# clamp(softplus(raw + bias), lo, hi) where dt enters (cumsum, decode) and the
# oracle runs on the same activation computed in fp64.
ACT = [
    # (batch, L, H, P, N, G, chunk, dtype): chunk-parallel state kernels, the walk, fp32
    (2, 300, 4, 64, 128, 2, 128, "bf16"),
    (4, 300, 32, 64, 128, 2, 128, "bf16"),
    (1, 200, 4, 16, 16, 1, 64, "f32"),
]


def raw_dt(shape, H, seed):
    rng = np.random.default_rng(seed)
    raw = rng.normal(-4.0, 1.0, size=shape).astype(np.float32)
    bias = rng.normal(0.0, 0.5, size=H).astype(np.float32)
    return raw, bias


@pytest.mark.parametrize("limit", [None, (0.001, 0.1)], ids=["nolimit", "limit"])
@pytest.mark.parametrize("case", ACT, ids=lambda c: "b%d-L%d-H%d-P%d-N%d-G%d-Q%d-%s" % c[:8])
def test_dt_activation_prefill(case, limit):
    b, L, H, P, N, G, Q, dt = case
    wl = W.small_workload(batch=b, seqlen=L, H=H, P=P, N=N, G=G, chunk=Q, dtype=dt, init_var=0.1)
    inp = W.generate(wl, 17 + H)
    raw, bias = raw_dt(inp.dt.shape, H, H + L)
    say("case: dt activation", case, limit)
    g = to_gpu(inp)
    y, fin = ssd.chunked_scan(g["x"], tdev(raw), g["A"], g["B"], g["C"], g["D"], Q, init_state=g["init"],
                              dt_softplus=True, dt_bias=tdev(bias), dt_limit=limit)
    torch.cuda.synchronize()
    dta = oracle.dt_activation(raw, bias, limit or (0.0, float("inf")))
    yr, fr = oracle.scan(inp.x, dta, inp.A, inp.B, inp.C, inp.D, init=inp.init)
    assert_close(host(y), yr, dt, "y")
    assert_close(host(fin), fr, dt, "final")


def test_dt_activation_decode_and_packed():
    """Packed prefill and then decode steps, both with the activation and no bias."""
    lens = (100, 0, 257, 64)
    wl = W.small_workload(seqlens=lens, H=8, P=64, N=64, G=2, chunk=64, dtype="f32", init_var=0.1,
                          decode_steps=3, decode_batch=len(lens))
    inp = W.generate(wl, 19)
    raw, _ = raw_dt(inp.dt.shape, 8, 5)
    g = to_gpu(inp)
    y, fin = ssd.chunked_scan(g["x"], tdev(raw), g["A"], g["B"], g["C"], g["D"], 64, init_state=g["init"],
                              cu_seqlens=g["cu"], dt_softplus=True)
    torch.cuda.synchronize()
    yr, fr = oracle.scan(inp.x, oracle.dt_activation(raw), inp.A, inp.B, inp.C, inp.D, init=inp.init,
                         cu_seqlens=inp.cu_seqlens)
    assert_close(host(y), yr, "f32", "y")
    assert_close(host(fin), fr, "f32", "final")
    state, ref = fin, fr
    for k, d in enumerate(inp.decode):
        rd, _ = raw_dt(d["dt"].shape, 8, 100 + k)
        yd = ssd.decode_step(state, tdev(d["x"]), tdev(rd), g["A"], tdev(d["B"]), tdev(d["C"]), g["D"],
                             dt_softplus=True, dt_limit=(0.0, 0.2))
        yref, ref = oracle.decode(ref, d["x"], oracle.dt_activation(rd, None, (0.0, 0.2)), inp.A, d["B"],
                                  d["C"], inp.D)
        assert_close(host(yd), yref, "f32", "decode y %d" % k)
        assert_close(host(state), ref, "f32", "decode state %d" % k)


def test_dt_activation_equals_activated_input():
    """The fused activation and the plain entry point on dt activated on the
    host (fp32) agree to fp32 rounding of dt."""
    wl = W.small_workload(batch=2, seqlen=333, H=4, P=32, N=64, G=1, chunk=64, dtype="f32", init_var=0.1)
    inp = W.generate(wl, 23)
    raw, bias = raw_dt(inp.dt.shape, 4, 9)
    g = to_gpu(inp)
    y1, f1 = ssd.chunked_scan(g["x"], tdev(raw), g["A"], g["B"], g["C"], g["D"], 64, init_state=g["init"],
                              dt_softplus=True, dt_bias=tdev(bias))
    pre = oracle.dt_activation(raw, bias).astype(np.float32)
    y2, f2 = ssd.chunked_scan(g["x"], tdev(pre), g["A"], g["B"], g["C"], g["D"], 64, init_state=g["init"])
    torch.cuda.synchronize()
    assert_close(host(y1), host(y2).astype(np.float64), "f32", "y")
    assert_close(host(f1), host(f2).astype(np.float64), "f32", "final")


# ------------------------------------------------------------------ cache semantics
def test_prefill_then_decode_equals_longer_prefill():
    wl = W.small_workload(batch=2, seqlen=600, H=4, P=64, N=128, G=1, chunk=128, dtype="f32",
                          init_var=0.1)
    inp = W.generate(wl, 90, A_range=(-0.3, -0.01))
    g = to_gpu(inp)
    L, k = 600, 5
    y_full, f_full = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 128,
                                      init_state=g["init"])
    sl = slice(0, L - k)
    _, state = ssd.chunked_scan(g["x"][:, sl].contiguous(), g["dt"][:, sl].contiguous(), g["A"],
                                g["B"][:, sl].contiguous(), g["C"][:, sl].contiguous(), g["D"], 128,
                                init_state=g["init"])
    for t in range(L - k, L):
        yd = ssd.decode_step(state, g["x"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"],
                             g["B"][:, t].contiguous(), g["C"][:, t].contiguous(), g["D"])
        assert_close(host(yd), host(y_full[:, t]), "f32", "decode vs prefill y at %d" % t)
    assert_close(host(state), host(f_full), "f32", "decode vs prefill state")


def test_decode_state_roundtrip_through_host_is_bitwise():
    wl = W.small_workload(batch=3, seqlen=100, H=4, P=64, N=64, G=2, chunk=64, dtype="bf16",
                          init_var=0.1, decode_steps=2)
    inp = W.generate(wl, 91)
    g = to_gpu(inp)
    _, st = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 64, init_state=g["init"])
    st2 = st.cpu().cuda()
    d = inp.decode[0]
    args = (tdev(d["x"], "bf16"), tdev(d["dt"]), g["A"], tdev(d["B"], "bf16"), tdev(d["C"], "bf16"), g["D"])
    y1 = ssd.decode_step(st, *args)
    y2 = ssd.decode_step(st2, *args)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(st, st2)


@pytest.mark.parametrize("P,N,dt", [(16, 16, "f32"), (64, 128, "bf16"), (32, 256, "bf16"), (128, 8, "f32"),
                                    (24, 40, "bf16"), (128, 256, "bf16"), (128, 256, "f32")])
def test_decode_shapes(P, N, dt):
    wl = W.small_workload(batch=5, seqlen=0, H=6, P=P, N=N, G=3, dtype=dt, init_var=0.1,
                          decode_steps=3, decode_batch=5)
    inp = W.generate(wl, 100 + P + N)
    state = tdev(inp.init)
    ref = inp.init.astype(np.float64)
    A, D = tdev(inp.A), tdev(inp.D)
    for k, d in enumerate(inp.decode):
        y = ssd.decode_step(state, tdev(d["x"], dt), tdev(d["dt"]), A, tdev(d["B"], dt), tdev(d["C"], dt), D)
        yr, ref = oracle.decode(ref, d["x"], d["dt"], inp.A, d["B"], d["C"], inp.D)
        assert_close(host(y), yr, dt, "decode y %d" % k)
        assert_close(host(state), ref, dt, "decode state %d" % k)


# ------------------------------------------------------------------ robustness
def test_deterministic_and_independent_of_workspace_contents():
    wl = W.small_workload(batch=2, seqlen=700, H=4, P=64, N=128, G=2, chunk=128, dtype="bf16",
                          init_var=0.1)
    inp = W.generate(wl, 110)
    g = to_gpu(inp)
    nbytes = ssd.workspace_size(g["x"], g["B"], 128)
    ws = torch.full((nbytes // 4,), float("nan"), device="cuda").view(torch.uint8)
    y_nan = torch.full(tuple(g["x"].shape), float("nan"), device="cuda")
    f_nan = torch.full((2, 4, 64, 128), float("nan"), device="cuda")
    y1, f1 = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 128, init_state=g["init"],
                              y=y_nan, final_state=f_nan, workspace=ws)
    y2, f2 = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 128, init_state=g["init"])
    torch.cuda.synchronize()
    assert torch.isfinite(y1.float()).all() and torch.isfinite(f1).all()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_bf16_output_is_the_rounded_fp32_output():
    """y in bf16 is exactly the fp32 y rounded to nearest even (same kernels,
    different store), for the prefill and the decode step."""
    wl = W.small_workload(batch=2, seqlen=500, H=4, P=64, N=128, G=2, chunk=128, dtype="bf16",
                          init_var=0.1, decode_steps=1)
    inp = W.generate(wl, 120)
    g = to_gpu(inp)
    y32, f32 = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 128, init_state=g["init"])
    y16, f16 = ssd.chunked_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 128, init_state=g["init"],
                                y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    assert torch.equal(y16, y32.to(torch.bfloat16)) and torch.equal(f16, f32)
    d = inp.decode[0]
    args = (tdev(d["x"], "bf16"), tdev(d["dt"]), g["A"], tdev(d["B"], "bf16"), tdev(d["C"], "bf16"), g["D"])
    s1, s2 = f32.clone(), f32.clone()
    yd32 = ssd.decode_step(s1, *args)
    yd16 = ssd.decode_step(s2, *args, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(yd16, yd32.to(torch.bfloat16)) and torch.equal(s1, s2)


@pytest.mark.parametrize("P", [24, 128])
def test_decode_bf16_output_rows_past_64(P):
    """The decode kernels store y with one coalesced store per 64 rows: bf16
    y is the rounded fp32 y for P below 64 and for rows 64..127, for the
    decode step and the windowed step."""
    wl = W.small_workload(batch=3, seqlen=0, H=4, P=P, N=64, G=2, dtype="bf16", init_var=0.1,
                          decode_steps=3, decode_batch=3)
    inp = W.generate(wl, 130 + P)
    A, D = tdev(inp.A), tdev(inp.D)
    d = inp.decode[0]
    args = (tdev(d["x"], "bf16"), tdev(d["dt"]), A, tdev(d["B"], "bf16"), tdev(d["C"], "bf16"), D)
    s1, s2 = tdev(inp.init), tdev(inp.init)
    y32 = ssd.decode_step(s1, *args)
    y16 = ssd.decode_step(s2, *args, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32.to(torch.bfloat16)) and torch.equal(s1, s2)
    ref_y, _ = oracle.decode(inp.init, d["x"], d["dt"], inp.A, d["B"], d["C"], inp.D)
    assert_close(host(y32), ref_y, "bf16", "decode y")
    win = [torch.stack([tdev(e[k], dt) for e in inp.decode], dim=1).contiguous()
           for k, dt in (("x", "bf16"), ("dt", "f32"), ("B", "bf16"), ("C", "bf16"))]
    for flush in (False, True):
        w1, w2 = tdev(inp.init), tdev(inp.init)
        y32 = ssd.decode_window_step(w1, win[0], win[1], A, win[2], win[3], D, 2, flush)
        y16 = ssd.decode_window_step(w2, win[0], win[1], A, win[2], win[3], D, 2, flush,
                                     y_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(y16, y32.to(torch.bfloat16)) and torch.equal(w1, w2), flush


def test_empty_batch_is_a_no_op():
    x = torch.zeros((0, 10, 2, 16), device="cuda")
    y, fin = ssd.chunked_scan(x, torch.zeros((0, 10, 2), device="cuda"), torch.zeros(2, device="cuda"),
                              torch.zeros((0, 10, 1, 16), device="cuda"),
                              torch.zeros((0, 10, 1, 16), device="cuda"), torch.zeros(2, device="cuda"), 64)
    torch.cuda.synchronize()
    assert y.shape == x.shape and fin.shape == (0, 2, 16, 16)


def test_binding_rejects_wrong_shapes():
    x = torch.zeros((1, 64, 2, 16), device="cuda")
    with pytest.raises(ValueError):
        ssd.chunked_scan(x, torch.zeros((1, 64, 3), device="cuda"), torch.zeros(2, device="cuda"),
                         torch.zeros((1, 64, 1, 16), device="cuda"), torch.zeros((1, 64, 1, 16), device="cuda"),
                         torch.zeros(2, device="cuda"), 64)
