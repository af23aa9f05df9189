#!/usr/bin/env python3
"""Benchmark of the SSD hot path on one MI355X.

One step = one chunked prefill over the Mamba-2 2.7B-shaped layer workload
(batch 8, L 8192, H 80, P 64, N 128, G 1, chunk 256, bf16 x/B/C, fp32 state)
followed by one cached decode step over the 2.7B-shaped decode batch (256
sequences, fp32 state [256, 80, 64, 128]).  Inputs are seeded synthetic
tensors already resident in HBM when timing starts.

Printed (one JSON line on stdout): prefill tokens/s as ``value``, TFLOP/s,
decode GB/s, the roofline of the dominant prefill kernel (chunk_scan), the
decode kernel's roofline, and the fp64 CPU oracle timed on a bounded sample
of the same workload on this host's cores.
Progress lines go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
MFMA_TARGET = 0.40              # the prefill's contraction kernels: fraction of the bf16 peak asked for


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def prefill_flops(wl, causal=False):
    """Algorithmic FLOPs of the chunked form: per full chunk 2Q^2N (C.B^T, per
    group) + 2Q^2P (masked scores times x) + 2QNP (chunk state) + 2QNP (state
    term of the output), per head.  Causal counts Q(Q+1)/2 pairs instead of Q^2."""
    Q, H, P, N, G = wl.chunk, wl.H, wl.P, wl.N, wl.G
    nch = wl.tokens // Q
    pairs = Q * (Q + 1) / 2 if causal else Q * Q
    return nch * (G * 2 * pairs * N + H * (2 * pairs * P + 4 * Q * N * P))


def kernel_work(wl, es=2, ys=4, fused=True):
    """Algorithmic FLOPs and HBM bytes of each MFMA kernel launch (dense batch).

    chunk_state: 2QNP per (chunk, head); reads x and B^T once, writes one fp32
    P x N state per (chunk, head).  With `fused` (one walk per (sequence,
    head, column tile) that also passes the states between chunks) those
    written states are the entering ones, and it also reads the initial and
    writes the final state; there is no separate state_passing launch.
    chunk_scan: 2QNP (state term) + 2Q^2P (dense intra-chunk product) per
    (chunk, head); reads x, C, the causal half of C.B^T, the per-chunk decay
    sums and one fp32 entering state per (chunk, head), writes y once."""
    Q, H, P, N, G, b, L = wl.chunk, wl.H, wl.P, wl.N, wl.G, wl.batch, wl.seqlen
    nch = b * (-(-L // Q))
    T = b * L
    nti = Q // 32
    state = nch * H * P * N * 4
    ks = {"flops": nch * H * 2 * Q * N * P,
          "flops_causal": nch * H * 2 * Q * N * P,
          "bytes": T * H * P * es + nch * G * N * Q * es + state + 2 * nch * H * Q * 4}
    kc = {"flops": nch * H * (2 * Q * N * P + 2 * Q * Q * P),
          "flops_causal": nch * H * (2 * Q * N * P + Q * (Q + 1) * P),
          "bytes": (T * H * P * es + T * H * P * ys + T * G * N * es + state
                    + nch * G * nti * (nti + 1) // 2 * 1024 * es + 2 * nch * H * Q * 4)}
    kp = {"flops": 0, "flops_causal": 0, "bytes": 2 * state + nch * H * 4 + 2 * b * H * P * N * 4}
    if fused == "scan_walk":
        # one launch: the chunk states, their passing and y; it reads x, C,
        # B^T, the causal C.B^T tiles, the decay sums and steps and the
        # initial states, and writes y and the final states.  No per-chunk
        # state and no per-token weight table reach memory.
        nt = 128 if N <= 128 else 256
        kw = {"flops": ks["flops"] + kc["flops"], "flops_causal": ks["flops_causal"] + kc["flops_causal"],
              "bytes": (T * H * P * es + T * H * P * ys + T * G * N * es + nch * G * nt * Q * es
                        + nch * G * nti * (nti + 1) // 2 * 1024 * es + 2 * nch * H * Q * 4
                        + 2 * b * H * P * N * 4)}
        return {"scan_walk": kw}
    if fused:
        ks["bytes"] += 2 * b * H * P * N * 4
        return {"chunk_state": ks, "chunk_scan": kc}
    return {"chunk_state": ks, "chunk_scan": kc, "state_passing": kp}


def roofline_of(wk, ms, kernel):
    """Roofline of one kernel launch from its algorithmic work and measured
    duration.  The roof that bounds it is the one its arithmetic intensity
    (algorithmic FLOPs per HBM byte) selects against the ridge point
    (bf16 peak / HBM peak); both fractions are reported either way."""
    gbs = wk["bytes"] / (ms * 1e-3) / 1e9
    tfl = wk["flops"] / (ms * 1e-3) / 1e12
    tfl_c = wk["flops_causal"] / (ms * 1e-3) / 1e12
    fh, fm = gbs / HBM_PEAK_GBS, tfl / BF16_PEAK_TFLOPS
    ai = wk["flops"] / wk["bytes"]
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    r = ({"bound": "mfma", "achieved": round(tfl, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
          "frac": round(fm, 4)} if ai > ridge else
         {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(fh, 4)})
    r.update({"traffic": None, "kernel": kernel, "avg_ms": round(ms, 4),
              "algorithmic_flops": wk["flops"], "algorithmic_flops_causal": wk["flops_causal"],
              "algorithmic_bytes": wk["bytes"], "flop_per_byte": round(ai, 1), "ridge_flop_per_byte": round(ridge, 1),
              "tflops": round(tfl, 2), "mfma_frac": round(fm, 4), "tflops_causal": round(tfl_c, 2),
              "mfma_frac_causal": round(tfl_c / BF16_PEAK_TFLOPS, 4), "hbm_frac": round(fh, 4)})
    return r


def decode_bytes(wd, es=2, ys=4):
    """HBM bytes of one decode step: the fp32 state read and written, x (es
    bytes per element), y (ys, fp32 by default), B and C, dt, A and D."""
    b, H, P, N, G = wd.nseq, wd.H, wd.P, wd.N, wd.G
    return (2 * b * H * P * N * 4 + b * H * P * es + b * H * P * ys + 2 * b * G * N * es + b * H * 4
            + 2 * H * 4)


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, max_seqs=None, one_core_seqs=1):
    """The fp64 oracle (sequential recurrence, OpenMP over (sequence, head))
    on the prefill workload's own inputs, timed twice: on all the host threads
    OpenMP gets, over all heads of the first `max_seqs` sequences (all of them
    by default, ~20 core-seconds), and on one thread over all heads of the
    first `one_core_seqs` sequences (~3 s).  Both are scaled to tokens/s of
    the whole layer (every head of a token)."""
    import oracle
    wl = inp.wl
    nseq = wl.batch if max_seqs is None else min(max_seqs, wl.batch)
    threads = oracle.threads()

    def timed(n, nthreads):
        init = None if inp.init is None else inp.init[:n]
        t0 = time.perf_counter()
        cpu0 = time.process_time()
        oracle.scan(inp.x[:n], inp.dt[:n], inp.A, inp.B[:n], inp.C[:n], inp.D, init=init, nthreads=nthreads)
        return time.perf_counter() - t0, time.process_time() - cpu0

    t, cpu_s = timed(nseq, 0)
    n1 = min(one_core_seqs, wl.batch)
    t1, _ = timed(n1, 1)
    return {"value": nseq * wl.seqlen / t, "unit": "tokens/s", "cores": int(threads),
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(), "kind": "oracle",
            "seconds": round(t, 3), "cpu_seconds": round(cpu_s, 1),
            "sample": "fp64 sequential oracle (C, OpenMP over (sequence, head)) on %d of %d "
                      "sequences x all %d heads x %d tokens of the prefill workload"
                      % (nseq, wl.batch, wl.H, wl.seqlen),
            "one_core": {"value": n1 * wl.seqlen / t1, "unit": "tokens/s", "cores": 1, "seconds": round(t1, 3),
                         "sample": "the same oracle on one thread: %d sequence x all %d heads x %d tokens"
                                   % (n1, wl.H, wl.seqlen)}}


def decode_vs_recompute(torch, ssd, context=4096, steps=64, reps=20):
    """Per-token cost of cached decode against recomputing the whole prefix, at
    batch 1 and `context` tokens, on the 130M-like (H=24) and 2.7B-like (H=80)
    layer shapes (P=64, N=128, bf16 x/B/C, fp32 state): the prefill of
    `context` tokens is what one token costs without a cache; the decode step
    is what it costs with one, launched eagerly or as a graph-captured loop of
    `steps` steps."""
    from mamba_ssd_chunked_02_amd.decode_loop import DecodeLoop
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(11)
    out = {}
    for name, H in (("130m_layer", 24), ("2p7b_layer", 80)):
        P, N = 64, 128
        x = torch.randn(1, context, H, P, generator=g).to(torch.bfloat16).to(dev)
        dt = (torch.rand(1, context, H, generator=g) * 0.099 + 0.001).to(dev)
        A = (-torch.exp(torch.rand(H, generator=g) * np.log(16.0))).to(dev)
        B = (torch.randn(1, context, 1, N, generator=g) / N ** 0.5).to(torch.bfloat16).to(dev)
        C = (torch.randn(1, context, 1, N, generator=g) / N ** 0.5).to(torch.bfloat16).to(dev)
        D = torch.randn(H, generator=g).to(dev)
        y = torch.empty(tuple(x.shape), device=dev)
        fin = torch.empty(1, H, P, N, device=dev)
        ws = torch.empty(ssd.workspace_size(x, B, 256), dtype=torch.uint8, device=dev)
        loop = DecodeLoop(steps, 1, H, P, N, 1, A, D, dtype=torch.bfloat16)
        loop.x.normal_()
        loop.dt.uniform_(0.001, 0.1)
        loop.B.normal_(0, N ** -0.5)
        loop.C.normal_(0, N ** -0.5)

        def timed(fn, n):
            for _ in range(3):
                fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            e1.synchronize()
            return e0.elapsed_time(e1) / n

        pre = timed(lambda: ssd.chunked_scan(x, dt, A, B, C, D, 256, y=y, final_state=fin, workspace=ws),
                    reps)
        graph = timed(loop.replay, reps) / steps
        eager = timed(loop.run_eager, reps) / steps
        out[name] = {"recompute_ms_per_token": round(pre, 4), "cached_graph_ms_per_token": round(graph, 5),
                     "cached_eager_ms_per_token": round(eager, 5),
                     "speedup_graph": round(pre / graph, 1), "speedup_eager": round(pre / eager, 1)}
        del x, dt, B, C, y, ws, loop
    out["what"] = ("batch 1, %d-token context: prefill of the whole context (no cache) vs one cached "
                   "decode step (graph-captured loop of %d steps, or eager launches)" % (context, steps))
    return out


def decode_window(torch, ssd, wd, window=16, reps=20):
    """Exact windowed decode against the ordinary decode step on the decode
    batch (b256 H80 P64 N128, bf16 x/B/C, fp32 state): a window of `window`
    tokens through ssd_decode_window_step (slot t = 0..window-1, the state
    written back at the last slot only) against `window` ordinary steps.  The
    window form reads the state every token and writes it once per window."""
    dev = torch.device("cuda:0")
    b, H, P, N, G = wd.nseq, wd.H, wd.P, wd.N, wd.G
    g = torch.Generator(device="cpu").manual_seed(13)
    state = (torch.randn(b, H, P, N, generator=g) * 0.3).to(dev)
    x = torch.randn(b, window, H, P, generator=g).to(torch.bfloat16).to(dev)
    dt = (torch.rand(b, window, H, generator=g) * 0.099 + 0.001).to(dev)
    A = (-torch.exp(torch.rand(H, generator=g) * np.log(16.0))).to(dev)
    B = (torch.randn(b, window, G, N, generator=g) / N ** 0.5).to(torch.bfloat16).to(dev)
    C = (torch.randn(b, window, G, N, generator=g) / N ** 0.5).to(torch.bfloat16).to(dev)
    D = torch.randn(H, generator=g).to(dev)
    y = torch.empty(b, H, P, device=dev)
    # per-token views for the ordinary step
    xs = [x[:, t].contiguous() for t in range(window)]
    dts = [dt[:, t].contiguous() for t in range(window)]
    Bs = [B[:, t].contiguous() for t in range(window)]
    Cs = [C[:, t].contiguous() for t in range(window)]

    def win():
        for t in range(window):
            ssd.decode_window_step(state, x, dt, A, B, C, D, t, t == window - 1, y=y)

    def plain():
        for t in range(window):
            ssd.decode_step(state, xs[t], dts[t], A, Bs[t], Cs[t], D, y=y)

    def timed(fn):
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / (reps * window)

    w_ms = timed(win)
    p_ms = timed(plain)
    # the two kernel variants on their own: a read-only step (slot 7) and a flush
    read_ms = timed(lambda: ssd.decode_window_step(state, x, dt, A, B, C, D, 7, False, y=y))
    flush_ms = timed(lambda: ssd.decode_window_step(state, x, dt, A, B, C, D, window - 1, True, y=y))
    sb = b * H * P * N * 4
    es = 2
    # per token: the state read, the state written once per window, the window
    # slots 0..t of x, B, C and dt read (mean over t), y written
    slots = (window + 1) / 2
    wbytes = sb + sb / window + slots * (b * H * P * es + 2 * b * G * N * es + b * H * 4) + b * H * P * 4 + 2 * H * 4
    pbytes = decode_bytes(wd)
    return {"window": window, "ms_per_token": round(w_ms, 4), "plain_ms_per_token": round(p_ms, 4),
            "speedup": round(p_ms / w_ms, 3), "bytes_per_token": int(wbytes), "plain_bytes_per_token": pbytes,
            "gbps": round(wbytes / (w_ms * 1e-3) / 1e9, 1),
            "read_only_step_ms": round(read_ms * window, 4), "flush_step_ms": round(flush_ms * window, 4),
            "read_only_step_gbps": round(sb / (read_ms * window * 1e-3) / 1e9, 1),
            "what": "ssd_decode_window_step over a %d-token window (state written once per window) vs "
                    "%d ssd_decode_step calls, b%d H%d P%d N%d, eager back-to-back" % (window, window, b, H, P, N)}


def conv1d_measure(torch, ssd, wl, wd, reps=20):
    """Causal conv1d + SiLU on the xBC channels of the 2.7B-shaped layer
    (C = H*P + 2*G*N = 5376, width 4, bf16 in and out), written straight into
    the scan's x, B and C buffers: the prefill batch (b8 L8192) and one decode
    step of the decode batch (b256).  Algorithmic bytes: x read once and the
    output written once (plus weights, bias and conv states)."""
    dev = torch.device("cuda:0")
    H, P, G, N, K = wl.H, wl.P, wl.G, wl.N, 4
    parts = [H * P, G * N, G * N]
    C = sum(parts)
    b, L = wl.batch, wl.seqlen
    g = torch.Generator(device="cpu").manual_seed(17)
    x = torch.randn(b, L, C, generator=g).to(torch.bfloat16).to(dev)
    w = ((torch.rand(C, K, generator=g) * 2 - 1) * 0.5).to(dev)
    bias = ((torch.rand(C, generator=g) * 2 - 1) * 0.5).to(dev)
    st = torch.randn(b, K - 1, C, generator=g).to(torch.bfloat16).to(dev)
    fin = torch.empty_like(st)
    outs = [torch.empty(b, L, c, dtype=torch.bfloat16, device=dev) for c in parts]

    def timed(fn, n):
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    pre = timed(lambda: ssd.causal_conv1d(x, w, bias, conv_state=st, final_conv_state=fin, split=parts,
                                          outs=outs), reps)
    pbytes = 2 * b * L * C * 2 + C * (K + 1) * 4 + 2 * b * (K - 1) * C * 2
    del x, outs
    bd = wd.nseq
    xd = torch.randn(bd, C, generator=g).to(torch.bfloat16).to(dev)
    sd = torch.randn(bd, K - 1, C, generator=g).to(torch.bfloat16).to(dev)
    od = [torch.empty(bd, c, dtype=torch.bfloat16, device=dev) for c in parts]
    step = timed(lambda: ssd.conv1d_step(sd, xd, w, bias, split=parts, outs=od), 100)
    sbytes = bd * C * 2 * 2 + 2 * bd * (K - 1) * C * 2 + C * (K + 1) * 4
    gbs = pbytes / (pre * 1e-3) / 1e9
    return {"prefill_ms": round(pre, 4), "prefill_tokens_per_s": round(b * L / (pre * 1e-3), 1),
            "prefill_bytes": pbytes, "prefill_gbps": round(gbs, 1), "prefill_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "step_ms": round(step, 5), "step_bytes": sbytes,
            "step_gbps": round(sbytes / (step * 1e-3) / 1e9, 1),
            "what": "causal conv1d width 4 + SiLU over xBC (C=%d) split into x/B/C: prefill b%d L%d, "
                    "decode step b%d; bf16 in/out, eager back-to-back" % (C, b, L, bd)}


def environment(torch, clocks=True):
    """What the numbers were measured on: device, HIP and torch versions, and
    the clock levels rocm-smi reports at bench start (the device is idle
    then, so sclk reads its idle level; None when rocm-smi is absent or
    clocks is False: under a profiler that preloads itself into every child,
    rocm-smi's interpreter would start as a GPU process)."""
    import subprocess
    env = {"gpu": torch.cuda.get_device_name(0), "gcn_arch": torch.cuda.get_device_properties(0).gcnArchName,
           "hip": torch.version.hip, "torch": torch.__version__, "clocks": None}
    if not clocks:
        return env
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        lines = [l.strip() for l in r.stdout.splitlines() if "sclk" in l or "mclk" in l or "fclk" in l]
        env["clocks"] = lines[:6] or None
    except Exception:  # pragma: no cover - rocm-smi absent or not permitted
        pass
    return env


def _pct(v):
    v = np.asarray(v)
    return {"p10": round(float(np.percentile(v, 10)), 4), "p50": round(float(np.percentile(v, 50)), 4),
            "p90": round(float(np.percentile(v, 90)), 4)}


def other_prefill(torch, ssd, reps=20):
    """Prefill throughput and TFLOPS of the other two prefill configurations, through the
    plain entry point: the 130M-shaped layer (b1 L4096 H24 P64 N128 G1) and
    the packed grouped batch ({1024, 4096, 12288, 32768} tokens, H128 P64
    N128 G8, offsets given with their host copy).  bf16 x/B/C, fp32 dt/A/D,
    initial states ~N(0, 0.1), chunk 256; inputs drawn on the GPU."""
    from mamba_ssd_chunked_02_amd import workloads as W
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(23)
    out = {}
    for name, lens, H, G, dense in (("130m_layer_b1_L4096", [4096], 24, 1, True),
                                    ("varlen_h128_g8_4seqs", [1024, 4096, 12288, 32768], 128, 8, False)):
        P, N = 64, 128
        T = sum(lens)
        lead = (1, T) if dense else (T,)
        x = torch.randn(*lead, H, P, generator=g).to(torch.bfloat16).to(dev)
        dt = (torch.rand(*lead, H, generator=g) * 0.099 + 0.001).to(dev)
        A = (-torch.exp(torch.rand(H, generator=g) * np.log(16.0))).to(dev)
        B = (torch.randn(*lead, G, N, generator=g) / N ** 0.5).to(torch.bfloat16).to(dev)
        C = (torch.randn(*lead, G, N, generator=g) / N ** 0.5).to(torch.bfloat16).to(dev)
        D = torch.randn(H, generator=g).to(dev)
        init = (torch.randn(len(lens), H, P, N, generator=g) * 0.1 ** 0.5).to(dev)
        cu_host = None if dense else [0] + list(np.cumsum(lens))
        cu = None if dense else torch.tensor(cu_host, dtype=torch.int32, device=dev)
        y = torch.empty(tuple(x.shape), device=dev)
        fin = torch.empty_like(init)
        ws = torch.empty(ssd.workspace_size(x, B, 256, cu_seqlens=cu), dtype=torch.uint8, device=dev)

        def run():
            ssd.chunked_scan(x, dt, A, B, C, D, 256, init_state=init, cu_seqlens=cu, cu_seqlens_host=cu_host,
                             y=y, final_state=fin, workspace=ws)
        for _ in range(3):
            run()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        wl = W.CONFIGS[1] if dense else W.CONFIGS[4]
        assert wl.tokens == T and wl.H == H and wl.G == G
        out[name] = {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
                     "tflops_dense": round(prefill_flops(wl) / (ms * 1e-3) / 1e12, 2),
                     "tflops_causal": round(prefill_flops(wl, causal=True) / (ms * 1e-3) / 1e12, 2)}
        del x, dt, B, C, y, ws
    out["what"] = "plain-entry-point prefill, back-to-back calls, the other two prefill configurations"
    return out


# the sources that define and launch the prefill kernels (the counters in the
# traffic summary describe those kernels only)
PREFILL_SOURCES = ("ssd_api.cpp", "ssd_device.h", "ssd_internal.h", "ssd_prefill.hip", "ssd_prefill_shared.h",
                   "ssd_scan_walk.hip")
# the sources that define and launch the decode kernel
DECODE_SOURCES = ("ssd_api.cpp", "ssd_device.h", "ssd_internal.h", "ssd_decode.hip")


def _source_digest(files=PREFILL_SOURCES):
    """sha256 of kernel sources, to tell whether counters are stale."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mamba_ssd_chunked_02_amd", "csrc")
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _traffic(path, kernel, alg_bytes, files=PREFILL_SOURCES):
    """HBM bytes per launch of `kernel` from a committed counter summary:
    lines `key: value` with fetch_kib, write_kib (per dispatch, rocprofv3
    FETCH_SIZE / WRITE_SIZE), copy_fetch_factor and copy_write_factor (known
    bytes of a plain copy / what the same counters read for it) and
    source_digest.  None when the file is missing or the kernels changed."""
    if not path or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("source_digest") != _source_digest(files):
            return None
        fetch = float(kv["fetch_kib"]) * 1024 * float(kv["copy_fetch_factor"])
        write = float(kv["write_kib"]) * 1024 * float(kv["copy_write_factor"])
    except (KeyError, ValueError):
        return None
    return {"bytes": round(fetch + write), "fetch_bytes": round(fetch), "write_bytes": round(write),
            "over_algorithmic": round((fetch + write) / alg_bytes, 3), "source": os.path.relpath(path, ROOT)}


def copy_calibration():
    """A plain device-to-device copy of 1 GiB (read 1 GiB, write 1 GiB), run
    under rocprofv3 --pmc to calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="leave out the reports beside the timed step (decode loop vs recompute, windowed\n"
                         "decode, conv1d, fused dt activation) and the rocm-smi clock query; the timed step\n"
                         "and its rooflines are unchanged")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic_scan_walk_2p7b.txt"),
                    help="rocprofv3 FETCH_SIZE/WRITE_SIZE summary of the dominant kernel")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the scan shards "
              "over independent (sequence, head) pairs with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import mamba_ssd_chunked_02_amd as ssd
    from mamba_ssd_chunked_02_amd import workloads as W

    dev = torch.device("cuda:0")
    env = environment(torch, clocks=not args.no_extras)
    wl = W.CONFIGS[3]
    wd = W.CONFIGS[2]
    log("generating prefill inputs:", wl.name)
    inp = W.generate(wl, W.SEED_BASE + 3, decode_steps=0)

    def up(a, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        if bf16:
            t = t.to(torch.bfloat16)
        return t.to(dev)

    x, dtt, A, Bm, Cm, D = (up(inp.x, True), up(inp.dt), up(inp.A), up(inp.B, True),
                            up(inp.C, True), up(inp.D))
    init = up(inp.init)
    y = torch.empty(tuple(x.shape), dtype=torch.float32, device=dev)  # fp32 y (the default)
    fin = torch.empty_like(init)
    nbytes = ssd.workspace_size(x, Bm, wl.chunk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    log("generating decode inputs:", wd.name)
    dinp = W.generate(wd, W.SEED_BASE + 2, decode_steps=1)
    state = up(dinp.init)
    d0 = dinp.decode[0]
    dx, ddt, dA, dB, dC, dD = (up(d0["x"], True), up(d0["dt"]), up(dinp.A), up(d0["B"], True),
                               up(d0["C"], True), up(dinp.D))
    dy = torch.empty(tuple(dx.shape), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def prefill(stage_ms=None):
        ssd.chunked_scan(x, dtt, A, Bm, Cm, D, wl.chunk, init_state=init, y=y, final_state=fin,
                         workspace=ws, stage_ms=stage_ms)

    def decode():
        ssd.decode_step(state, dx, ddt, dA, dB, dC, dD, y=dy)

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        prefill([])
        decode()
    torch.cuda.synchronize()

    log("timing", args.steps, "steps")
    # the library queues its kernels on torch's current stream, which these
    # events are recorded on.  The K steps are queued back to back between
    # two synchronizations, as a serving loop runs them: the host prepares
    # the next launches while the GPU works, so the events time the GPU's
    # work rather than the host's argument checks before each launch
    stream = torch.cuda.current_stream(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_wall0 = time.perf_counter()
    torch.cuda.synchronize()
    for e0, e1, e2 in evs:
        e0.record(stream)
        prefill()
        e1.record(stream)
        decode()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    pre_ms = [e0.elapsed_time(e1) for e0, e1, _ in evs]
    dec_ms = [e1.elapsed_time(e2) for _, e1, e2 in evs]
    log("timed region %.3f s" % wall)

    # the same prefill with the dt activation fused (the raw input is the
    # inverse softplus of the workload's dt, so the kernels see the same dt)
    raw = up(np.log(np.expm1(inp.dt.astype(np.float64))).astype(np.float32))

    y16 = None if args.no_extras else torch.empty(tuple(x.shape), dtype=torch.bfloat16, device=dev)

    def back_to_back(act):
        def one():
            if act == "softplus":
                ssd.chunked_scan(x, raw, A, Bm, Cm, D, wl.chunk, init_state=init, y=y, final_state=fin,
                                 workspace=ws, dt_softplus=True)
            elif act == "bf16_y":
                ssd.chunked_scan(x, dtt, A, Bm, Cm, D, wl.chunk, init_state=init, y=y16, final_state=fin,
                                 workspace=ws)
            else:
                prefill()
        for _ in range(3):
            one()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(args.steps):
            one()
        a1.record(stream)
        a1.synchronize()
        return a0.elapsed_time(a1) / args.steps

    plain_b2b_ms = back_to_back(None) if not args.no_extras else None
    act_ms = back_to_back("softplus") if not args.no_extras else None
    y16_ms = back_to_back("bf16_y") if not args.no_extras else None
    del raw, y16

    # per-kernel durations: the same prefill through the measuring entry point
    # (HIP events before and after every stage on the same stream)
    stages = []
    for i in range(args.steps):
        st = []
        prefill(st)
        stages.append(st)

    # the decode kernel in steady state: back-to-back steps on the same state,
    # as a serving loop runs them (in the step above it follows a prefill)
    for _ in range(20):
        decode()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(100):
        decode()
    c1.record(stream)
    c1.synchronize()
    decode_steady_ms = c0.elapsed_time(c1) / 100

    stages = np.array(stages)              # [steps, 6] ms
    stage_mean = stages.mean(axis=0)
    prefill_ms = float(np.mean(pre_ms))
    decode_ms = float(np.mean(dec_ms))
    tokens = wl.tokens
    value = tokens / (prefill_ms * 1e-3)
    dense_tf = prefill_flops(wl) / (prefill_ms * 1e-3) / 1e12
    causal_tf = prefill_flops(wl, causal=True) / (prefill_ms * 1e-3) / 1e12

    # rooflines of the prefill kernels; the slowest one is the reported one.
    # The stages that ran tell the path: the scan walk alone, the state walk
    # (state passing inside chunk_state) + chunk_scan, or all three
    if float(stage_mean[ssd.STAGES.index("scan_walk")]) > 0.0:
        fused = "scan_walk"
    else:
        fused = float(stage_mean[ssd.STAGES.index("state_passing")]) == 0.0
    work = kernel_work(wl, fused=fused)
    names = {"chunk_state": ("ssd_chunk_state_passing_kernel<bf16,NT=128,Q=256>" if fused else
                             "ssd_chunk_state_kernel<bf16,NT=128,Q=256>"),
             "state_passing": "ssd_state_passing_kernel",
             "chunk_scan": "ssd_chunk_scan_kernel<bf16,f32,NT=128,Q=256>",
             "scan_walk": "ssd_scan_walk_kernel<f32 y,NU=5>"}
    roofs = {}
    for k, wk in work.items():
        ms = float(stage_mean[ssd.STAGES.index(k)])
        roofs[k] = roofline_of(wk, ms, names[k])
    dominant = max(roofs, key=lambda k: roofs[k]["avg_ms"])
    roof = dict(roofs[dominant])
    if args.traffic:
        roof["traffic"] = _traffic(args.traffic, names[dominant], roof["algorithmic_bytes"])
        roofs[dominant]["traffic"] = roof["traffic"]
    # the contraction kernels: chunk_state and chunk_scan, or the scan walk
    # that does both (state_passing has no contraction)
    mk = [k for k in work if k != "state_passing"]
    mfma_ms = float(sum(stage_mean[ssd.STAGES.index(k)] for k in mk))
    contraction_tf = sum(work[k]["flops"] for k in mk) / (mfma_ms * 1e-3) / 1e12
    contraction_tf_c = sum(work[k]["flops_causal"] for k in mk) / (mfma_ms * 1e-3) / 1e12
    # the contraction kernels against the 40% bf16 target, beside the dominant
    # kernel's own roofline (which is the HBM roof: its arithmetic intensity
    # sits left of the ridge)
    roof["contraction_kernels"] = {
        "ms": round(mfma_ms, 4), "tflops_dense": round(contraction_tf, 2),
        "mfma_frac_dense": round(contraction_tf / BF16_PEAK_TFLOPS, 4),
        "tflops_causal": round(contraction_tf_c, 2),
        "mfma_frac_causal": round(contraction_tf_c / BF16_PEAK_TFLOPS, 4),
        "mfma_target": MFMA_TARGET}
    dbytes = decode_bytes(wd)
    dgbs = dbytes / (decode_ms * 1e-3) / 1e9
    roof_dec = {"bound": "hbm", "achieved": round(dgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dgbs / HBM_PEAK_GBS, 4),
                "traffic": _traffic(os.path.join(ROOT, "profiles", "traffic_decode_2p7b.txt"),
                                    "ssd_decode_kernel", dbytes, DECODE_SOURCES),
                "kernel": "ssd_decode_kernel<bf16,32>", "avg_ms": round(decode_ms, 4),
                "algorithmic_bytes": dbytes}

    # context for the HBM fractions: a plain device copy of the decode state's
    # size (read + write), the practical streaming rate of this device
    src = torch.empty_like(state)
    dst = torch.empty_like(state)
    for _ in range(3):
        dst.copy_(src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    c1.synchronize()
    copy_ms = c0.elapsed_time(c1) / 10
    copy_gbs = 2 * state.numel() * 4 / (copy_ms * 1e-3) / 1e9
    # the same rooflines against what this device streams in practice
    for r in [roof, roof_dec] + list(roofs.values()):
        if r["unit"] == "GB/s":
            r["frac_of_copy_rate"] = round(r["achieved"] / copy_gbs, 4)
        elif r.get("hbm_frac") is not None:
            r["frac_of_copy_rate"] = round(r["hbm_frac"] * HBM_PEAK_GBS / copy_gbs, 4)
    del src, dst

    dvr = dwin = dconv = dother = None
    if not args.no_extras:
        log("cached decode vs full-prefix recompute")
        dvr = decode_vs_recompute(torch, ssd)
        log("windowed exact decode vs ordinary decode")
        dwin = decode_window(torch, ssd, wd)
        log("causal conv1d")
        dconv = conv1d_measure(torch, ssd, wl, wd)
        log("other prefill configurations")
        dother = other_prefill(torch, ssd)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        try:
            cpu = cpu_baseline(inp)
        except Exception as e:  # pragma: no cover - reported, not fatal
            cpu = {"error": repr(e)}

    out = {
        "metric": "SSD prefill tokens/s + TFLOPS; decode-step HBM GB/s vs peak (2.7B shape)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prefill_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Mamba-2 2.7B-shaped SSD layer: prefill b8 L8192 H80 P64 N128 G1 "
                               "chunk256 (bf16 x/B/C, fp32 dt/A/D/state, init~N(0,0.1)) + one "
                               "decode step b256 H80 P64 N128 (fp32 state)",
                   "global_batch": wl.batch, "seq_len": wl.seqlen, "parallelism": "none (1 GPU)"},
        "tflops_dense": round(dense_tf, 2),
        "tflops_causal": round(causal_tf, 2),
        "stage_ms": {k: round(float(v), 4) for k, v in zip(ssd.STAGES, stage_mean)},
        "stage_ms_sum": round(float(stage_mean.sum()), 4),
        "stage_ms_note": "per-stage HIP events through ssd_chunked_scan_profiled, separate runs; "
                         "ms_per_step is the plain entry point between two events",
        "decode": {"ms_per_step": round(decode_ms, 4), "gbps": round(dgbs, 1),
                   "frac_of_hbm_peak": round(dgbs / HBM_PEAK_GBS, 4), "bytes_per_step": dbytes,
                   "steady_ms_per_step": round(decode_steady_ms, 4),
                   "steady_gbps": round(dbytes / (decode_steady_ms * 1e-3) / 1e9, 1),
                   "steady": "100 back-to-back steps after the timed region"},
        "step_ms_prefill_plus_decode": round(prefill_ms + decode_ms, 4),
        "ms_per_step_note": "each timed step is one prefill then one decode step, each between HIP events; "
                            "the K steps are queued back to back between two synchronizations; "
                            "ms_per_step and value cover the prefill part (the metric is prefill tokens/s), "
                            "decode.ms_per_step the decode part, step_ms_prefill_plus_decode both",
        "decode_vs_recompute": dvr,
        "decode_window": dwin,
        "conv1d": dconv,
        "other_prefill": dother,
        "prefill_dt_activation": None if act_ms is None else {
            "ms_per_step": round(act_ms, 4), "tokens_per_s": round(tokens / (act_ms * 1e-3), 1),
            "plain_ms_per_step": round(plain_b2b_ms, 4),
            "what": "same prefill through ssd_chunked_scan_dt_act (softplus fused into the cumsum kernel) "
                    "and through ssd_chunked_scan, back-to-back calls each"},
        "prefill_bf16_y": None if y16_ms is None else {
            "ms_per_step": round(y16_ms, 4), "tokens_per_s": round(tokens / (y16_ms * 1e-3), 1),
            "plain_ms_per_step": round(plain_b2b_ms, 4),
            "what": "same prefill with y stored in bf16 (RNE of the fp32 y; 671 MB less written), "
                    "back-to-back calls; context only, value is the fp32-y default"},
        "tflops_contraction_kernels": round(contraction_tf, 2),
        "frac_bf16_peak_contraction_kernels": round(contraction_tf / BF16_PEAK_TFLOPS, 4),
        "prefill_path": fused if isinstance(fused, str) else ("state_walk" if fused else "chunk_parallel"),
        "roofline": roof,
        "roofline_kernels": roofs,
        "roofline_decode": roof_dec,
        "copy_reference": {"bytes": 2 * state.numel() * 4, "ms": round(copy_ms, 4), "gbps": round(copy_gbs, 1),
                           "frac_of_hbm_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
                           "what": "torch device-to-device copy of a buffer the size of the decode state"},
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(wall, 3),
        "distribution_ms": {"prefill": _pct(pre_ms), "decode": _pct(dec_ms),
                            "what": "p10 / median / p90 over the timed steps (HIP events per call)"},
        "environment": env,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
