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


def chunk_scan_work(wl, cps, es=2):
    """Algorithmic FLOPs and HBM bytes of one chunk_scan launch (dense batch)."""
    Q, H, P, N, G, b, L = wl.chunk, wl.H, wl.P, wl.N, wl.G, wl.batch, wl.seqlen
    cpseq = -(-L // Q)
    spseq = -(-cpseq // cps)
    updates = 0
    for s in range(spseq):
        n = min(cps, cpseq - s * cps)
        updates += n if s == spseq - 1 else n - 1
    nch = b * cpseq
    flops = nch * H * (2 * Q * N * P + 2 * Q * Q * P) + b * updates * H * 2 * Q * N * P
    nti = Q // 32
    T = b * L
    bytes_ = (2 * T * H * P * es + T * G * N * es + nch * G * nti * (nti + 1) // 2 * 1024 * 4
              + nch * G * N * Q * es + 2 * nch * H * Q * 4 + b * spseq * H * P * N * 4
              + b * H * P * N * 4)
    return flops, bytes_


def decode_bytes(wd, es=2):
    b, H, P, N, G = wd.nseq, wd.H, wd.P, wd.N, wd.G
    return 2 * b * H * P * N * 4 + 2 * b * H * P * es + 2 * b * G * N * es + b * H * 4 + 2 * H * 4


def cpu_baseline(inp, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the prefill workload: one
    sequence, a few heads, all of its tokens; scaled to full-layer tokens/s."""
    import oracle
    wl = inp.wl
    cores = len(os.sched_getaffinity(0))
    threads = oracle.threads()
    heads = max(1, min(wl.H, 2 * threads))
    sl = np.arange(heads)
    x = inp.x[:1, :, sl]
    dt = inp.dt[:1, :, sl]
    B = inp.B[:1]
    C = inp.C[:1]
    init = None if inp.init is None else inp.init[:1, sl]
    t0 = time.perf_counter()
    oracle.scan(x, dt, inp.A[sl], B, C, inp.D[sl], init=init)
    t = time.perf_counter() - t0
    # grow the sample toward the budget if the first pass was short
    if t < budget_s / 4 and heads < wl.H:
        heads = int(min(wl.H, max(heads + 1, heads * budget_s / 2 / max(t, 1e-3))))
        sl = np.arange(heads)
        x = inp.x[:1, :, sl]
        dt = inp.dt[:1, :, sl]
        init = None if inp.init is None else inp.init[:1, sl]
        t0 = time.perf_counter()
        oracle.scan(x, dt, inp.A[sl], B, C, inp.D[sl], init=init)
        t = time.perf_counter() - t0
    tokens_equiv = wl.seqlen * heads / wl.H
    return {"value": tokens_equiv / t, "unit": "tokens/s", "cores": int(threads),
            "host_cpus": int(cores), "kind": "oracle", "seconds": t,
            "sample": "fp64 sequential oracle (C, OpenMP over (sequence, head)) on 1 of %d "
                      "sequences x %d of %d heads x %d tokens of the prefill workload; value = "
                      "full-layer tokens/s (tokens x heads/H / time)" % (wl.batch, heads, wl.H,
                                                                         wl.seqlen)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunks-per-segment", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the scan shards "
              "over independent (sequence, head) pairs with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import mamba_ssd_chunked_02_amd as ssd
    from mamba_ssd_chunked_02_amd import workloads as W

    dev = torch.device("cuda:0")
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
    nbytes = ssd.workspace_size(x, Bm, wl.chunk, chunks_per_segment=args.chunks_per_segment)
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
                         workspace=ws, chunks_per_segment=args.chunks_per_segment,
                         stage_ms=stage_ms)

    def decode():
        ssd.decode_step(state, dx, ddt, dA, dB, dC, dD, y=dy)

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        prefill([])
        decode()
    torch.cuda.synchronize()

    log("timing", args.steps, "steps")
    stream = torch.cuda.current_stream(dev)
    stages = []
    dec_ms = []
    t_wall0 = time.perf_counter()
    torch.cuda.synchronize()
    for i in range(args.steps):
        st = []
        prefill(st)                       # per-stage HIP events on the library's stream
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        decode()
        e1.record(stream)
        e1.synchronize()
        stages.append(st)
        dec_ms.append(e0.elapsed_time(e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    log("timed region %.3f s" % wall)

    stages = np.array(stages)              # [steps, 6] ms
    stage_mean = stages.mean(axis=0)
    prefill_ms = float(stages.sum(axis=1).mean())
    decode_ms = float(np.mean(dec_ms))
    tokens = wl.tokens
    value = tokens / (prefill_ms * 1e-3)
    dense_tf = prefill_flops(wl) / (prefill_ms * 1e-3) / 1e12
    causal_tf = prefill_flops(wl, causal=True) / (prefill_ms * 1e-3) / 1e12

    # chunk_scan (dominant prefill kernel) roofline
    from ctypes import c_size_t  # noqa: F401  (kept for readers of the layout)
    cps = args.chunks_per_segment or _auto_cps(wl)
    ks_flops, ks_bytes = chunk_scan_work(wl, cps)
    ks_ms = float(stage_mean[5])
    ks_tflops = ks_flops / (ks_ms * 1e-3) / 1e12
    ks_gbs = ks_bytes / (ks_ms * 1e-3) / 1e9
    frac_mfma = ks_tflops / BF16_PEAK_TFLOPS
    frac_hbm = ks_gbs / HBM_PEAK_GBS
    if frac_hbm >= frac_mfma:
        roof = {"bound": "hbm", "achieved": round(ks_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(frac_hbm, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(ks_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(frac_mfma, 4), "traffic": None}
    roof.update({"kernel": "ssd_chunk_scan_kernel<bf16,64,128>", "avg_ms": round(ks_ms, 4),
                 "algorithmic_flops": ks_flops, "algorithmic_bytes": ks_bytes,
                 "mfma_frac": round(frac_mfma, 4), "hbm_frac": round(frac_hbm, 4)})
    dbytes = decode_bytes(wd)
    dgbs = dbytes / (decode_ms * 1e-3) / 1e9
    roof_dec = {"bound": "hbm", "achieved": round(dgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dgbs / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "ssd_decode_kernel<bf16,32>", "avg_ms": round(decode_ms, 4),
                "algorithmic_bytes": dbytes}

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
                   "global_batch": wl.batch, "seq_len": wl.seqlen, "parallelism": "none (1 GPU)",
                   "chunks_per_segment": cps},
        "tflops_dense": round(dense_tf, 2),
        "tflops_causal": round(causal_tf, 2),
        "stage_ms": {k: round(float(v), 4) for k, v in zip(ssd.STAGES, stage_mean)},
        "decode": {"ms_per_step": round(decode_ms, 4), "gbps": round(dgbs, 1),
                   "frac_of_hbm_peak": round(dgbs / HBM_PEAK_GBS, 4), "bytes_per_step": dbytes},
        "step_ms_prefill_plus_decode": round(prefill_ms + decode_ms, 4),
        "roofline": roof,
        "roofline_decode": roof_dec,
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


def _auto_cps(wl):
    """The library's automatic chunks-per-segment rule for a dense batch."""
    cpseq = -(-wl.seqlen // wl.chunk)
    pairs = max(1, wl.batch * wl.H)
    want = max(1, min(-(-2048 // pairs), cpseq))
    return -(-cpseq // want)


if __name__ == "__main__":
    main()
