"""The algorithmic bytes and FLOPs behind the benchmark's roofline figures,
checked against the same quantities written out from the shapes of the
2.7B-shaped workloads (prefill b8 L8192 H80 P64 N128 G1 chunk 256 with bf16
x/B/C and fp32 y; decode b256 with fp32 state and y)."""
import importlib.util
import os

from mamba_ssd_chunked_02_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)

MB = 1e6
b, L, H, P, N, Q = 8, 8192, 80, 64, 128, 256
chunks = b * L // Q                      # 256 chunks of 256 tokens
x_bytes = b * L * H * P * 2              # bf16 x, read once
y_bytes = b * L * H * P * 4              # fp32 y, written once
state_slots = chunks * H * P * N * 4     # one fp32 state per (chunk, head)
tables = 2 * chunks * H * Q * 4          # two fp32 per-token tables per (chunk, head)


def test_workload_is_the_2p7b_prefill():
    wl = W.CONFIGS[3]
    assert (wl.batch, wl.seqlen, wl.H, wl.P, wl.N, wl.G, wl.chunk) == (b, L, H, P, N, 1, Q)


def test_chunk_state_walk_bytes_and_flops():
    ks = bench.kernel_work(W.CONFIGS[3])["chunk_state"]
    bt = chunks * N * Q * 2              # B^T of every chunk, bf16
    init_final = 2 * b * H * P * N * 4
    assert ks["bytes"] == x_bytes + bt + state_slots + tables + init_final == 1_442_840_576
    assert ks["flops"] == chunks * H * 2 * Q * N * P == 85_899_345_920


def test_chunk_scan_bytes_and_flops():
    kc = bench.kernel_work(W.CONFIGS[3])["chunk_scan"]
    c_rows = b * L * N * 2
    cb_causal = chunks * (8 * 9 // 2) * 32 * 32 * 2   # 36 causal 32x32 tiles per chunk, bf16
    assert kc["bytes"] == x_bytes + y_bytes + c_rows + state_slots + cb_causal + tables
    assert abs(kc["bytes"] / MB - 2761.9) < 0.05
    assert kc["flops"] == chunks * H * (2 * Q * N * P + 2 * Q * Q * P) == 257_698_037_760


def test_decode_step_bytes():
    wd = W.CONFIGS[2]
    nb = 256
    state = nb * H * P * N * 4
    assert state == 671_088_640
    expect = 2 * state + nb * H * P * 2 + nb * H * P * 4 + 2 * nb * N * 2 + nb * H * 4 + 2 * H * 4
    assert bench.decode_bytes(wd) == expect == 1_350_255_232


def test_scan_walk_bytes_and_flops():
    """The fused walk: x and y once, C rows, B^T, the causal C.B^T tiles, the
    decay sums and steps, the initial and final states; no per-chunk state."""
    kw = bench.kernel_work(W.CONFIGS[3], fused="scan_walk")["scan_walk"]
    bt = chunks * N * Q * 2
    c_rows = b * L * N * 2
    cb_causal = chunks * (8 * 9 // 2) * 32 * 32 * 2
    init_final = 2 * b * H * P * N * 4
    assert kw["bytes"] == x_bytes + y_bytes + c_rows + bt + cb_causal + tables + init_final
    assert abs(kw["bytes"] / MB - 2149.6) < 0.1
    assert kw["flops"] == 85_899_345_920 + 257_698_037_760
    causal_pairs = Q * (Q + 1) // 2
    assert kw["flops_causal"] == chunks * H * (2 * Q * N * P + 2 * Q * N * P + 2 * causal_pairs * P)


def test_roofline_bound_follows_arithmetic_intensity():
    """The roof is chosen by flops per byte against the ridge (bf16 peak / HBM
    peak), not by whichever fraction is larger."""
    kw = bench.kernel_work(W.CONFIGS[3], fused="scan_walk")["scan_walk"]
    r = bench.roofline_of(kw, 0.8, "k")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["flop_per_byte"] < r["ridge_flop_per_byte"] == 312.5
    dense = {"flops": 10 ** 15, "flops_causal": 10 ** 15, "bytes": 10 ** 9}
    assert bench.roofline_of(dense, 1.0, "k")["bound"] == "mfma"


def test_traffic_summary_is_read_only_while_its_sources_match(tmp_path):
    """A counter summary scales FETCH_SIZE / WRITE_SIZE (KiB) by the copy
    calibration factors, and is ignored once the kernel sources it describes
    have changed (a different digest)."""
    good = bench._source_digest(bench.DECODE_SOURCES)
    body = "kernel: k\nfetch_kib: 1000.0\nwrite_kib: 2000.0\ncopy_fetch_factor: 2.000\ncopy_write_factor: 1.000\n"
    f = tmp_path / "t.txt"
    f.write_text(body + "source_digest: %s\n" % good)
    t = bench._traffic(str(f), "k", 6 * 1024 * 1000, bench.DECODE_SOURCES)
    assert t["fetch_bytes"] == 2 * 1000 * 1024 and t["write_bytes"] == 2000 * 1024
    assert t["over_algorithmic"] == round(4000 * 1024 / (6 * 1024 * 1000), 3)
    f.write_text(body + "source_digest: 0000000000000000\n")
    assert bench._traffic(str(f), "k", 1, bench.DECODE_SOURCES) is None
    assert bench._source_digest(bench.DECODE_SOURCES) != bench._source_digest(bench.PREFILL_SOURCES)
