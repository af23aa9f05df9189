"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/ssd.h declares, and rejects bad arguments on the host before any
launch (fake, never-dereferenced device addresses are used)."""
import ctypes
import os
import re

import pytest

import mamba_ssd_chunked_02_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_CHUNK, E_WS, E_HIP, E_UNSUP, E_SEQ = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
E_VALUE = -10
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.library_path()):
        import mamba_ssd_chunked_02_amd.build as b
        b.build()
    return ssd.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:ssd_status|const char\*)\s+(ssd_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["ssd_chunked_scan", "ssd_decode_step", "ssd_chunked_scan_workspace_size",
              "ssd_status_string", "ssd_last_error_detail", "ssd_chunked_scan_dt_act",
              "ssd_decode_step_dt_act", "ssd_decode_window_step", "ssd_causal_conv1d",
              "ssd_causal_conv1d_step"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_only_the_abi_is_exported(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.library_path()], capture_output=True,
                         text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    ours = {s for s in syms if s.startswith("ssd_")}
    assert ours == set(declared_functions())


def shape(**kw):
    s = ssd._Shape()
    d = dict(batch=1, seqlen=512, nheads=4, headdim=16, dstate=16, ngroups=1, dtype=0, ydtype=0, path=0,
             reserved=0)
    d.update(kw)
    for k, v in d.items():
        setattr(s, k, v)
    return s


def ws_size(lib, sh, chunk=64):
    n = ctypes.c_size_t(0)
    st = lib.ssd_chunked_scan_workspace_size(ctypes.byref(sh), chunk, ctypes.byref(n))
    return st, n.value


def test_workspace_size_valid(lib):
    st, n = ws_size(lib, shape())
    assert st == OK and n > 0
    st2, n2 = ws_size(lib, shape(seqlen=1024))
    assert st2 == OK and n2 > n
    st3, n3 = ws_size(lib, shape(batch=8, seqlen=8192, nheads=80, headdim=64, dstate=128, dtype=1), 256)
    assert st3 == OK and n3 < 2 ** 31
    # the scan walk keeps the per-chunk states on chip: its workspace has no
    # [chunks, H, P, N] fp32 region and no per-token weight table, only a
    # [chunks, H] table of (cs_last, decay to the sequence's end) pairs
    big = dict(batch=8, seqlen=8192, nheads=80, headdim=64, dstate=128, dtype=1)
    sizes = {p: ws_size(lib, shape(path=p, **big), 256) for p in (1, 2, 3)}
    assert all(v[0] == OK for v in sizes.values())
    states = 8 * 32 * 80 * 64 * 128 * 4
    weights = 8 * 32 * 80 * 256 * 4
    tails = 8 * 32 * 80 * 2 * 4
    assert sizes[1][1] == sizes[2][1]
    assert sizes[2][1] - sizes[3][1] == states + weights - tails


@pytest.mark.parametrize("kw,chunk,code", [
    (dict(dtype=7), 64, E_DTYPE),
    (dict(ydtype=2), 64, E_DTYPE),
    (dict(reserved=1), 64, E_SHAPE),
    (dict(path=-1), 64, E_VALUE),
    (dict(path=4), 64, E_VALUE),
    # the scan walk covers bf16 inputs, 256-token chunks and dstate in (64, 128] only
    (dict(path=3), 64, E_UNSUP),
    (dict(path=3, dtype=1, dstate=128), 128, E_UNSUP),
    (dict(path=3, dtype=1, dstate=64), 256, E_UNSUP),
    (dict(path=3, dtype=0, dstate=128), 256, E_UNSUP),
    (dict(nheads=0), 64, E_SHAPE),
    (dict(nheads=6, ngroups=4), 64, E_SHAPE),
    (dict(headdim=12), 64, E_SHAPE),
    (dict(headdim=136), 64, E_SHAPE),
    (dict(dstate=264), 64, E_SHAPE),
    (dict(dstate=4), 64, E_SHAPE),
    (dict(batch=-1), 64, E_SHAPE),
    (dict(seqlen=-5), 64, E_SHAPE),
    (dict(nheads=300000, ngroups=1), 64, E_SHAPE),
    (dict(), 48, E_CHUNK),
    (dict(), 512, E_CHUNK),
])
def test_shape_errors(lib, kw, chunk, code):
    st, _ = ws_size(lib, shape(**kw), chunk)
    assert st == code
    assert lib.ssd_last_error_detail().decode()


def test_null_shape_and_out(lib):
    n = ctypes.c_size_t(0)
    assert lib.ssd_chunked_scan_workspace_size(None, 64, ctypes.byref(n)) == E_NULL
    sh = shape()
    assert lib.ssd_chunked_scan_workspace_size(ctypes.byref(sh), 64, None) == E_NULL


def test_cu_seqlens_host_validation(lib):
    cu_dev = FAKE
    for cu, code in [([0, 5, 3, 9], E_SEQ), ([1, 5, 9, 9], E_SEQ), ([0, 5, 7, 8], E_SEQ),
                     ([0, 5, 7, 9], OK)]:
        arr = (ctypes.c_int32 * 4)(*cu)
        sh = shape(batch=3, seqlen=9)
        sh.cu_seqlens = cu_dev
        sh.cu_seqlens_host = ctypes.addressof(arr)
        st, _ = ws_size(lib, sh)
        assert st == code, cu


def scan(lib, sh, chunk=64, ws_bytes=None, **ptrs):
    p = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=FAKE, init=None, y=FAKE + 4096,
             final=None, ws=FAKE + 8192)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = ws_size(lib, sh, chunk)[1]
    return lib.ssd_chunked_scan(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], chunk, p["init"],
                                p["y"], p["final"], ctypes.byref(sh), p["ws"], ws_bytes, None)


def test_scan_pointer_errors(lib):
    sh = shape()
    for name in ["x", "dt", "A", "B", "C", "D", "y"]:
        assert scan(lib, sh, **{name: None}) == E_NULL, name
    assert scan(lib, sh, ws=None) == E_WS
    for name in ["x", "B", "C", "y", "init", "final", "ws"]:
        assert scan(lib, sh, **{name: FAKE + 8}) == E_ALIGN, name
    # dt, A and D are read one fp32 element at a time: 4-byte alignment suffices
    for name in ["dt", "A", "D"]:
        assert scan(lib, sh, **{name: FAKE + 2}) == E_ALIGN, name
        assert scan(lib, sh, ws_bytes=1, **{name: FAKE + 4}) == E_WS, name
    n = ws_size(lib, sh)[1]
    assert scan(lib, sh, ws_bytes=n - 1) == E_WS
    assert scan(lib, sh, y=FAKE) == E_SHAPE  # y aliases x


def test_decode_errors(lib):
    sh = shape(batch=2)

    def dec(**kw):
        p = dict(state=FAKE, x=FAKE + 16, dt=FAKE + 32, A=FAKE + 48, B=FAKE + 64, C=FAKE + 80,
                 D=FAKE + 96, y=FAKE + 112)
        p.update(kw)
        return lib.ssd_decode_step(p["state"], p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"],
                                   p["y"], ctypes.byref(kw.get("sh", sh)), None)

    for name in ["state", "x", "dt", "A", "B", "C", "D", "y"]:
        assert dec(**{name: None}) == E_NULL
    for name in ["state", "x", "B", "C", "y"]:
        assert dec(**{name: FAKE + 8}) == E_ALIGN
    # per-step slices of a [steps, batch, H] dt buffer sit at multiples of
    # 4 * batch * H bytes: dt, A and D need only 4-byte alignment
    for name in ["dt", "A", "D"]:
        assert dec(**{name: FAKE + 2}) == E_ALIGN
        assert dec(y=FAKE + 16, **{name: FAKE + 4 + {"dt": 32, "A": 48, "D": 96}[name]}) == E_SHAPE
    assert dec(y=FAKE + 16) == E_SHAPE
    bad = shape(batch=2, ngroups=3)
    assert lib.ssd_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16,
                               ctypes.byref(bad), None) == E_SHAPE
    assert lib.ssd_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == E_NULL
    # more (sequence, head) blocks than one launch grid holds
    assert dec(sh=shape(batch=1 << 30, nheads=8, headdim=8)) == E_SHAPE
    assert "launch grid" in lib.ssd_last_error_detail().decode()


def test_status_strings(lib):
    for code in [OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_CHUNK, E_WS, E_HIP, E_UNSUP, E_SEQ, E_VALUE]:
        s = lib.ssd_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.ssd_status_string(123).decode() == "unknown status"


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ssd, "_lib", None)
    monkeypatch.setattr(ssd, "_PKG", str(tmp_path))
    with pytest.raises(RuntimeError, match="not built"):
        ssd.load()


def test_dt_activation_argument_errors(lib):
    """The *_dt_act entry points validate the activation first: NULL act, a
    misaligned bias, and clamp ranges that are negative, NaN, infinite at the
    bottom or inverted; then the usual argument checks apply."""
    sh = shape(batch=2)
    inf, nan = float("inf"), float("nan")

    def act(bias=None, lo=0.0, hi=inf):
        a = ssd._DtAct()
        a.dt_bias, a.dt_min, a.dt_max = bias, lo, hi
        return a

    def scan_act(a, s=sh):
        return lib.ssd_chunked_scan_dt_act(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, None, FAKE + 4096, None,
                                           None if a is None else ctypes.byref(a), ctypes.byref(s),
                                           FAKE + 8192, 1, None)

    def dec_act(a, s=sh):
        return lib.ssd_decode_step_dt_act(FAKE, FAKE + 16, FAKE + 32, FAKE + 48, FAKE + 64, FAKE + 80,
                                          FAKE + 96, FAKE + 112, None if a is None else ctypes.byref(a),
                                          ctypes.byref(s), None)

    for call in (scan_act, dec_act):
        assert call(None) == E_NULL
        assert call(act(bias=FAKE + 2)) == E_ALIGN
        for lo, hi in [(-0.1, 1.0), (nan, 1.0), (0.0, nan), (inf, inf), (0.5, 0.1)]:
            assert call(act(lo=lo, hi=hi)) == E_VALUE, (lo, hi)
            assert lib.ssd_last_error_detail().decode()
        # a valid activation reaches the usual checks (a bad dtype here)
        assert call(act(lo=0.001, hi=0.1), shape(batch=2, dtype=7)) == E_DTYPE
    assert scan_act(act()) == E_WS  # workspace_bytes 1 is too small


def test_window_step_errors(lib):
    sh = shape(batch=2)

    def win(window=16, t=0, flush=0, act=None, **kw):
        p = dict(state=FAKE, x=FAKE + 16, dt=FAKE + 32, A=FAKE + 48, B=FAKE + 64, C=FAKE + 80,
                 D=FAKE + 96, y=FAKE + 112)
        p.update(kw)
        return lib.ssd_decode_window_step(p["state"], p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"],
                                          p["y"], window, t, flush, act, ctypes.byref(sh), None)

    for window, t, flush in [(0, 0, 0), (17, 0, 0), (16, 16, 0), (4, -1, 0), (4, 0, 2)]:
        assert win(window, t, flush) == E_VALUE, (window, t, flush)
    for name in ["state", "x", "dt", "A", "B", "C", "D", "y"]:
        assert win(**{name: None}) == E_NULL, name
        assert win(**{name: FAKE + (2 if name in ("dt", "A", "D") else 8)}) == E_ALIGN, name
    assert win(y=FAKE + 16) == E_SHAPE  # y aliases x
    a = ssd._DtAct()
    a.dt_bias, a.dt_min, a.dt_max = None, -1.0, 1.0
    assert win(act=ctypes.byref(a)) == E_VALUE


def conv_shape(**kw):
    s = ssd._ConvShape()
    d = dict(batch=2, seqlen=100, channels=64, width=4, dtype=1, ydtype=1, activation=1, reserved=0)
    d.update(kw)
    for k, v in d.items():
        setattr(s, k, v)
    return s


def conv_outs(parts=(64,), base=FAKE + 4096):
    o = ssd._ConvOutputs()
    o.nparts = len(parts)
    for i, c in enumerate(parts):
        o.channels[i] = c
        o.out[i] = base + 1024 * i
    return o


def test_conv1d_argument_errors(lib):
    X, Wt, Bs, S0, S1 = FAKE, FAKE + 16, FAKE + 32, FAKE + 48, FAKE + 64

    def conv(x=X, w=Wt, b=Bs, s0=S0, s1=S1, out=None, sh=None):
        out = conv_outs() if out is None else out
        sh = conv_shape() if sh is None else sh
        return lib.ssd_causal_conv1d(x, w, b, s0, s1, ctypes.byref(out), ctypes.byref(sh), None)

    def step(state=S0, x=X, w=Wt, b=Bs, out=None, sh=None):
        out = conv_outs() if out is None else out
        sh = conv_shape() if sh is None else sh
        return lib.ssd_causal_conv1d_step(state, x, w, b, ctypes.byref(out), ctypes.byref(sh), None)

    assert lib.ssd_causal_conv1d(X, Wt, Bs, S0, S1, None, ctypes.byref(conv_shape()), None) == E_NULL
    assert lib.ssd_causal_conv1d(X, Wt, Bs, S0, S1, ctypes.byref(conv_outs()), None, None) == E_NULL
    for f in (conv, step):
        assert f(sh=conv_shape(dtype=2)) == E_DTYPE
        assert f(sh=conv_shape(ydtype=-1)) == E_DTYPE
        assert f(sh=conv_shape(activation=2)) == E_VALUE
        assert f(sh=conv_shape(reserved=1)) == E_SHAPE
        for c in (0, 4, 12, 2 ** 20 + 8):
            assert f(sh=conv_shape(channels=c), out=conv_outs((max(c, 8),))) == E_SHAPE, c
        for k in (0, 1, 5):
            assert f(sh=conv_shape(width=k)) == E_SHAPE, k
        assert f(sh=conv_shape(batch=-1)) == E_SHAPE
        # output parts: count, sizes, sum, unused entries, NULL, alignment, aliasing
        o = conv_outs(); o.nparts = 0
        assert f(out=o) == E_SHAPE
        assert f(out=conv_outs((32, 24))) == E_SHAPE      # sums to 56, not 64
        assert f(out=conv_outs((60, 4))) == E_SHAPE       # not multiples of 8
        o = conv_outs((64,)); o.channels[1] = 8
        assert f(out=o) == E_SHAPE
        o = conv_outs((32, 32)); o.out[1] = None
        assert f(out=o) == E_NULL
        o = conv_outs((32, 32)); o.out[1] = FAKE + 4104
        assert f(out=o) == E_ALIGN
        o = conv_outs((64,)); o.out[0] = X
        assert f(out=o) == E_SHAPE
        assert f(w=None) == E_NULL
        assert f(x=None) == E_NULL
        assert f(x=X + 8) == E_ALIGN
        assert f(w=Wt + 4) == E_ALIGN
        assert f(b=Bs + 4) == E_ALIGN
    # prefill-only checks: seqlen, packed offsets, state alignment and aliasing
    assert conv(sh=conv_shape(seqlen=-1)) == E_SHAPE
    assert conv(s0=S0 + 8) == E_ALIGN
    assert conv(s1=S1 + 8) == E_ALIGN
    assert conv(s1=X) == E_SHAPE
    o = conv_outs((64,)); o.out[0] = S1
    assert conv(out=o) == E_SHAPE
    sh = conv_shape(batch=3, seqlen=10)
    host = (ctypes.c_int32 * 4)(0, 4, 3, 10)
    sh.cu_seqlens = FAKE + 256
    sh.cu_seqlens_host = ctypes.addressof(host)
    assert conv(sh=sh) == E_SEQ
    host2 = (ctypes.c_int32 * 4)(0, 4, 6, 9)
    sh.cu_seqlens_host = ctypes.addressof(host2)
    assert conv(sh=sh) == E_SEQ
    sh = conv_shape(batch=0, seqlen=10)
    sh.cu_seqlens = FAKE + 256
    assert conv(sh=sh) == E_SHAPE
    sh = conv_shape()
    sh.cu_seqlens_host = ctypes.addressof(host2)
    assert conv(sh=sh) == E_SHAPE
    # step-only checks: the state pointer
    assert step(state=None) == E_NULL
    assert step(state=S0 + 8) == E_ALIGN
    assert step(state=X) == E_SHAPE
    o = conv_outs((64,)); o.out[0] = S0
    assert step(out=o) == E_SHAPE


def test_noalloc_rejects_before_any_device_call(lib):
    """ssd_chunked_scan_noalloc validates the shape, then the workspace size
    against the static array, before it touches the device."""
    assert lib.ssd_chunked_scan_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, None, FAKE + 4096, None,
                                        ctypes.byref(shape(dtype=7)), None) == E_DTYPE
    big = shape(batch=8, seqlen=8192, nheads=80, headdim=64, dstate=128, dtype=1)
    assert lib.ssd_chunked_scan_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, None, FAKE + 4096, None,
                                        ctypes.byref(big), None) == E_WS
    assert "static array" in lib.ssd_last_error_detail().decode()
    assert ssd.NOALLOC_SCRATCH_BYTES == 64 << 20
    import re
    m = re.search(r"#define SSD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == ssd.NOALLOC_SCRATCH_BYTES
