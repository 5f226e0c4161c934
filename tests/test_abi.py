"""The C ABI without a GPU: the library loads, exports what the header declares,
plans and sizes workspaces, and rejects bad arguments before touching a device.

Pointers passed here are fake addresses; every call is one that validation
rejects, so nothing is ever dereferenced or launched.
"""
import ctypes
import os
import re

import pytest

from selective_state_space_39_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

OK, E_NULL, E_SHAPE, E_N, E_DTYPE, E_ALIGN, E_WS, E_ALIAS = 0, -1, -2, -3, -4, -5, -6, -7


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = binding.lib()
    names = declared_functions()
    assert {"ssm_scan_fwd", "ssm_state_update", "ssm_abi_version", "ssm_last_error",
            "ssm_scan_fwd_workspace_bytes", "ssm_scan_fwd_plan"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in ssm_scan.h but not exported"


def test_abi_version_matches_header():
    m = re.search(r"#define\s+SSM_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert binding.abi_version() == int(m.group(1)) == binding.ABI_VERSION


def test_plan_and_workspace():
    L = binding.lib()
    # single chunk: no workspace
    assert binding.plan(1, 64, 16384, 1, 0) == (64, 1)
    assert L.ssm_scan_fwd_workspace_bytes(1, 64, 16384, 16, 1, 0) == 0
    # explicit chunks: (n-1) carries of D * (1 + 16) floats, S part padded to 256 bytes
    cl, nc = binding.plan(2, 300, 200, 1, 64)
    assert (cl, nc) == (64, 5)
    carries = 2 * 4 * 200
    assert binding.workspace_bytes(2, 300, 200, 1, 64) == (carries * 4 + 255) // 256 * 256 + carries * 16 * 4
    # automatic plan for the named workloads: whole number of chunks, aligned length
    for (b, l, d) in [(8, 2048, 1536), (4, 2048, 5120), (1, 131072, 2048), (1, 256, 16)]:
        cl, nc = binding.plan(b, l, d, 1, 0)
        assert cl % 32 == 0 and nc == -(-l // cl) and nc >= 1


def test_plan_choices_for_the_measured_shapes():
    """The cost model picks what a chunk-length sweep on the GPU measured fastest
    (130M layer: 64 vs 32/96/128; 2.8B layer: 64 vs 96/128/192/256; 128k: 256 vs
    512/1024; 1 x 2048 x 768: 32 vs 64/128), and the backward plan keeps
    64-token chunks on the 130M layer."""
    assert binding.plan(8, 2048, 1536, 1, 0) == (64, 32)
    assert binding.plan(4, 2048, 5120, 1, 0) == (64, 32)
    assert binding.plan(1, 131072, 2048, 1, 0) == (256, 512)
    assert binding.bwd_plan(8, 2048, 1536, 1, 0) == (64, 32)
    # few channels (12 wavefronts per chunk): many short chunks; measured 36 us at 32 vs 50 us at 64
    assert binding.plan(1, 2048, 768, 1, 0) == (32, 64)


def test_chunk_bytes_limit():
    """A chunk's rows are addressed with 32-bit offsets: at most 2 GiB per chunk (4 bytes per element)."""
    L = binding.lib()
    # explicit chunk: 4096 tokens x 2^22 channels x 4 B = 64 GiB -> rejected, forward and backward
    assert L.ssm_scan_fwd_workspace_bytes(1, 4096, 1 << 22, 16, 1, 4096) == E_SHAPE
    assert L.ssm_scan_bwd_workspace_bytes(1, 4096, 1 << 22, 16, 1, 4096) == E_SHAPE
    # automatic plan: capped at (2^31 - 1) / (2^22 * 4) rounded down to 32 = 96 tokens
    cl, nc = binding.plan(1, 1024, 1 << 22, 1, 0)
    assert cl <= 96 and cl % 32 == 0 and nc == -(-1024 // cl)
    cl, nc = binding.bwd_plan(1, 1024, 1 << 22, 1, 0)
    assert cl <= 96 and cl % 32 == 0
    # not even 32 tokens fit
    assert L.ssm_scan_fwd_workspace_bytes(1, 64, 1 << 26, 16, 1, 0) == E_SHAPE


@pytest.mark.parametrize("args,code", [
    ((1, 10, 8, 8, 1, 0), E_N),
    ((1, 10, 8, 16, 7, 0), E_DTYPE),
    ((0, 10, 8, 16, 1, 0), E_SHAPE),
    ((1, 0, 8, 16, 1, 0), E_SHAPE),
    ((1, 10, 0, 16, 1, 0), E_SHAPE),
    ((1, 10, 8, 16, 1, 48), E_SHAPE),          # chunk_len not a multiple of 32
    ((1, 10, 8, 16, 1, -32), E_SHAPE),
    ((70000, 10, 8, 16, 1, 0), E_SHAPE),       # batch beyond the grid limit
    ((1, 1 << 40, 1 << 20, 16, 1, 0), E_SHAPE),  # overflow
])
def test_shape_errors(args, code):
    L = binding.lib()
    assert L.ssm_scan_fwd_workspace_bytes(*args) == code
    assert L.ssm_last_error().decode()


class Fake:
    """Distinct, well aligned fake device addresses for every argument."""

    def __init__(self, batch=2, L=64, D=128, io=1):
        es = 2 if io == 1 else 4
        self.sizes = dict(x=batch * L * D * es, delta=batch * L * D * es, z=batch * L * D * es,
                          B=batch * L * 16 * es, C=batch * L * 16 * es, A=D * 64, Dskip=D * 4, dt_bias=D * 4,
                          h0=batch * D * 64, y=batch * L * D * es, h_last=batch * D * 64, ws=1 << 20)
        addr = 1 << 40
        self.p = {}
        for k, n in self.sizes.items():
            self.p[k] = addr
            addr += (n + 4095) // 4096 * 4096 + 4096
        self.batch, self.L, self.D, self.io = batch, L, D, io

    def call(self, chunk_len=32, ws_bytes=1 << 20, **over):
        p = dict(self.p)
        p.update(over)
        v = lambda k: ctypes.c_void_p(p[k]) if p[k] is not None else None
        return binding.lib().ssm_scan_fwd(v("x"), v("delta"), v("z"), v("B"), v("C"), v("A"), v("Dskip"),
                                          v("dt_bias"), v("h0"), v("y"), v("h_last"), self.batch, self.L,
                                          self.D, 16, self.io, chunk_len, v("ws"), ws_bytes, None)


@pytest.mark.parametrize("name", ["x", "delta", "B", "C", "A", "Dskip", "dt_bias", "y"])
def test_null_required(name):
    f = Fake()
    assert f.call(**{name: None}) == E_NULL
    assert name in binding.lib().ssm_last_error().decode()


def test_workspace_errors():
    f = Fake()
    assert f.call(ws=None) == E_WS
    assert f.call(ws_bytes=10) == E_WS


@pytest.mark.parametrize("name,off", [("x", 1), ("y", 1), ("B", 8), ("C", 2), ("A", 2), ("h0", 2),
                                      ("h_last", 1), ("ws", 8)])
def test_alignment(name, off):
    f = Fake()
    assert f.call(**{name: f.p[name] + off}) == E_ALIGN


@pytest.mark.parametrize("out,inp", [("y", "x"), ("y", "delta"), ("y", "z"), ("y", "B"), ("h_last", "h0"),
                                     ("h_last", "A"), ("y", "ws"), ("h_last", "y")])
def test_alias(out, inp):
    f = Fake()
    assert f.call(**{out: f.p[inp]}) == E_ALIAS


def test_state_update_validation():
    L = binding.lib()
    v = ctypes.c_void_p
    base = 1 << 40
    ptrs = [v(base + i * (1 << 24)) for i in range(10)]
    # N != 16
    assert L.ssm_state_update(*ptrs, 4, 128, 8, 1, None) == E_N
    # NULL state
    assert L.ssm_state_update(None, *ptrs[1:], 4, 128, 16, 1, None) == E_NULL
    # misaligned state (needs 16 bytes)
    bad = list(ptrs)
    bad[0] = v(base + 4)
    assert L.ssm_state_update(*bad, 4, 128, 16, 1, None) == E_ALIGN
    # y on top of h
    bad = list(ptrs)
    bad[9] = ptrs[0]
    assert L.ssm_state_update(*bad, 4, 128, 16, 1, None) == E_ALIAS
    assert L.ssm_state_update(*ptrs, 4, 128, 16, 9, None) == E_DTYPE


def test_binding_rejects_bad_tensors_on_cpu():
    import torch
    x = torch.zeros(1, 4, 8, dtype=torch.float16)
    with pytest.raises(TypeError):
        binding.scan_fwd(x, x, torch.zeros(8, 16), x, x, torch.zeros(8), torch.zeros(8))


# ---------------------------------------------------------------------------
# backward entry points
# ---------------------------------------------------------------------------

def _part(floats):
    return (floats * 4 + 255) // 256 * 256


def test_bwd_plan_and_workspace():
    # (batch, L, D) = (2, 300, 200), 64-token chunks: 5 chunks, 4 carries per row
    assert binding.bwd_plan(2, 300, 200, 1, 64) == (64, 5)
    carries = 2 * 4 * 200
    expect = (2 * (_part(carries) + _part(carries * 16))     # state and adjoint carries
              + _part(2 * 5 * (64 // 4) * 17 * 200)          # sub-chunk checkpoints (16 states + step sum)
              + _part(2 * 300 * 4 * 32)                      # per-wavefront dB | dC sums
              + _part(2 * 5 * 18 * 200))                     # per-chunk parameter sums
    assert binding.bwd_workspace_bytes(2, 300, 200, 1, 64) == expect
    # one chunk: no carries, still checkpoints and partial sums
    cl, nc = binding.bwd_plan(1, 40, 16, 0, 64)
    assert (cl, nc) == (64, 1)
    assert binding.bwd_workspace_bytes(1, 40, 16, 0, 64) == (_part(64 // 4 * 17 * 16) + _part(40 * 1 * 32)
                                                              + _part(18 * 16))
    for (b, l, d) in [(8, 2048, 1536), (4, 2048, 5120), (1, 131072, 2048), (1, 256, 16)]:
        cl, nc = binding.bwd_plan(b, l, d, 1, 0)
        assert cl % 32 == 0 and nc == -(-l // cl) and nc >= 1
    L = binding.lib()
    assert L.ssm_scan_bwd_workspace_bytes(1, 10, 8, 16, 1, 48) == E_SHAPE
    assert L.ssm_scan_bwd_workspace_bytes(1, 10, 8, 8, 1, 0) == E_N


@pytest.mark.parametrize("inp", ["x", "delta", "z", "B", "C", "A", "Dskip", "dt_bias", "h0"])
def test_workspace_on_an_input(inp):
    """The carry pass writes the workspace while other workgroups still read the inputs."""
    f = Fake()
    assert f.call(ws=f.p[inp]) == E_ALIAS
    assert "workspace overlaps " + inp in binding.lib().ssm_last_error().decode()
    # a workspace that starts inside the input and runs past its end overlaps it too
    assert f.call(ws=f.p[inp] + (f.sizes[inp] - 16) // 16 * 16) == E_ALIAS


def test_workspace_overlap_needs_a_workspace():
    """A one-chunk plan needs no workspace: an unused pointer on top of an input is not an error."""
    f = Fake(L=32)
    assert f.call(chunk_len=32, ws=f.p["x"], ws_bytes=0) not in (E_ALIAS, E_WS)


def _noalloc(f, chunk_len=32, **over):
    p = dict(f.p)
    p.update(over)
    v = lambda k: ctypes.c_void_p(p[k]) if p[k] is not None else None
    return binding.lib().ssm_scan_fwd_noalloc(v("x"), v("delta"), v("z"), v("B"), v("C"), v("A"), v("Dskip"),
                                              v("dt_bias"), v("h0"), v("y"), v("h_last"), f.batch, f.L, f.D, 16,
                                              f.io, chunk_len, None)


def test_noalloc_validation():
    """ssm_scan_fwd_noalloc validates like ssm_scan_fwd, and refuses plans whose carries exceed its scratch."""
    f = Fake()
    assert _noalloc(f, x=None) == E_NULL
    assert _noalloc(f, y=f.p["x"]) == E_ALIAS
    assert _noalloc(f, B=f.p["B"] + 8) == E_ALIGN
    assert _noalloc(f, chunk_len=40) == E_SHAPE
    # 2 x 64 x 128 in 32-token chunks needs a few KB: valid, so only the missing device stops it here
    assert _noalloc(f) == -8
    # 1 x 65536 x 2048 in 64-token chunks: 1023 chunk carries of 2048 channels x 17 floats = 142 MB > 64 MiB
    assert _noalloc(Fake(1, 65536, 2048), chunk_len=64) == E_WS
    assert "scratch" in binding.lib().ssm_last_error().decode()
    # the automatic plan picks chunks whose carries fit (the workspace plan of this shape needs 68 MiB)
    assert binding.workspace_bytes(1, 131072, 2048, 1, 0) > 64 << 20
    assert _noalloc(Fake(1, 131072, 2048), chunk_len=0) == -8
    # no plan fits: 2^20 channels cap a chunk at 480 tokens, and 2184 carries of 2^20 channels are far too many
    assert _noalloc(Fake(1, 1 << 20, 1 << 20), chunk_len=0) == E_WS


BWD_ARGS = ["x", "delta", "z", "B", "C", "A", "Dskip", "dt_bias", "h0", "dout", "dh_last",
            "dx", "ddelta", "dz", "dB", "dC", "dA", "dDskip", "ddt_bias", "dh0"]


class FakeBwd:
    def __init__(self, batch=2, L=64, D=128, io=1):
        es = 2 if io == 1 else 4
        seq, bc, st = batch * L * D * es, batch * L * 16 * es, batch * D * 64
        self.sizes = dict(x=seq, delta=seq, z=seq, B=bc, C=bc, A=D * 64, Dskip=D * 4, dt_bias=D * 4, h0=st,
                          dout=seq, dh_last=st, dx=seq, ddelta=seq, dz=seq, dB=batch * L * 64,
                          dC=batch * L * 64, dA=D * 64, dDskip=D * 4, ddt_bias=D * 4, dh0=st, ws=64 << 20)
        addr = 1 << 40
        self.p = {}
        for k, n in self.sizes.items():
            self.p[k] = addr
            addr += (n + 4095) // 4096 * 4096 + 4096
        self.batch, self.L, self.D, self.io = batch, L, D, io

    def call(self, chunk_len=32, ws_bytes=64 << 20, **over):
        p = dict(self.p)
        p.update(over)
        v = lambda k: ctypes.c_void_p(p[k]) if p[k] is not None else None
        return binding.lib().ssm_scan_bwd(*[v(k) for k in BWD_ARGS], self.batch, self.L, self.D, 16, self.io,
                                          chunk_len, v("ws"), ws_bytes, None)


@pytest.mark.parametrize("name", ["x", "delta", "B", "C", "A", "Dskip", "dt_bias", "dout", "dx", "ddelta",
                                  "dB", "dC", "dA", "dDskip", "ddt_bias"])
def test_bwd_null_required(name):
    assert FakeBwd().call(**{name: None}) == E_NULL
    assert name in binding.lib().ssm_last_error().decode()


def test_bwd_gate_pairing_and_workspace():
    f = FakeBwd()
    assert f.call(dz=None) == E_NULL          # gated scan needs dz
    assert f.call(z=None) == E_NULL           # dz without z
    assert f.call(ws=None) == E_WS
    assert f.call(ws_bytes=100) == E_WS
    assert f.call(chunk_len=40) == E_SHAPE


@pytest.mark.parametrize("name,off", [("dout", 1), ("dx", 1), ("dz", 1), ("dB", 2), ("dA", 2), ("dh0", 2),
                                      ("dh_last", 1), ("ws", 128)])
def test_bwd_alignment(name, off):
    f = FakeBwd()
    assert f.call(**{name: f.p[name] + off}) == E_ALIGN


@pytest.mark.parametrize("out,inp", [("dx", "x"), ("ddelta", "dout"), ("dz", "z"), ("dB", "B"), ("dC", "ws"),
                                     ("dA", "A"), ("dh0", "h0"), ("dh0", "dh_last"), ("dx", "ddelta"),
                                     ("dDskip", "dA"), ("ddt_bias", "dDskip")])
def test_bwd_alias(out, inp):
    f = FakeBwd()
    assert f.call(**{out: f.p[inp]}) == E_ALIAS


@pytest.mark.parametrize("inp", ["x", "delta", "z", "B", "C", "A", "Dskip", "dt_bias", "h0", "dout", "dh_last"])
def test_bwd_workspace_on_an_input(inp):
    f = FakeBwd()
    assert f.call(ws=f.p[inp] // 256 * 256) == E_ALIAS
    assert "workspace overlaps " + inp in binding.lib().ssm_last_error().decode()


@pytest.mark.parametrize("out", ["dx", "ddelta", "dz", "dB", "dA", "dh0"])
def test_bwd_workspace_on_an_output(out):
    f = FakeBwd()
    assert f.call(ws=f.p[out] // 256 * 256) == E_ALIAS


def test_conv_scan_validation():
    f = Fake()
    v = ctypes.c_void_p
    L = binding.lib()
    p = f.p
    base = 1 << 44
    w, b, init, last = v(base), v(base + (1 << 24)), v(base + (2 << 24)), v(base + (3 << 24))

    def call(k=4, conv_w=w, conv_b=b, conv_init=init, conv_last=last, y=p["y"], x=p["x"]):
        return L.ssm_conv_scan_fwd(v(x), conv_w, conv_b, k, conv_init, v(p["delta"]), v(p["z"]), v(p["B"]),
                                   v(p["C"]), v(p["A"]), v(p["Dskip"]), v(p["dt_bias"]), v(p["h0"]), v(y),
                                   v(p["h_last"]), conv_last, f.batch, f.L, f.D, 16, f.io, 32, v(p["ws"]), 1 << 20,
                                   None)
    assert call(k=0) == E_SHAPE and call(k=5) == E_SHAPE
    assert call(conv_w=None) == E_NULL and call(conv_b=None) == E_NULL
    assert call(conv_init=v(base + (2 << 24) + 1)) == E_ALIGN
    assert call(conv_last=v(p["x"])) == E_ALIAS             # conv_last on top of xin
    assert call(conv_last=v(p["y"] + 64)) == E_ALIAS        # conv_last inside y
    # the workspace on top of the convolution's own inputs
    for q in (w, b, init):
        assert L.ssm_conv_scan_fwd(v(p["x"]), w, b, 4, init, v(p["delta"]), v(p["z"]), v(p["B"]), v(p["C"]),
                                   v(p["A"]), v(p["Dskip"]), v(p["dt_bias"]), v(p["h0"]), v(p["y"]),
                                   v(p["h_last"]), last, f.batch, f.L, f.D, 16, f.io, 32, q, 1 << 20,
                                   None) == E_ALIAS


def test_conv_decode_validation():
    L = binding.lib()
    v = ctypes.c_void_p
    base = 1 << 40
    p = [v(base + i * (1 << 24)) for i in range(13)]
    # h, conv_state, xin, conv_w, conv_b | k | delta, z, B, C, A, Dskip, dt_bias, y
    call = lambda q, k=4, N=16: L.ssm_conv_state_update(*q[:5], k, *q[5:], 4, 128, N, 1, None)
    assert call(p, k=0) == E_SHAPE and call(p, k=5) == E_SHAPE
    assert call(p, N=8) == E_N
    q = list(p); q[1] = None
    assert call(q) == E_NULL                      # conv state needed for K > 1
    q = list(p); q[1] = p[0]
    assert call(q) == E_ALIAS                     # conv state on top of h
    q = list(p); q[1] = v(base + (1 << 24) + 1)
    assert call(q) == E_ALIGN


def test_ssd_validation():
    L = binding.lib()
    v = ctypes.c_void_p
    base = 1 << 40
    p = [v(base + i * (1 << 28)) for i in range(12)]
    ws = binding.lib().ssm_ssd_fwd_workspace_bytes(2, 100, 4, 64, 128, 1)
    # x, delta, z, B, C, A, Dskip, dt_bias, h0, y, h_last | batch, L, H, P, N, io | workspace, bytes
    call = lambda q, P=64, N=128, io=1, H=4, nws=ws: L.ssm_ssd_fwd(*q[:11], 2, 100, H, P, N, io, q[11], nws, None)
    assert call(p, io=0) == E_DTYPE                 # bf16 only
    assert call(p, N=96) == E_N and call(p, N=16) == E_N
    assert call(p, P=32) == E_SHAPE
    assert call(p, H=0) == E_SHAPE
    q = list(p); q[0] = None
    assert call(q) == E_NULL
    q = list(p); q[0] = v(base + 8)
    assert call(q) == E_ALIGN                       # x must be 16-byte aligned
    q = list(p); q[9] = p[0]
    assert call(q) == E_ALIAS                       # y on top of x
    q = list(p); q[10] = p[8]
    assert call(q) == E_ALIAS                       # h_last on top of h0
    q = list(p); q[11] = None
    assert call(q) == E_WS                   # workspace missing
    assert call(p, nws=ws - 1) == E_WS       # workspace too small
    q = list(p); q[11] = p[3]
    assert call(q) == E_ALIAS                       # workspace on top of B
    q = list(p); q[11] = p[9]
    assert call(q) == E_ALIAS                       # workspace on top of y
    q = list(p); q[11] = v(base + 11 * (1 << 28) + 4)
    assert call(q) == E_ALIGN


def test_ssd_workspace_formula():
    """One 64 x 64 bf16 block of C . B per (batch row, 64-token chunk), ragged chunks rounded up."""
    f = binding.lib().ssm_ssd_fwd_workspace_bytes
    for batch, L in ((1, 1), (2, 64), (2, 65), (8, 2048), (3, 1000)):
        assert f(batch, L, 80, 64, 128, 1) == batch * -(-L // 64) * 64 * 64 * 2
        assert f(batch, L, 80, 64, 64, 1) == batch * -(-L // 64) * 64 * 64 * 2
        assert f(batch, L, 80, 64, 256, 1) == batch * -(-L // 64) * 64 * 64 * 2
    assert f(1, 100, 4, 64, 96, 1) == E_N and f(1, 100, 4, 64, 512, 1) == E_N
    assert f(1, 100, 4, 32, 128, 1) == E_SHAPE
    assert f(1, 100, 4, 64, 128, 0) == E_DTYPE
    assert f(1, 20_000_000, 1, 64, 64, 1) == E_SHAPE  # a batch row's blocks beyond 32-bit offsets


def test_last_error_is_per_thread():
    """Each thread reads the message of its own last failing call."""
    import threading
    L = binding.lib()
    out = {}

    def worker(name, args):
        for _ in range(200):
            L.ssm_scan_fwd_workspace_bytes(*args)
            out[name] = L.ssm_last_error().decode()

    t1 = threading.Thread(target=worker, args=("n", (1, 10, 8, 8, 1, 0)))       # N != 16
    t2 = threading.Thread(target=worker, args=("dtype", (1, 10, 8, 16, 7, 0)))  # bad dtype
    t1.start(); t2.start(); t1.join(); t2.join()
    assert "N = 8" in out["n"] and "dtype" in out["dtype"]


def _size_ints():
    from hypothesis import strategies as st
    return st.one_of(st.integers(-3, 300), st.integers(1, 1 << 20), st.integers(-(1 << 62), 1 << 62),
                     st.sampled_from([0, 1, 31, 32, 33, 64, 65535, 65536, 1 << 31, (1 << 31) - 1, 1 << 40]))


def _check_plan(fn, batch, L, D, dtype, chunk):
    cl, nc = ctypes.c_int64(-7), ctypes.c_int64(-7)
    rc = fn(batch, L, D, 16, dtype, chunk, ctypes.byref(cl), ctypes.byref(nc))
    return rc, cl.value, nc.value


def test_host_queries_never_misbehave():
    """Random (including negative, zero and huge) shapes through every host-only query: each call either
    succeeds with a consistent plan and workspace or returns one of the header's error codes with a message;
    a successful plan covers L with whole chunks whose rows fit 32-bit offsets."""
    from hypothesis import given, settings, strategies as st
    L = binding.lib()
    errors = {E_NULL, E_SHAPE, E_N, E_DTYPE, E_ALIGN, E_WS, E_ALIAS}

    @settings(max_examples=400, deadline=None)
    @given(batch=_size_ints(), length=_size_ints(), D=_size_ints(), N=st.sampled_from([16, 8, 0, -1, 64, 128, 256]),
           dtype=st.sampled_from([0, 1, 2, -1]), chunk=_size_ints())
    def run(batch, length, D, N, dtype, chunk):
        for ws_fn, plan_fn in ((L.ssm_scan_fwd_workspace_bytes, L.ssm_scan_fwd_plan),
                               (L.ssm_scan_bwd_workspace_bytes, L.ssm_scan_bwd_plan)):
            ws = ws_fn(batch, length, D, N, dtype, chunk)
            if ws < 0:
                assert ws in errors and L.ssm_last_error(), (batch, length, D, N, dtype, chunk, ws)
                continue
            assert N == 16 and dtype in (0, 1) and batch >= 1 and length >= 1 and D >= 1
            rc, cl, nc = _check_plan(plan_fn, batch, length, D, dtype, chunk)
            assert rc == OK, (batch, length, D, dtype, chunk, rc)
            assert cl >= 1 and nc == -(-length // cl) and (nc == 1 or cl % 32 == 0)
            assert chunk <= 0 or cl == chunk or (nc == 1 and cl >= length)
            assert nc == 1 or cl * D * 4 <= (1 << 31) - 1
            carries = (nc - 1) * batch * D * 17 * 4
            assert ws >= carries
        ws = L.ssm_ssd_fwd_workspace_bytes(batch, length, D, 64, N, dtype)
        if ws < 0:
            assert ws in errors and L.ssm_last_error()
        else:
            assert N in (64, 128, 256) and dtype == 1
            ns, sc = binding.ssd_plan(batch, length, D, N)
            gram = batch * -(-length // 64) * 64 * 64 * 2
            assert ws == gram + (batch * D * (ns - 1) * (64 * N + 1) * 4 if ns > 1 else 0)

    run()


def test_plans_of_plausible_shapes_are_consistent():
    """Shapes a caller would pass (the automatic plan or an explicit multiple of 32): the plan covers L with
    whole chunks, honours an explicit chunk length, keeps a chunk's rows within 32-bit offsets, and the
    workspace holds the (n - 1) carries of 17 floats per (batch row, channel)."""
    from hypothesis import given, settings, strategies as st
    L = binding.lib()

    @settings(max_examples=300, deadline=None)
    @given(batch=st.integers(1, 64), length=st.integers(1, 300000), D=st.integers(1, 20000),
           dtype=st.sampled_from([0, 1]), chunk=st.one_of(st.just(0), st.integers(1, 2000).map(lambda k: 32 * k)))
    def run(batch, length, D, dtype, chunk):
        for ws_fn, plan_fn in ((L.ssm_scan_fwd_workspace_bytes, L.ssm_scan_fwd_plan),
                               (L.ssm_scan_bwd_workspace_bytes, L.ssm_scan_bwd_plan)):
            ws = ws_fn(batch, length, D, 16, dtype, chunk)
            rc, cl, nc = _check_plan(plan_fn, batch, length, D, dtype, chunk)
            if chunk and chunk * D * 4 > (1 << 31) - 1:
                assert ws == E_SHAPE and rc == E_SHAPE           # an explicit chunk beyond the offset limit
                continue
            assert ws >= 0 and rc == OK, (batch, length, D, dtype, chunk, ws, rc)
            assert cl >= 1 and nc == -(-length // cl) and (nc == 1 or cl % 32 == 0)
            assert chunk == 0 or cl == chunk or (nc == 1 and cl >= length)
            assert nc == 1 or cl * D * 4 <= (1 << 31) - 1
            assert ws >= (nc - 1) * batch * D * 17 * 4
            if plan_fn is L.ssm_scan_fwd_plan:
                assert (ws == 0) == (nc == 1)

    run()


def test_ssd_segment_plan():
    """Sequences that fill the GPU are walked whole; fewer are cut into segments of whole 64-token chunks, at
    least 16 chunks each except the last, covering L exactly, with every (sequence, segment) workgroup
    resident at once (three per CU up to N = 128, two at N = 256)."""
    from hypothesis import given, settings, strategies as st

    @settings(max_examples=300, deadline=None)
    @given(batch=st.integers(1, 16), length=st.integers(1, 400000), H=st.integers(1, 128),
           N=st.sampled_from([64, 128, 256]))
    def run(batch, length, H, N):
        from hypothesis import assume
        assume(length * H * 64 * 2 <= (1 << 31) - 1)           # one batch row within 32-bit offsets
        ns, sc = binding.ssd_plan(batch, length, H, N)
        nch = -(-length // 64)
        resident = 256 * (2 if N > 128 else 3)                    # workgroups resident on 256 CUs
        assert ns >= 1 and sc >= 1 and (ns - 1) * sc < nch <= ns * sc
        if 2 * batch * H > resident or nch < 32:
            assert ns == 1
        if ns > 1:
            assert sc >= 16 and batch * H * ns <= resident
    run()
    assert binding.ssd_plan(8, 2048, 80, 128) == (1, 32)           # the 2.7B layer: walked whole
    assert binding.ssd_plan(1, 131072, 80, 128) == (9, 228)        # long context, one row: 720 workgroups
    assert binding.ssd_plan(1, 131072, 80, 256) == (6, 342)        # N = 256: two workgroups per CU
