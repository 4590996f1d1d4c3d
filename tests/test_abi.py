"""Host-side checks of the C ABI: the library loads, exports every function
include/hyena.h declares, plans lengths as documented, and rejects bad
arguments with status codes before anything touches a GPU.  Runs on CPU."""
import ctypes
import os

import pytest

import hyena_long_conv_amd as H

pytestmark = pytest.mark.skipif(not os.path.exists(H.LIB_PATH), reason="library not built")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, ALIAS = 0, 1, 2, 3, 4, 5, 6
vp = ctypes.c_void_p


def test_exports_every_header_symbol():
    names = H.header_functions()
    assert {"hyena_forward", "hyena_filter_gen", "hyena_filter_spectrum", "hyena_plan"} <= set(names)
    lib = ctypes.CDLL(H.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = H.lib()
    for code in range(8):
        assert lib.hyena_status_str(code)
    assert lib.hyena_status_str(0) == b"ok"


@pytest.mark.parametrize("L,M,path", [(1, 128, "single"), (17, 128, "single"), (32, 128, "single"),
                                      (33, 128, "single"), (65, 256, "single"), (256, 512, "single"),
                                      (1000, 2048, "single"), (2048, 4096, "single"), (8192, 16384, "single"),
                                      (16384, 32768, "single"), (16385, 36864, "fourstep"),
                                      (20000, 40960, "fourstep"), (50000, 102400, "fourstep"),
                                      (70000, 204800, "fourstep"),
                                      (65536, 131072, "fourstep"), (100000, 204800, "fourstep"),
                                      (131072, 262144, "fourstep"), (1 << 20, 1 << 21, "fourstep"),
                                      (1 << 22, 1 << 23, "fourstep")])
def test_plan_lengths(L, M, path):
    p = H.plan(L)
    assert p["M"] == M and p["path"] == path
    assert p["M"] >= 2 * L - 1
    N = M // 2
    if path == "fourstep":
        assert p["n1"] * p["n2"] == N and 64 <= p["n2"] <= 8192 and p["n2"] & (p["n2"] - 1) == 0
        # power-of-two columns, or an odd column length (FFT length 2^a 3^b 5^c)
        assert (16 <= p["n1"] <= 1024 and p["n1"] & (p["n1"] - 1) == 0
                or p["n1"] in (3, 5, 9, 15, 25, 27) or p["n1"] in (6, 10, 18, 30, 50, 54) and p["n2"] <= 2048)
        # never longer than the power of two >= 2L
        assert M <= 1 << (2 * L - 1).bit_length()
    assert p["spec_stride"] >= N + 1
    assert p["spec_stride"] % 16 == 0


def test_plan_forced_paths(monkeypatch):
    monkeypatch.setenv("HYENA_FORCE_PATH", "fourstep")
    p = H.plan(300)
    assert p["path"] == "fourstep" and p["M"] >= 600 and p["n1"] * p["n2"] == p["M"] // 2
    monkeypatch.setenv("HYENA_FOURSTEP_N1", "64")
    p = H.plan(300)
    assert p["n1"] == 64 and p["n2"] >= 64 and p["n1"] * p["n2"] == p["M"] // 2
    monkeypatch.setenv("HYENA_FOURSTEP_N1", "25")          # odd column length: FFT length 2 * 25 * 16
    p = H.plan(300)
    assert (p["n1"], p["n2"], p["M"]) == (25, 64, 3200)
    monkeypatch.setenv("HYENA_FOURSTEP_N1", "50")          # lane-pair column length 2 x 25
    p = H.plan(300)
    assert (p["n1"], p["n2"], p["M"]) == (50, 64, 6400)
    monkeypatch.setenv("HYENA_FOURSTEP_N1", "48")          # neither a power of two nor an odd column length
    with pytest.raises(H.HyenaError):
        H.plan(300)
    monkeypatch.delenv("HYENA_FOURSTEP_N1")
    monkeypatch.setenv("HYENA_FORCE_PATH", "single")
    assert H.plan(16384)["path"] == "single"
    with pytest.raises(H.HyenaError):                       # too long for one workgroup
        H.plan(16385)


def test_plan_bad_lengths():
    for L in (0, -1, (1 << 22) + 1):
        with pytest.raises(H.HyenaError) as e:
            H.plan(L)
        assert e.value.code == SHAPE
    assert H.lib().hyena_plan(16, None) == NULL


def test_size_queries():
    assert H.spectrum_bytes(768, 2, 2048) == 2 * 768 * H.plan(2048)["spec_stride"] * 8
    assert H.spectrum_workspace_bytes(768, 2, 2048) == 0
    assert H.forward_workspace_bytes(4, 768, 2, 2048) == 0
    ws = H.forward_workspace_bytes(1, 768, 2, 65536, "bf16")
    assert ws > 0 and ws % (H.plan(65536)["M"] // 2 * 8) == 0
    assert H.spectrum_bytes(0, 2, 16) == -1 and H.spectrum_bytes(4, 9, 16) == -1
    assert H.forward_workspace_bytes(0, 4, 2, 16) == -1


# Fake, well-aligned, non-overlapping device addresses: every call below must
# fail validation on the host, so none of them is ever dereferenced.
A, Bp, C, Dp, Y, W = (0x10000000 * k for k in range(1, 7))


def _fwd(v=A, x=(Bp, C), spec=Dp, y=Y, B=1, D=4, N=2, L=64, io=0, ws=0, wsb=0):
    xs = None if x is None else (vp * max(1, len(x)))(*x)
    return H.lib().hyena_forward(vp(v), xs, vp(spec), vp(y), B, D, N, L, io, vp(ws), wsb, None)


def test_forward_rejects_bad_arguments():
    assert _fwd(v=0) == NULL
    assert _fwd(x=None) == NULL
    assert _fwd(x=(Bp, 0)) == NULL
    assert _fwd(spec=0) == NULL
    assert _fwd(y=0) == NULL
    assert _fwd(B=0) == SHAPE
    assert _fwd(D=0) == SHAPE
    assert _fwd(N=0, x=(Bp,)) == SHAPE
    assert _fwd(L=0) == SHAPE
    assert _fwd(L=(1 << 22) + 1) == SHAPE
    assert _fwd(N=9, x=tuple(Bp + 0x1000000 * i for i in range(9))) == UNSUP
    assert _fwd(io=7) == UNSUP
    assert _fwd(v=A + 4) == ALIGN
    assert _fwd(x=(Bp, C + 8)) == ALIGN
    assert _fwd(y=Y + 2) == ALIGN
    assert _fwd(spec=Dp + 4) == ALIGN
    assert _fwd(y=A) == ALIAS                       # y == v
    assert _fwd(y=C + 64) == ALIAS                  # y inside x_2
    assert _fwd(y=Dp + 16) == ALIAS                 # y inside the spectrum
    # four-step path needs a workspace
    assert _fwd(L=65536, ws=0, wsb=0) == WS
    assert _fwd(L=65536, ws=W, wsb=1024) == WS
    assert _fwd(L=65536, ws=A, wsb=1 << 24, y=Y) == ALIAS


def _fwd_static(v=A, x=(Bp, C), spec=Dp, y=Y, B=1, D=4, N=2, L=64, io=0):
    xs = None if x is None else (vp * max(1, len(x)))(*x)
    return H.lib().hyena_forward_static(vp(v), xs, vp(spec), vp(y), B, D, N, L, io, None)


def test_forward_static_rejects_bad_arguments():
    # the same host checks as hyena_forward, before the scratch is looked up
    assert _fwd_static(v=0) == NULL
    assert _fwd_static(x=(Bp, 0)) == NULL
    assert _fwd_static(B=0) == SHAPE
    assert _fwd_static(L=(1 << 22) + 1) == SHAPE
    assert _fwd_static(N=9, x=tuple(Bp + 0x1000000 * i for i in range(9))) == UNSUP
    assert _fwd_static(io=7) == UNSUP
    assert _fwd_static(y=Y + 2) == ALIGN
    assert _fwd_static(y=A) == ALIAS
    assert _fwd_static(L=65536, y=C + 64) == ALIAS


def test_spectrum_and_filter_gen_reject_bad_arguments():
    lib = H.lib()
    assert lib.hyena_filter_spectrum(None, 4, 2, 64, vp(Dp), None, 0, None) == NULL
    assert lib.hyena_filter_spectrum(vp(A), 4, 2, 64, None, None, 0, None) == NULL
    assert lib.hyena_filter_spectrum(vp(A), 0, 2, 64, vp(Dp), None, 0, None) == SHAPE
    assert lib.hyena_filter_spectrum(vp(A), 4, 9, 64, vp(Dp), None, 0, None) == UNSUP
    assert lib.hyena_filter_spectrum(vp(A + 4), 4, 2, 64, vp(Dp), None, 0, None) == ALIGN
    assert lib.hyena_filter_spectrum(vp(A), 4, 2, 64, vp(A + 256), None, 0, None) == ALIAS
    assert lib.hyena_filter_spectrum(vp(A), 4, 2, 65536, vp(Dp), None, 0, None) == WS
    assert lib.hyena_spectrum_export(None, 4, 2, 64, vp(Y), None) == NULL
    assert lib.hyena_spectrum_export(vp(Dp), 4, 2, 64, vp(Dp), None) == ALIAS
    p = H.FilterParams(4, 2, 8, 64, A, 0, Bp, 0, C, 0, Dp)
    assert lib.hyena_filter_gen(ctypes.byref(p), 64, None, None) == NULL
    assert lib.hyena_filter_gen(None, 64, vp(Y), None) == NULL
    assert lib.hyena_filter_gen(ctypes.byref(H.FilterParams(4, 2, 8, 64, 0, 0, Bp, 0, C, 0, Dp)), 64, vp(Y), None) == NULL
    assert lib.hyena_filter_gen(ctypes.byref(H.FilterParams(4, 2, 8, 48, A, 0, Bp, 0, C, 0, Dp)), 64, vp(Y), None) == UNSUP
    assert lib.hyena_filter_gen(ctypes.byref(H.FilterParams(4, 2, 17, 64, A, 0, Bp, 0, C, 0, Dp)), 64, vp(Y), None) == SHAPE
    assert lib.hyena_filter_gen(ctypes.byref(p), 0, vp(Y), None) == SHAPE
    assert lib.hyena_filter_gen(ctypes.byref(p), 64, vp(Y + 4), None) == ALIGN


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(H, "_lib", None)
    monkeypatch.setattr(H, "LIB_PATH", "/nonexistent/libhyena_mi355x.so")
    with pytest.raises(RuntimeError, match="missing"):
        H.lib()


def _bp(D=4, N=2, T=3, W_in=A, w=Bp, W_out=C, b_in=0, b_out=0):
    return H.BlockParams(D, N, T, 0, W_in, b_in, w, W_out, b_out)


def test_block_calls_reject_bad_arguments():
    lib = H.lib()
    st = (vp * 3)(Y, Y + 0x1000000, Y + 0x2000000)
    inp = lambda u=Dp, p=None, s=st, B=1, L=64, io=0: lib.hyena_in_projection(
        vp(u), None if p is False else ctypes.byref(p or _bp()), s, B, L, io, None)
    assert inp(u=0) == NULL
    assert inp(p=False) == NULL
    assert inp(s=None) == NULL
    assert inp(p=_bp(W_in=0)) == NULL
    assert inp(p=_bp(w=0)) == NULL
    assert inp(s=(vp * 3)(Y, 0, Y + 0x2000000)) == NULL
    assert inp(B=0) == SHAPE
    assert inp(L=0) == SHAPE
    assert inp(p=_bp(T=0)) == SHAPE
    assert inp(p=_bp(T=17)) == SHAPE
    assert inp(p=_bp(N=9)) == UNSUP
    assert inp(io=5) == UNSUP
    assert inp(u=Dp + 8) == ALIGN
    assert inp(s=(vp * 3)(Y, Y + 0x1000000, Y + 0x2000000 + 4)) == ALIGN
    assert inp(s=(vp * 3)(Dp, Y + 0x1000000, Y + 0x2000000)) == ALIAS      # v over u
    assert inp(s=(vp * 3)(Y, Y + 64, Y + 0x2000000)) == ALIAS               # two streams overlap
    outp = lambda y=Dp, p=None, o=Y, B=1, L=64: lib.hyena_out_projection(
        vp(y), ctypes.byref(p or _bp()), vp(o), B, L, 0, None)
    assert outp(y=0) == NULL
    assert outp(o=0) == NULL
    assert outp(p=_bp(W_out=0)) == NULL
    assert outp(L=(1 << 22) + 1) == SHAPE
    assert outp(o=Y + 2) == ALIGN
    assert outp(o=Dp) == ALIAS
    assert H.block_workspace_bytes(2, 768, 2, 2048) == 4 * 2 * 768 * 2048 * 4
    assert H.block_workspace_bytes(0, 768, 2, 2048) == -1
    ws = H.block_workspace_bytes(1, 8, 2, 65536, "bf16")
    assert ws > 4 * 8 * 65536 * 2
    blk = lambda u=Dp, o=Y, w=W, wsb=1 << 30: lib.hyena_block_forward(
        vp(u), ctypes.byref(_bp()), vp(A), vp(o), 1, 64, 0, vp(w), wsb, None)
    assert blk(w=0) == NULL
    assert blk(wsb=16) == WS
    assert blk(o=Dp) == ALIAS


def test_backward_rejects_bad_arguments():
    lib = H.lib()
    x = (vp * 2)(Bp, C)
    gx = (vp * 2)(Y + 0x100000, Y + 0x200000)
    bw = lambda v=A, x=x, spec=Dp, gy=W, gv=Y, gx=gx, gh=Y + 0x300000, B=1, D=4, N=2, L=64, io=0, ws=0x70000000, wsb=1 << 24: \
        lib.hyena_backward(vp(v), x, vp(spec), vp(gy), vp(gv), gx, vp(gh), B, D, N, L, io, vp(ws), wsb, None)
    assert bw(v=0) == NULL
    assert bw(gy=0) == NULL
    assert bw(gh=0) == NULL
    assert bw(ws=0) == NULL
    assert bw(gx=(vp * 2)(Y + 0x100000, 0)) == NULL
    assert bw(B=0) == SHAPE
    assert bw(N=9, x=(vp * 9)(*[Bp + 0x10000 * i for i in range(9)])) == UNSUP
    assert bw(L=9000, wsb=1 << 20) == WS                        # long rows need the larger workspace
    assert bw(gv=Y + 4) == ALIGN
    assert bw(wsb=16) == WS
    assert bw(gv=A) == ALIAS                                    # gv over v
    assert bw(gh=Y) == ALIAS                                    # gh over gv
    assert bw(gx=(vp * 2)(Y + 0x100000, Bp)) == ALIAS           # gx_2 over x_1
    assert H.backward_workspace_bytes(4, 768, 2, 2048) > 0
    # four-step lengths: saved c_n, one temporary row buffer, per-row spectra, the pass intermediate
    R, L = 4, 20000
    assert H.backward_workspace_bytes(1, 4, 2, L) >= (2 + 1) * R * L * 4 + R * (32768 + 1) * 8
    # 8192 < L <= 16384: the single-path spectrum is rewritten into the four-step layout (extra N*D rows)
    assert H.backward_workspace_bytes(1, 4, 2, 12000) > H.backward_workspace_bytes(1, 4, 2, 8192)


def test_filter_family_calls_reject_bad_arguments():
    lib = H.lib()
    assert lib.hyena_filter_gen_li(None, vp(Bp), 4, 2, 8, 64, vp(Y), None) == NULL
    assert lib.hyena_filter_gen_li(vp(A), vp(Bp), 4, 2, 0, 64, vp(Y), None) == SHAPE
    assert lib.hyena_filter_gen_li(vp(A), vp(Bp), 4, 2, 65, 64, vp(Y), None) == SHAPE
    assert lib.hyena_filter_gen_li(vp(A), vp(Bp), 4, 2, 8, 64, vp(Y + 4), None) == ALIGN
    assert lib.hyena_filter_gen_li(vp(A), vp(Bp), 4, 2, 8, 64, vp(A), None) == ALIAS
    assert lib.hyena_filter_gen_mr(vp(A), None, 4, 2, 16, vp(Y), None) == NULL
    assert lib.hyena_filter_gen_mr(vp(A), vp(Bp), 4, 2, 0, vp(Y), None) == SHAPE
    assert lib.hyena_filter_gen_mr(vp(A), vp(Bp), 4, 2, 16, vp(A + 64), None) == ALIAS
    x = (vp * 2)(Bp, C)
    fir = lambda v=A, x=x, h=Dp, Lh=7, y=Y, B=1, D=4, N=2, L=64, io=0: lib.hyena_forward_fir(
        vp(v), x, vp(h), Lh, vp(y), B, D, N, L, io, None)
    assert fir(h=0) == NULL
    assert fir(Lh=0) == SHAPE
    assert fir(Lh=257) == SHAPE
    assert fir(N=9, x=(vp * 9)(*[Bp + 0x10000 * i for i in range(9)])) == UNSUP
    assert fir(y=Y + 2) == ALIGN
    assert fir(y=C) == ALIAS
    assert fir(y=Dp) == ALIAS


@pytest.mark.parametrize("L,path", [(128, "single"), (2048, "single"), (32768, "single"), (65536, "fourstep"),
                                    (1 << 22, "fourstep")])
def test_plan_circular(L, path):
    p = H.plan(L, circular=True)
    assert p["M"] == L and p["path"] == path
    if path == "fourstep":
        assert p["n1"] * p["n2"] == L // 2


def test_plan_circular_rejects_other_lengths():
    for L in (100, 64, 3000, 127):
        with pytest.raises(H.HyenaError) as e:
            H.plan(L, circular=True)
        assert e.value.code == UNSUP
    assert H.spectrum_bytes(4, 2, 1000, circular=True) == -1
    assert H.lib().hyena_plan_ex(256, 7, ctypes.byref(H.PlanInfo())) == UNSUP


@pytest.mark.parametrize("dims,circ,P", [((65, 4), False, 256), ((512, 3), False, 1024), ((256, 256), True, 256),
                                         ((1024, 1024), True, 1024), ((20, 24, 18), False, 64),
                                         ((64, 3, 1), False, 128), ((64, 64, 64), True, 64),
                                         ((128, 128, 128), True, 128),
                                         ((8, 8), False, 16), ((1, 1), False, 16), ((9, 9), False, 32),
                                         ((56, 56), False, 128), ((64, 3), False, 128), ((4, 4, 4), False, 8),
                                         ((5, 2, 3), False, 16), ((16, 16, 16), False, 32), ((16, 16), True, 16),
                                         ((128, 128), True, 128), ((8, 8, 8), True, 8), ((32, 32, 32), True, 32)])
def test_nd_plan(dims, circ, P):
    assert H.nd_plan(dims, circ) == P
    NC = P ** len(dims) // 2
    Q = NC // (P // 2)
    stride = -(-(NC + Q) // 64) * 64
    assert H.nd_spectrum_bytes(6, dims, circ) == 6 * stride * 8
    # multi-pass 2-D grids (P >= 256) need a workspace of whole complex grids; single-pass ones none
    ws = H.nd_workspace_bytes(6, dims, circ)
    multi = P >= 256 if len(dims) == 2 else P >= 64
    assert (ws >= NC * 8 and ws % (NC * 8) == 0) if multi else ws == 0


def test_nd_plan_rejects_unsupported():
    for dims, circ, code in [((513, 4), False, UNSUP), ((65, 1, 1), False, UNSUP), ((32, 16), True, UNSUP),
                             ((8, 8), True, UNSUP), ((2048, 2048), True, UNSUP), ((12, 12), True, UNSUP),
                             ((4,), False, UNSUP), ((4, 4, 4, 4), False, UNSUP), ((0, 4), False, SHAPE),
                             ((5000, 4), False, SHAPE)]:
        with pytest.raises(H.HyenaError) as e:
            H.nd_plan(dims, circ)
        assert e.value.code == code, (dims, circ)
        assert H.nd_spectrum_bytes(2, dims, circ) == -1


def test_nd_calls_reject_bad_arguments():
    lib = H.lib()
    d2 = (ctypes.c_int64 * 2)(16, 16)
    bad = (ctypes.c_int64 * 2)(600, 16)
    xs = (vp * 2)(Bp, C)
    fwd = lambda **k: lib.hyena_nd_forward(
        vp(k.get("v", A)), k.get("x", xs), vp(k.get("spec", Dp)), vp(k.get("y", Y)), k.get("B", 2),
        k.get("D", 3), k.get("N", 2), k.get("ndim", 2), k.get("dims", d2), k.get("circ", 0), k.get("ps", 0),
        k.get("io", 0), vp(k.get("ws", 0)), k.get("wsb", 0), None)
    assert fwd(v=0) == NULL
    assert fwd(x=None) == NULL
    assert fwd(x=(vp * 2)(Bp, 0)) == NULL
    assert fwd(dims=None) == NULL
    assert fwd(B=0) == SHAPE
    assert fwd(N=0) == SHAPE
    assert fwd(N=9) == UNSUP
    assert fwd(ps=2) == UNSUP
    assert fwd(io=5) == UNSUP
    assert fwd(ndim=4) == UNSUP
    assert fwd(dims=bad) == UNSUP
    assert fwd(circ=1, dims=(ctypes.c_int64 * 2)(16, 8)) == UNSUP
    assert fwd(v=A + 4) == ALIGN
    assert fwd(y=A) == ALIAS
    assert fwd(y=C + 64) == ALIAS
    assert fwd(y=Dp + 16) == ALIAS
    big = (ctypes.c_int64 * 2)(200, 200)                        # P = 512: multi-pass, needs a workspace
    assert fwd(dims=big) == WS
    assert fwd(dims=big, ws=W, wsb=1024) == WS
    assert fwd(dims=big, ws=W + 8, wsb=1 << 24) == ALIGN
    assert fwd(dims=big, ws=A, wsb=1 << 24) == ALIAS
    sp = lambda k=A, rows=4, dims=d2, spec=Dp, ws=0, wsb=0: lib.hyena_nd_filter_spectrum(
        vp(k), rows, 2, dims, 0, vp(spec), vp(ws), wsb, None)
    assert sp(k=0) == NULL
    assert sp(rows=0) == SHAPE
    assert sp(dims=bad) == UNSUP
    assert sp(k=A + 8) == ALIGN
    assert sp(spec=A + 64) == ALIAS
    assert sp(dims=big) == WS
    assert sp(dims=big, ws=Dp + 64, wsb=1 << 24) == ALIAS
    assert H.nd_workspace_bytes(4, (200, 200)) >= 512 * 256 * 8
    assert H.nd_workspace_bytes(4, (8, 8)) == 0


def test_forward_workspace_bf16_intermediate_up_to_order_2():
    """Four-step lengths: bf16 activations keep the intermediate as 4-byte
    bf16 pairs up to order 2 (half the fp32 workspace), float2 beyond."""
    L, B, D = 65536, 1, 64
    for N in (1, 2, 3):
        f = H.forward_workspace_bytes(B, D, N, L, "fp32")
        b = H.forward_workspace_bytes(B, D, N, L, "bf16")
        assert f > 0
        assert b == (f // 2 if N <= 2 else f), (N, f, b)
    assert H.forward_workspace_bytes(B, D, 2, 2048, "bf16") == 0      # single path: no workspace
