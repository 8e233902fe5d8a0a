"""Host-side checks of libgma.so: it loads without a GPU, exports every entry point that
include/gma.h declares, and rejects invalid arguments before making any HIP call.
No test here launches work (fake device pointers never reach a kernel)."""
import ctypes
import os
import re

import pytest

from gaussian_mixture_sequence_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gma.h")
OK, NULLP, SHAPE, VALUE, UNSUP, MISAL, WS, HIP = range(8)
FAKE = 0x10000  # aligned, never dereferenced: validation fails before any HIP call


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gb.LIB_PATH):
        from gaussian_mixture_sequence_amd import build
        build.build()
    return gb.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gma_[a-z_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(gb.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in enumerate(gb.STATUS_NAMES):
        assert gb.gma_status_string(code) == name
    assert gb.gma_status_string(99) == "GMA_ERR_UNKNOWN"


def ws_size(op, B, H, N, dr, dv, K, io, chunk=64):
    out = ctypes.c_size_t(0)
    st = gb.load().gma_workspace_size(op, ctypes.byref(gb.Shape(B, H, N, dr, dv, K)), io, chunk, ctypes.byref(out))
    return st, out.value


def test_workspace_size_validation(lib):
    F, BF = gb.GMA_F32, gb.GMA_BF16
    R, Bd, C = gb.GMA_OP_RESPONSIBILITIES, gb.GMA_OP_BIDIR, gb.GMA_OP_CAUSAL
    assert ws_size(Bd, 1, 1, 256, 16, 32, 8, F)[0] == OK
    assert ws_size(Bd, 8, 8, 4096, 64, 64, 64, BF)[0] == OK
    assert ws_size(C, 2, 16, 32768, 64, 128, 256, BF)[0] == OK
    assert ws_size(Bd, -1, 1, 8, 16, 32, 8, F)[0] == SHAPE
    assert ws_size(Bd, 1, 1, -8, 16, 32, 8, F)[0] == SHAPE
    assert ws_size(Bd, 1, 1, 8, 16, 32, 257, F)[0] == UNSUP
    assert ws_size(Bd, 1, 1, 8, 16, 32, 0, F)[0] == UNSUP
    assert ws_size(Bd, 1, 1, 8, 129, 32, 8, F)[0] == UNSUP
    assert ws_size(Bd, 1, 1, 8, 24, 32, 8, BF)[0] == UNSUP      # bf16 d_r set
    assert ws_size(Bd, 1, 1, 8, 16, 48, 8, BF)[0] == UNSUP      # bf16 d_v set
    assert ws_size(R, 1, 1, 8, 16, 0, 8, BF)[0] == OK            # d_v ignored
    assert ws_size(C, 1, 1, 8, 16, 32, 8, F, chunk=24)[0] == UNSUP
    for ch in (16, 32, 64, 128):  # the chunk set of the causal scan
        assert ws_size(C, 1, 1, 8, 16, 32, 8, F, chunk=ch)[0] == OK, ch
        assert ws_size(C, 1, 1, 8, 16, 32, 8, BF, chunk=ch)[0] == (UNSUP if ch == 16 else OK), ch
    for ch in (0, 8, 24, 48, 96, 256):
        assert ws_size(C, 1, 1, 8, 16, 32, 8, F, chunk=ch)[0] == UNSUP, ch
    assert ws_size(7, 1, 1, 8, 16, 32, 8, F)[0] == VALUE
    assert ws_size(Bd, 1, 1, 8, 16, 32, 8, 5)[0] == VALUE
    assert gb.load().gma_workspace_size(Bd, None, F, 64, ctypes.byref(ctypes.c_size_t())) == NULLP


def test_workspace_is_bounded_in_sequence_length(lib):
    """Scratch is O(K d_v) per problem and split: it stops growing with N (linear total
    memory in N comes only from the caller's inputs and output)."""
    for op in (gb.GMA_OP_BIDIR, gb.GMA_OP_CAUSAL):
        sizes = [ws_size(op, 4, 4, n, 32, 64, 128, gb.GMA_BF16)[1] for n in (65536, 1 << 18, 1 << 20)]
        assert sizes[0] == sizes[1] == sizes[2], sizes


def call_bidir(lib, xq=FAKE, xk=FAKE, v=FAKE, io=gb.GMA_F32, mu=FAKE, s2=FAKE, pi=FAKE, eps=1e-6, o=FAKE,
               shape=(1, 1, 64, 16, 32, 8), ws=FAKE, ws_bytes=None, causal=False, chunk=64):
    sh = gb.Shape(*shape)
    op = gb.GMA_OP_CAUSAL if causal else gb.GMA_OP_BIDIR
    if ws_bytes is None:
        st, ws_bytes = ws_size(op, *shape, io, chunk)
    if causal:
        return lib.gma_forward_causal(xq, xk, v, io, mu, s2, pi, eps, o, ctypes.byref(sh), chunk, ws, ws_bytes, None)
    return lib.gma_forward_bidir(xq, xk, v, io, mu, s2, pi, eps, o, ctypes.byref(sh), ws, ws_bytes, None)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_argument_errors(lib, causal):
    c = dict(causal=causal)
    assert call_bidir(lib, xq=None, **c) == NULLP
    assert call_bidir(lib, o=None, **c) == NULLP
    assert call_bidir(lib, pi=None, **c) == NULLP
    assert call_bidir(lib, ws=None, **c) == NULLP
    assert call_bidir(lib, eps=0.0, **c) == VALUE
    assert call_bidir(lib, eps=-1.0, **c) == VALUE
    assert call_bidir(lib, eps=float("nan"), **c) == VALUE
    assert call_bidir(lib, eps=float("inf"), **c) == VALUE
    assert call_bidir(lib, io=3, **c) == VALUE
    assert call_bidir(lib, shape=(1, -1, 64, 16, 32, 8), **c) == SHAPE
    assert call_bidir(lib, shape=(1, 1, 64, 16, 32, 300), **c) == UNSUP
    assert call_bidir(lib, xk=FAKE + 2, **c) == MISAL
    assert call_bidir(lib, o=FAKE + 8, **c) == MISAL
    assert call_bidir(lib, ws=FAKE + 4, **c) == MISAL
    st, need = ws_size(gb.GMA_OP_CAUSAL if causal else gb.GMA_OP_BIDIR, 1, 1, 64, 16, 32, 8, gb.GMA_F32)
    assert need > 0
    assert call_bidir(lib, ws_bytes=need - 1, **c) == WS
    if causal:
        assert call_bidir(lib, chunk=48, **c) == UNSUP


@pytest.mark.parametrize("causal", [False, True])
def test_empty_problems_enqueue_nothing(lib, causal):
    """B*H*N == 0 is valid and returns before any HIP call."""
    for shape in [(1, 1, 0, 16, 32, 8), (0, 4, 128, 16, 32, 8), (2, 0, 128, 16, 32, 8)]:
        assert call_bidir(lib, shape=shape, causal=causal) == OK
        assert call_bidir(lib, shape=shape, causal=causal, io=gb.GMA_BF16) == OK


def test_responsibilities_argument_errors(lib):
    sh = gb.Shape(1, 1, 64, 16, 1, 8)
    st, need = ws_size(gb.GMA_OP_RESPONSIBILITIES, 1, 1, 64, 16, 1, 8, gb.GMA_F32)
    f = lib.gma_responsibilities
    assert f(None, 0, FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(sh), FAKE, need, None) == NULLP
    assert f(FAKE, 0, FAKE, FAKE, FAKE, FAKE, 9, ctypes.byref(sh), FAKE, need, None) == VALUE
    assert f(FAKE, 0, FAKE, FAKE, FAKE, FAKE + 2, 0, ctypes.byref(sh), FAKE, need, None) == MISAL
    assert f(FAKE, 0, FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(sh), FAKE, need - 1, None) == WS
    empty = gb.Shape(1, 1, 0, 16, 1, 8)
    assert f(FAKE, 0, FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(empty), FAKE, need, None) == OK


def cross_ws(B, H, Nq, Nk, dr, dv, K, io):
    out = ctypes.c_size_t(0)
    st = gb.load().gma_cross_workspace_size(ctypes.byref(gb.CrossShape(B, H, Nq, Nk, dr, dv, K)), io,
                                            ctypes.byref(out))
    return st, out.value


def call_cross(lib, xq=FAKE, xk=FAKE, v=FAKE, io=gb.GMA_F32, eps=1e-6, o=FAKE, shape=(1, 1, 64, 96, 16, 32, 8),
               ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = cross_ws(*shape, io)[1]
    return lib.gma_forward_cross(xq, xk, v, io, FAKE, FAKE, FAKE, eps, o, ctypes.byref(gb.CrossShape(*shape)), ws,
                                 ws_bytes, None)


def test_cross_workspace_size_validation(lib):
    F, BF = gb.GMA_F32, gb.GMA_BF16
    assert cross_ws(8, 8, 4096, 16384, 64, 64, 64, BF)[0] == OK
    assert cross_ws(1, 1, 0, 0, 16, 32, 8, F)[0] == OK
    assert cross_ws(1, 1, -1, 8, 16, 32, 8, F)[0] == SHAPE
    assert cross_ws(1, 1, 8, -1, 16, 32, 8, F)[0] == SHAPE
    assert cross_ws(1, 1, 1 << 41, 8, 16, 32, 8, F)[0] == SHAPE
    assert cross_ws(1 << 20, 1 << 10, 1 << 11, 8, 16, 32, 8, F)[0] == SHAPE   # B*H*N_q beyond 2^40
    assert cross_ws(1, 1, 8, 8, 24, 32, 8, BF)[0] == UNSUP
    assert cross_ws(1, 1, 8, 8, 16, 32, 0, F)[0] == UNSUP
    assert lib.gma_cross_workspace_size(None, F, ctypes.byref(ctypes.c_size_t())) == NULLP
    # with N_q = N_k the plan is the bidirectional one
    assert cross_ws(4, 4, 4096, 4096, 32, 64, 128, BF)[1] == ws_size(gb.GMA_OP_BIDIR, 4, 4, 4096, 32, 64, 128, BF)[1]
    # scratch stops growing with either length
    sizes = [cross_ws(4, 4, nq, nk, 32, 64, 128, BF)[1] for nq, nk in ((65536, 1 << 18), (1 << 20, 65536), (1 << 20, 1 << 20))]
    assert sizes[0] == sizes[1] == sizes[2], sizes


def test_cross_argument_errors(lib):
    assert call_cross(lib, xq=None) == NULLP
    assert call_cross(lib, xk=None) == NULLP
    assert call_cross(lib, o=None) == NULLP
    assert call_cross(lib, ws=None) == NULLP
    assert call_cross(lib, eps=0.0) == VALUE
    assert call_cross(lib, eps=float("nan")) == VALUE
    assert call_cross(lib, io=3) == VALUE
    assert call_cross(lib, shape=(1, 1, -3, 96, 16, 32, 8), ws_bytes=1 << 20) == SHAPE
    assert call_cross(lib, shape=(1, 1, 64, 96, 16, 32, 300), ws_bytes=1 << 20) == UNSUP
    assert call_cross(lib, v=FAKE + 4) == MISAL
    need = cross_ws(1, 1, 64, 96, 16, 32, 8, gb.GMA_F32)[1]
    assert need > 0 and call_cross(lib, ws_bytes=need - 1) == WS


def test_cross_without_output_rows_enqueues_nothing(lib):
    """No query rows (or no problems) is valid and returns before any HIP call."""
    for shape in [(1, 1, 0, 96, 16, 32, 8), (0, 2, 64, 96, 16, 32, 8), (1, 1, 0, 0, 16, 32, 8)]:
        for io in (gb.GMA_F32, gb.GMA_BF16):
            assert call_cross(lib, shape=shape, io=io) == OK
    # a side without rows may come without storage; a side with rows may not
    assert call_cross(lib, xq=None, o=None, shape=(1, 1, 0, 96, 16, 32, 8)) == OK
    assert call_cross(lib, xk=None, v=None, shape=(1, 1, 0, 0, 16, 32, 8)) == OK
    assert call_cross(lib, xk=None, shape=(1, 1, 0, 96, 16, 32, 8)) == NULLP


def test_causal_state_argument_errors(lib):
    """State pointers: optional, 16-byte aligned, state_out not overlapping state_in."""
    shape = (1, 1, 64, 16, 32, 8)
    sh = gb.Shape(*shape)
    st, need = ws_size(gb.GMA_OP_CAUSAL, *shape, gb.GMA_F32)
    f = lib.gma_forward_causal_state
    args = lambda s_in, s_out, n=64: (FAKE, FAKE, FAKE, gb.GMA_F32, FAKE, FAKE, FAKE, 1e-6, FAKE,
                                      ctypes.byref(gb.Shape(1, 1, n, 16, 32, 8)), 64, s_in, s_out, FAKE, need, None)
    sbytes = 8 * 33 * 4
    assert f(*args(FAKE + 4, None)) == MISAL
    assert f(*args(None, FAKE + 8)) == MISAL
    assert f(*args(FAKE, FAKE + sbytes - 16)) == VALUE          # overlap
    assert f(*args(FAKE + sbytes - 16, FAKE)) == VALUE
    assert f(FAKE, FAKE, FAKE, gb.GMA_F32, FAKE, FAKE, FAKE, 0.0, FAKE, ctypes.byref(sh), 64, None, None, FAKE, need,
             None) == VALUE
    assert f(*args(None, None, n=0)) == OK                       # no positions, no state: nothing to do


def test_diagnostics_argument_errors(lib):
    F, BF = gb.GMA_F32, gb.GMA_BF16
    D = gb.GMA_OP_DIAGNOSTICS
    assert ws_size(D, 64, 8, 1024, 64, 0, 128, BF)[0] == OK
    # fp32 input keeps every head's responsibilities; bf16 input runs fused, with per-head operand
    # tables and per-block partial sums only
    assert ws_size(D, 64, 8, 1024, 64, 0, 128, F)[1] >= 64 * 8 * 1024 * 128 * 4
    assert ws_size(D, 64, 8, 1024, 64, 0, 128, BF)[1] < 4 << 20
    assert ws_size(D, 1, 1, 8, 24, 0, 8, BF)[0] == UNSUP
    assert ws_size(D, 1, 1, -8, 16, 0, 8, F)[0] == SHAPE
    shape = (2, 3, 64, 16, 0, 8)
    need = ws_size(D, *shape, F)[1]
    f = lib.gma_responsibility_diagnostics
    sh = ctypes.byref(gb.Shape(*shape))
    assert f(FAKE, F, FAKE, FAKE, FAKE, sh, None, FAKE, FAKE, FAKE, FAKE, need, None) == NULLP   # usage
    assert f(FAKE, F, FAKE, FAKE, FAKE, sh, FAKE, None, FAKE, FAKE, FAKE, need, None) == NULLP   # stats
    assert f(None, F, FAKE, FAKE, FAKE, sh, FAKE, FAKE, None, None, FAKE, need, None) == NULLP
    assert f(FAKE, F, FAKE, FAKE, FAKE, sh, FAKE, FAKE, FAKE + 4, None, FAKE, need, None) == MISAL
    assert f(FAKE, F, FAKE, FAKE, FAKE, sh, FAKE, FAKE, None, None, FAKE, need - 1, None) == WS
    assert f(FAKE, 7, FAKE, FAKE, FAKE, sh, FAKE, FAKE, None, None, FAKE, need, None) == VALUE


@pytest.mark.parametrize("causal", [False, True])
def test_backward_argument_errors(lib, causal):
    F, BF = gb.GMA_F32, gb.GMA_BF16
    Bw = gb.GMA_OP_BACKWARD_CAUSAL if causal else gb.GMA_OP_BACKWARD_BIDIR
    fn = lib.gma_backward_causal if causal else lib.gma_backward_bidir
    assert ws_size(Bw, 8, 8, 4096, 64, 64, 64, F)[0] == OK
    # bf16 I/O: fp32 sizes (d 7 is fine), and fp32 copies of the I/O in the workspace
    assert ws_size(Bw, 8, 8, 4096, 64, 64, 64, BF)[0] == OK
    assert ws_size(Bw, 1, 1, 64, 7, 5, 13, BF)[0] == OK
    assert ws_size(Bw, 8, 8, 4096, 64, 64, 64, BF)[1] >= ws_size(Bw, 8, 8, 4096, 64, 64, 64, F)[1] + 7 * 8 * 8 * 4096 * 64 * 4
    assert ws_size(Bw, 1, 1, 8, 16, 0, 8, F)[0] == UNSUP          # needs values
    assert ws_size(Bw, 1, 1, 8, 129, 32, 8, F)[0] == UNSUP
    assert ws_size(Bw, 1, -1, 8, 16, 32, 8, F)[0] == SHAPE
    # more scratch than the forward: the gradient memory and the parameter partials
    fwd = gb.GMA_OP_CAUSAL if causal else gb.GMA_OP_BIDIR
    assert ws_size(Bw, 8, 8, 4096, 64, 64, 64, F)[1] > ws_size(fwd, 8, 8, 4096, 64, 64, 64, F)[1]
    shape = (2, 3, 64, 16, 32, 8)
    need = ws_size(Bw, *shape, F)[1]
    sh = ctypes.byref(gb.Shape(*shape))

    def call(xq=FAKE, io=F, pi=FAKE, eps=1e-6, d_o=FAKE, dxk=FAKE, dmu=FAKE, dpi=FAKE, ws=FAKE, nb=need, s=sh):
        return fn(xq, FAKE, FAKE, io, FAKE, FAKE, pi, eps, d_o, FAKE, dxk, FAKE, dmu, FAKE, dpi, s, ws, nb, None)

    assert call(xq=None) == NULLP
    assert call(d_o=None) == NULLP
    assert call(dxk=None) == NULLP
    assert call(dmu=None) == NULLP
    assert call(pi=None) == NULLP
    assert call(ws=None) == NULLP
    assert call(io=9) == VALUE
    assert call(eps=0.0) == VALUE
    assert call(eps=float("nan")) == VALUE
    assert call(d_o=FAKE + 4) == MISAL
    assert call(dpi=FAKE + 8) == MISAL
    assert call(nb=need - 1) == WS
    # no heads: nothing to write, returns before any HIP call
    sh0 = gb.Shape(2, 0, 64, 16, 32, 8)
    assert call(s=ctypes.byref(sh0), nb=ws_size(Bw, 2, 0, 64, 16, 32, 8, F)[1], dmu=None, dpi=None) == OK


def test_backward_cross_argument_errors(lib):
    F, BF = gb.GMA_F32, gb.GMA_BF16
    size = lib.gma_backward_cross_workspace_size

    def ws(shape, io=F):
        out = ctypes.c_size_t(0)
        return size(ctypes.byref(gb.CrossShape(*shape)), io, ctypes.byref(out)), out.value

    assert ws((8, 8, 4096, 16384, 64, 64, 64))[0] == OK
    assert ws((8, 8, 4096, 16384, 64, 64, 64), BF)[0] == OK
    assert ws((1, 1, 8, 8, 129, 32, 8))[0] == UNSUP
    assert ws((1, 1, -1, 8, 16, 32, 8))[0] == SHAPE
    assert ws((1, 1, 8, 8, 16, 32, 8), 5)[0] == VALUE
    assert size(None, F, ctypes.byref(ctypes.c_size_t())) == NULLP
    # N_q = N_k: the bidirectional backward's workspace
    same = ctypes.c_size_t(0)
    assert lib.gma_workspace_size(gb.GMA_OP_BACKWARD_BIDIR, ctypes.byref(gb.Shape(2, 3, 700, 16, 32, 8)), F, 0,
                                  ctypes.byref(same)) == OK
    assert ws((2, 3, 700, 700, 16, 32, 8))[1] == same.value
    shape = (2, 3, 64, 100, 16, 32, 8)
    need = ws(shape)[1]
    sh = ctypes.byref(gb.CrossShape(*shape))

    def call(xq=FAKE, xk=FAKE, d_o=FAKE, dv=FAKE, eps=1e-6, nb=need, s=sh):
        return lib.gma_backward_cross(xq, xk, FAKE, F, FAKE, FAKE, FAKE, eps, d_o, FAKE, FAKE, dv, FAKE, FAKE, FAKE,
                                      s, FAKE, nb, None)

    assert call(xq=None) == NULLP
    assert call(xk=None) == NULLP
    assert call(dv=None) == NULLP
    assert call(d_o=FAKE + 4) == MISAL
    assert call(eps=0.0) == VALUE
    assert call(nb=need - 1) == WS


def test_backward_causal_state_argument_errors(lib):
    F = gb.GMA_F32
    shape = (2, 3, 64, 16, 32, 8)
    need = ws_size(gb.GMA_OP_BACKWARD_CAUSAL, *shape, F)[1]
    sh = ctypes.byref(gb.Shape(*shape))
    sb = 2 * 3 * 8 * 33 * 4  # bytes of one [B,H,K,d_v+1] state

    def call(sin=None, dso=None, dsi=FAKE + 0x100000, xq=FAKE):
        return lib.gma_backward_causal_state(xq, FAKE, FAKE, F, FAKE, FAKE, FAKE, 1e-6, FAKE, sin, dso, FAKE, FAKE,
                                             FAKE, FAKE, FAKE, FAKE, dsi, sh, FAKE, need, None)

    assert call(xq=None) == NULLP
    assert call(sin=FAKE + 4) == MISAL
    assert call(dsi=FAKE + 8) == MISAL
    assert call(dso=FAKE + 0x100000 + sb - 16) == VALUE    # dstate_in overlaps dstate_out
    assert call(sin=FAKE + 0x100000 - sb + 16) == VALUE    # dstate_in overlaps state_in


BF16_DIMS = [(dr, K, dv) for dr in (16, 32, 64, 128) for K in (8, 32, 50, 64, 100, 128, 200, 256) for dv in (32, 64, 128)]


@pytest.mark.parametrize("dr,K,dv", BF16_DIMS, ids=lambda x: str(x))
def test_bidir_single_launch_grid_fits_resident_bound(lib, dr, K, dv):
    """The single-launch bf16 bidirectional forward makes each workgroup wait for every split of
    its problem, so its grid must be resident at once.  For every supported dim set, and problem
    counts from one head up to thousands at sequences up to 2^20 positions, the planned grid stays
    within what 256 CUs hold by the kernel's own LDS (160 KiB per CU) and by the two waves per SIMD
    its register budget guarantees, or uses one split per problem (no cross-workgroup wait)."""
    for B, H in ((1, 1), (1, 3), (8, 8), (4, 4), (2, 16), (40, 25)):
        for N in (1, 1000, 4096, 65536, 262144, 1 << 20):
            info = gb.gma_plan_info(gb.GMA_OP_BIDIR, B, H, N, dr, dv, K, gb.GMA_BF16)
            assert info["workgroups"] == B * H * info["splits"]
            assert info["splits"] * info["rows_per_split"] >= N
            assert 0 < info["lds_bytes"] <= 160 * 1024
            assert info["threads_per_workgroup"] in (256, 512)
            per_cu = min((160 * 1024) // info["lds_bytes"], (4 * 2 * 64) // info["threads_per_workgroup"])
            assert info["resident_bound"] <= 256 * max(per_cu, 1)
            if 1 < info["splits"] <= 8:  # the single launch: every workgroup resident
                assert info["waits_on_all_splits"] == 1
                assert info["workgroups"] <= 256 * per_cu, (B, H, N, info)
            else:  # one split per problem, or the write, combine and read launches
                assert info["waits_on_all_splits"] == 0


def test_backward_splits(lib):
    """The backward's own split rule: splits of whole 64-position tiles, about 512 workgroups for
    the bidirectional passes and about 2048 for the causal ones (the forward's rule left half the
    CUs idle at B8 H8 N1024)."""
    F = gb.GMA_F32
    info = lambda op, *sh: gb.gma_plan_info(op, *sh, F)
    b = info(gb.GMA_OP_BACKWARD_BIDIR, 8, 8, 1024, 64, 64, 64)
    assert (b["splits"], b["rows_per_split"], b["workgroups"]) == (8, 128, 512)
    b = info(gb.GMA_OP_BACKWARD_BIDIR, 8, 8, 4096, 64, 64, 64)
    assert (b["splits"], b["rows_per_split"], b["workgroups"]) == (8, 512, 512)
    c = info(gb.GMA_OP_BACKWARD_CAUSAL, 8, 8, 1024, 64, 64, 256)
    assert (c["splits"], c["rows_per_split"], c["workgroups"]) == (16, 64, 1024)
    c = info(gb.GMA_OP_BACKWARD_CAUSAL, 8, 12, 2048, 64, 64, 32)
    assert (c["splits"], c["rows_per_split"]) == (16, 128)
    for op in (gb.GMA_OP_BACKWARD_BIDIR, gb.GMA_OP_BACKWARD_CAUSAL):
        for sh in [(1, 1, 1, 16, 32, 8), (2, 3, 700, 16, 32, 8), (1, 2, 100000, 32, 32, 64), (64, 64, 300, 16, 16, 8)]:
            r = info(op, *sh)
            N = sh[2]
            assert r["rows_per_split"] % 64 == 0 and r["splits"] * r["rows_per_split"] >= N
            assert (r["splits"] - 1) * r["rows_per_split"] < N            # no empty split
            assert r["workgroups"] == sh[0] * sh[1] * r["splits"]
            assert r["threads_per_workgroup"] == r["lds_bytes"] == r["chunk_used"] == 0


def test_plan_info_validation(lib):
    info = gb.PlanInfo()
    sh = gb.Shape(1, 1, 8, 16, 32, 8)
    assert lib.gma_plan_info(gb.GMA_OP_BIDIR, None, gb.GMA_BF16, 0, ctypes.byref(info)) == NULLP
    assert lib.gma_plan_info(gb.GMA_OP_BIDIR, ctypes.byref(sh), gb.GMA_BF16, 0, None) == NULLP
    assert lib.gma_plan_info(gb.GMA_OP_RESPONSIBILITIES, ctypes.byref(sh), gb.GMA_BF16, 0, ctypes.byref(info)) == VALUE
    assert lib.gma_plan_info(gb.GMA_OP_CAUSAL, ctypes.byref(sh), gb.GMA_BF16, 24, ctypes.byref(info)) == UNSUP
    assert lib.gma_plan_info(gb.GMA_OP_BIDIR, ctypes.byref(gb.Shape(1, 1, 8, 24, 32, 8)), gb.GMA_BF16, 0,
                             ctypes.byref(info)) == UNSUP
    c = gb.gma_plan_info(gb.GMA_OP_CAUSAL, 8, 12, 2048, 64, 64, 32, gb.GMA_BF16, 64)
    assert c["threads_per_workgroup"] == 0 and c["workgroups"] == 96 * c["splits"]
    f = gb.gma_plan_info(gb.GMA_OP_BIDIR, 8, 8, 4096, 64, 64, 64, gb.GMA_F32)
    assert f["lds_bytes"] == 0 and f["waits_on_all_splits"] == 0


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_causal_chunk_used(lib, io):
    """The scan runs the largest power of two not above the requested chunk that its tiles allow:
    never more than requested, at least 32 with bf16 (its 32-position score tiles), at most 64 on
    the bf16 path and 32 for 256 padded components with d_r <= 64."""
    dt = gb.GMA_BF16 if io == "bf16" else gb.GMA_F32
    for dr, dv, K in ((64, 64, 32), (16, 32, 8), (32, 64, 128), (64, 128, 256), (128, 128, 256), (64, 32, 50)):
        used = {}
        for ch in (16, 32, 64, 128):
            if io == "bf16" and ch == 16:
                continue
            u = gb.gma_plan_info(gb.GMA_OP_CAUSAL, 2, 3, 1000, dr, dv, K, dt, ch)["chunk_used"]
            assert u <= ch and u & (u - 1) == 0, (dr, dv, K, ch, u)
            if io == "bf16":
                assert 32 <= u <= 64 and (u == 32 if (K > 128 and dr <= 64) else True), (dr, dv, K, ch, u)
            used[ch] = u
        vals = [used[c] for c in sorted(used)]
        assert vals == sorted(vals), used  # a longer request never runs a shorter chunk
    assert gb.gma_plan_info(gb.GMA_OP_BIDIR, 1, 1, 100, 64, 64, 64, dt)["chunk_used"] == 0
