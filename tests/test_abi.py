"""CPU tests of the C ABI of libmssm.so: the library loads without a GPU,
exports every function include/mssm.h declares, and rejects invalid
arguments on the host with the documented status codes before any HIP call
(no valid call is made here: without a GPU it would have nothing to run on)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mssm.h")

mssm = pytest.importorskip("selective_state_space_mssm_amd")
lib = mssm.lib
P = mssm.Problem

FAKE = 0x10000  # aligned, non-null stand-in pointer: validation fails before any use
MIS = 0x10004   # misaligned


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mssm_status|size_t|const char\*)\s+(mssm_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_function():
    names = header_functions()
    assert len(names) == 26, names
    for n in names:
        assert hasattr(lib, n), f"libmssm.so does not export {n}"
    assert sorted(mssm.EXPORTS) == names


def test_status_strings():
    for code, name in mssm.binding.STATUS.items():
        s = lib.mssm_status_string(code).decode()
        assert s.startswith(name), (code, s)
    assert "unknown" in lib.mssm_status_string(-99).decode()
    assert b"gfx950" in lib.mssm_build_info()


def fwd(p, u=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dskip=None, z=None, dt_bias=None,
        h0=None, y=FAKE, hf=None, ws=None, wsb=0):
    pp = ctypes.byref(p) if p is not None else None
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.mssm_scan_fwd(pp, v(u), v(delta), v(A), v(Bm), v(Cm), v(Dskip), v(z), v(dt_bias),
                             v(h0), v(y), v(hf), v(ws), wsb, None)


def conv_fwd(p, d_conv=4, **kw):
    names = ["x", "conv_w", "conv_b", "x_prev", "delta", "A", "Bm", "Cm", "Dskip", "z", "dt_bias", "h0", "y",
             "h_final", "u_out"]
    required = {"x", "conv_w", "delta", "A", "Bm", "Cm", "y"}
    args = []
    for n in names:
        x = kw.get(n, FAKE if n in required else None)
        args.append(None if x is None else ctypes.c_void_p(x))
    ws = kw.get("ws", None)
    return lib.mssm_conv_scan_fwd(ctypes.byref(p) if p is not None else None, d_conv, *args,
                                  None if ws is None else ctypes.c_void_p(ws), kw.get("wsb", 0), None)


def bwd(p, **kw):
    names = ["u", "delta", "A", "Bm", "Cm", "Dskip", "z", "dt_bias", "h0", "dy", "dh_final", "du",
             "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dh0"]
    required = {"u", "delta", "A", "Bm", "Cm", "dy", "du", "ddelta", "dA", "dB", "dC"}
    args = []
    for n in names:
        x = kw.get(n, FAKE if n in required else None)
        args.append(None if x is None else ctypes.c_void_p(x))
    ws = kw.get("ws", FAKE)
    return lib.mssm_scan_bwd(ctypes.byref(p) if p is not None else None, *args,
                             None if ws is None else ctypes.c_void_p(ws), kw.get("wsb", 1 << 40), None)


def step(p, **kw):
    names = ["u_t", "delta_t", "A", "Bm_t", "Cm_t", "Dskip", "z_t", "dt_bias", "state", "y_t"]
    required = {"u_t", "delta_t", "A", "Bm_t", "Cm_t", "state", "y_t"}
    args = [None if kw.get(n, FAKE if n in required else None) is None
            else ctypes.c_void_p(kw.get(n, FAKE)) for n in names]
    return lib.mssm_step(ctypes.byref(p) if p is not None else None, *args, None)


def good(B=2, L=64, D=32, N=16, dtype=0, sp=1):
    return P(B, L, D, N, dtype, sp)


def test_problem_validation():
    assert fwd(None) == -1
    assert fwd(good(dtype=2)) == -3
    assert fwd(good(dtype=-1)) == -3
    for bad in (good(B=0), good(L=0), good(D=0), good(N=0), good(B=-3), good(L=-1)):
        assert fwd(bad) == -2
    assert fwd(good(B=1 << 20, D=1 << 11)) == -2     # B*D >= 2^31
    assert fwd(good(L=1 << 31)) == -2
    assert fwd(good(N=65)) == -4
    assert fwd(good(N=128)) == -4
    # any dstate up to 64 is valid (not a power of two: padded in the workspace), so N = 12 gets as far as the
    # workspace check
    assert lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(good(N=12))) > 0
    assert fwd(good(N=12)) == -6
    # the same checks guard the backward and the step
    assert bwd(good(N=65)) == -4
    assert bwd(good(dtype=5)) == -3
    assert step(good(N=96)) == -4
    assert step(good(D=0)) == -2


def test_step_ignores_seqlen_for_validation():
    # seqlen = 0 is fine for the step; use a null state so validation still stops the call
    assert step(P(2, 0, 32, 16, 0, 1), state=None) == -1


def test_required_pointers():
    for k in ("u", "delta", "A", "Bm", "Cm", "y"):
        assert fwd(good(), **{k: None}) == -1, k
    for k in ("u", "delta", "A", "Bm", "Cm", "dy", "du", "ddelta", "dA", "dB", "dC"):
        assert bwd(good(), **{k: None}) == -1, k
    assert bwd(good(), z=FAKE, dz=None) == -1      # dz required with a gate
    for k in ("u_t", "delta_t", "A", "Bm_t", "Cm_t", "state", "y_t"):
        assert step(good(), **{k: None}) == -1, k


def test_alignment():
    for k in ("u", "delta", "A", "Bm", "Cm", "Dskip", "z", "dt_bias", "h0", "y", "hf"):
        assert fwd(good(), **{k: MIS}) == -5, k
    for k in ("u", "dy", "dB", "dD", "dh0", "dh_final"):
        assert bwd(good(), **{k: MIS}) == -5, k
    assert step(good(), state=MIS) == -5


def test_conv_front_end_validation():
    # the problem checks of the forward, then the conv's own: width, required taps, alignment
    assert conv_fwd(None) == -1
    assert conv_fwd(good(N=72)) == -4
    assert conv_fwd(good(L=0)) == -2
    for k in (0, 5, -1):
        assert conv_fwd(good(), d_conv=k) == -2, k
    for k in ("x", "conv_w", "delta", "A", "Bm", "Cm", "y"):
        assert conv_fwd(good(), **{k: None}) == -1, k
    for k in ("x", "conv_w", "conv_b", "x_prev", "u_out", "h_final"):
        assert conv_fwd(good(), **{k: MIS}) == -5, k
    long_ = P(1, 1 << 20, 1536, 16, 1, 1)
    nws = lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(long_))
    assert conv_fwd(long_, ws=None) == -6
    assert conv_fwd(long_, ws=FAKE, wsb=nws - 1) == -6


def test_conv_backward_validation():
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731

    def cb(p, d_conv=4, x=FAKE, w=FAKE, b=None, xp=None, du=FAKE, dx=FAKE, dw=FAKE, db=None, dxp=None, ws=FAKE,
           wsb=1 << 40):
        return lib.mssm_conv_bwd(ctypes.byref(p) if p is not None else None, d_conv, v(x), v(w), v(b), v(xp), v(du),
                                 v(dx), v(dw), v(db), v(dxp), v(ws), wsb, None)
    assert cb(None) == -1
    assert cb(good(dtype=3)) == -3
    assert cb(good(L=0)) == -2
    assert cb(good(N=12), x=None) == -1   # the state size plays no part: validation goes on to the pointers
    for k in (0, 5):
        assert cb(good(), d_conv=k) == -2
    for k in ("x", "w", "du", "dx", "dw"):
        assert cb(good(), **{k: None}) == -1, k
    for k in ("x", "w", "b", "xp", "du", "dx", "dw", "db", "dxp"):
        assert cb(good(), **{k: MIS}) == -5, k
    nws = lib.mssm_conv_bwd_workspace_bytes(ctypes.byref(good()), 4)
    assert nws > 0
    assert cb(good(), ws=None) == -6
    assert cb(good(), wsb=nws - 1) == -6
    assert lib.mssm_conv_bwd_workspace_bytes(ctypes.byref(good()), 9) == 0


def test_conv_step_validation():
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731

    def cs(p, d_conv=4, **kw):
        names = ["x_t", "conv_w", "conv_b", "conv_state", "delta_t", "A", "Bm_t", "Cm_t", "Dskip", "z_t", "dt_bias",
                 "state", "y_t"]
        req = {"x_t", "conv_w", "conv_state", "delta_t", "A", "Bm_t", "Cm_t", "state", "y_t"}
        args = [v(kw.get(n, FAKE if n in req else None)) for n in names]
        return lib.mssm_conv_step(ctypes.byref(p) if p is not None else None, d_conv, *args, None)
    assert cs(None) == -1
    assert cs(good(N=72)) == -4
    for k in (0, 5):
        assert cs(good(), d_conv=k) == -2
    for k in ("x_t", "conv_w", "conv_state", "delta_t", "A", "Bm_t", "Cm_t", "state", "y_t"):
        assert cs(good(), **{k: None}) == -1, k
    for k in ("x_t", "conv_w", "conv_b", "conv_state", "state", "y_t"):
        assert cs(good(), **{k: MIS}) == -5, k


def ssd(p, **kw):
    names = ["x", "dt", "A", "Bm", "Cm", "Dskip", "dt_bias", "h0", "y", "h_final"]
    required = {"x", "dt", "A", "Bm", "Cm", "y"}
    args = [None if kw.get(n, FAKE if n in required else None) is None else
            ctypes.c_void_p(kw.get(n, FAKE)) for n in names]
    ws = kw.get("ws", None)
    return lib.mssm_ssd_fwd(ctypes.byref(p) if p is not None else None, *args,
                            None if ws is None else ctypes.c_void_p(ws), kw.get("wsb", 0), None)


def test_ssd_validation():
    S = mssm.binding.SsdProblem
    good = lambda **k: S(**{**dict(batch=2, seqlen=100, nheads=3, headdim=64, dstate=64, dtype=0,  # noqa: E731
                                   delta_softplus=1), **k})
    assert ssd(None) == -1
    assert ssd(good(dtype=7)) == -3
    for k in ("batch", "seqlen", "nheads", "headdim", "dstate"):
        assert ssd(good(**{k: 0})) == -2, k
    assert ssd(good(batch=1 << 20, nheads=1 << 11)) == -2   # B*H >= 2^31
    assert ssd(good(seqlen=1 << 31)) == -2
    assert ssd(good(batch=1, nheads=1 << 17)) == -2         # H * P >= 2^23
    assert ssd(good(headdim=32)) == -4                      # built for P = 64, 128, 192, 256
    assert ssd(good(headdim=96)) == -4 and ssd(good(headdim=320)) == -4
    assert ssd(good(batch=1 << 20, nheads=1 << 10, headdim=128)) == -2  # B * H * P / 64 >= 2^31
    assert ssd(good(dstate=16)) == -4                       # built for N in {64, 128}
    for n in ("x", "dt", "A", "Bm", "Cm", "y"):
        assert ssd(good(), **{n: None}) == -1, n
    for n in ("x", "dt", "A", "Bm", "Cm", "Dskip", "dt_bias", "h0", "y", "h_final"):
        assert ssd(good(), **{n: MIS}) == -5, n
    # few (batch, head) pairs: the sequence is cut into segments and scratch is required
    q = lambda **k: lib.mssm_ssd_fwd_workspace_bytes(ctypes.byref(good(**k)))  # noqa: E731
    need = q(seqlen=1000)  # 6 pairs, 16 chunks: 8 segments of 128 steps
    assert need == 6 * 8 * (64 * 64 + 1) * 4
    assert q(seqlen=1000, dtype=1) == need + 2 * 1000 * 3 * 64 * 4  # bf16: float32 outputs before the correction
    # a 128-channel head is two 64-channel sub-heads: 12 (batch, sub-head) pairs, 8 segments
    assert q(seqlen=1000, headdim=128) == 12 * 8 * (64 * 64 + 1) * 4
    assert q() == 0 and q(seqlen=1000, batch=64, nheads=2) == 0 and q(seqlen=1000, dstate=16) == 0
    assert ssd(good(seqlen=1000)) == -6
    assert ssd(good(seqlen=1000), ws=FAKE, wsb=need - 1) == -6
    assert ssd(good(seqlen=1000), ws=MIS, wsb=need) == -5


def test_ssd_training_pair_validation():
    """mssm_ssd_fwd_train / mssm_ssd_bwd_saved: the SSD calls' checks plus the
    context (required, aligned, at least mssm_ssd_ctx_bytes: the state
    entering every 64-step chunk and the final one); with time segments the
    training forward's scratch is the forward's plus each chunk's decay from
    its segment's start."""
    S = mssm.binding.SsdProblem
    good = lambda **k: S(**{**dict(batch=2, seqlen=100, nheads=3, headdim=64, dstate=64, dtype=0,  # noqa: E731
                                   delta_softplus=1), **k})
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    nctx = lib.mssm_ssd_ctx_bytes(ctypes.byref(good()))
    assert nctx == 2 * 3 * (2 + 1) * 64 * 64 * 4
    assert lib.mssm_ssd_ctx_bytes(ctypes.byref(good(headdim=128))) == 2 * nctx
    assert lib.mssm_ssd_ctx_bytes(ctypes.byref(good(dstate=16))) == 0
    assert lib.mssm_ssd_fwd_workspace_bytes(ctypes.byref(good(seqlen=1000))) > 0     # segments
    seg = lib.mssm_ssd_fwd_workspace_bytes(ctypes.byref(good(seqlen=1000)))
    assert lib.mssm_ssd_fwd_train_workspace_bytes(ctypes.byref(good(seqlen=1000))) == \
        (seg + 255) // 256 * 256 + 2 * 3 * 16 * 4  # 6 pairs, 16 chunks
    assert lib.mssm_ssd_fwd_train_workspace_bytes(ctypes.byref(good())) == 0  # no segments, no scratch
    nb = lib.mssm_ssd_bwd_workspace_bytes(ctypes.byref(good()))
    assert lib.mssm_ssd_bwd_saved_workspace_bytes(ctypes.byref(good())) == nb - 2 * 3 * 3 * 64 * 64 * 4

    def fwd_tr(p, ctx=FAKE, ctxb=1 << 40, x=FAKE):
        return lib.mssm_ssd_fwd_train(ctypes.byref(p) if p is not None else None, v(x), v(FAKE), v(FAKE), v(FAKE),
                                      v(FAKE), None, None, None, v(FAKE), None, v(ctx), ctxb, None, 0, None)

    def bwd_sv(p, ctx=FAKE, ctxb=1 << 40, ws=FAKE, wsb=1 << 40, dy=FAKE):
        return lib.mssm_ssd_bwd_saved(ctypes.byref(p) if p is not None else None, v(FAKE), v(FAKE), v(FAKE),
                                      v(FAKE), v(FAKE), None, None, v(ctx), ctxb, v(dy), None, v(FAKE), v(FAKE),
                                      v(FAKE), v(FAKE), v(FAKE), None, None, None, v(ws), wsb, None)
    for call in (fwd_tr, bwd_sv):
        assert call(None) == -1
        assert call(good(dstate=16)) == -4
        assert call(good(), ctx=None) == -1
        assert call(good(), ctx=MIS) == -5
        assert call(good(), ctxb=nctx - 1) == -6
    assert fwd_tr(good(), x=None) == -1
    assert bwd_sv(good(), dy=None) == -1
    assert bwd_sv(good(), ws=None) == -6


def test_workspace_sizes_and_checks():
    tiny = good(1, 64, 32, 16)
    assert lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(tiny)) == 0
    long_ = P(1, 1 << 20, 1536, 16, 1, 1)
    nws = lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(long_))
    assert nws > 0
    # undersized or missing workspace is rejected before anything runs
    assert fwd(long_, ws=None, wsb=0) == -6
    assert fwd(long_, ws=FAKE, wsb=nws - 1) == -6
    nbw = lib.mssm_scan_bwd_workspace_bytes(ctypes.byref(good()))
    assert nbw > 0
    assert bwd(good(), ws=None) == -6
    assert bwd(good(), ws=FAKE, wsb=nbw - 1) == -6
    # invalid problems report no workspace
    assert lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(good(N=65))) == 0
    assert lib.mssm_scan_bwd_workspace_bytes(None) == 0


def fwd_train(p, ctx=FAKE, ctxb=1 << 40, ws=FAKE, wsb=1 << 40, **kw):
    pp = ctypes.byref(p) if p is not None else None
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    a = dict(u=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dskip=None, z=None, dt_bias=None, h0=None, y=FAKE,
             hf=None)
    a.update(kw)
    return lib.mssm_scan_fwd_train(pp, *(v(a[k]) for k in ("u", "delta", "A", "Bm", "Cm", "Dskip", "z", "dt_bias",
                                                            "h0", "y", "hf")), v(ctx), ctxb, v(ws), wsb, None)


def bwd_saved(p, ctx=FAKE, ctxb=1 << 40, ws=FAKE, wsb=1 << 40, **kw):
    pp = ctypes.byref(p) if p is not None else None
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    a = dict(u=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dskip=None, z=None, dt_bias=None, dy=FAKE, dhf=None,
             du=FAKE, ddelta=FAKE, dA=FAKE, dB=FAKE, dC=FAKE, dD=None, dz=None, ddt_bias=None, dh0=None)
    a.update(kw)
    head = [v(a[k]) for k in ("u", "delta", "A", "Bm", "Cm", "Dskip", "z", "dt_bias")]
    tail = [v(a[k]) for k in ("dy", "dhf", "du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dh0")]
    return lib.mssm_scan_bwd_saved(pp, *head, v(ctx), ctxb, *tail, v(ws), wsb, None)


def test_training_pair_validation():
    """mssm_scan_fwd_train / mssm_scan_bwd_saved: the forward's and backward's
    checks, plus the context: required, at least mssm_scan_ctx_bytes, aligned
    (a state size that is not a power of two has its next power's context)."""
    p = good(2, 100, 70, 16)
    nctx = lib.mssm_scan_ctx_bytes(ctypes.byref(p))
    tiles = (100 + 15) // 16
    assert nctx >= 2 * tiles * 16 * 70 * 4 + 2 * 100 * 70 * 4
    # any state size up to 64: one that is not a power of two has the context of the next power of two
    assert lib.mssm_scan_ctx_bytes(ctypes.byref(good(2, 100, 70, 12))) == nctx
    assert lib.mssm_scan_ctx_bytes(ctypes.byref(good(N=65))) == 0
    assert lib.mssm_scan_ctx_bytes(None) == 0
    nws = lib.mssm_scan_bwd_saved_workspace_bytes(ctypes.byref(p))
    assert 0 < nws < lib.mssm_scan_bwd_workspace_bytes(ctypes.byref(p))  # no pre-pass scratch
    assert lib.mssm_scan_bwd_saved_workspace_bytes(ctypes.byref(good(2, 100, 70, 12))) > nws  # + padded copies
    for call in (fwd_train, bwd_saved):
        assert call(None) == -1
        assert call(good(N=65)) == -4
        assert call(p, ctx=None) == -1
        assert call(p, ctx=MIS) == -5
        assert call(p, ctxb=nctx - 1) == -6
        assert call(p, u=None) == -1
        assert call(p, A=MIS) == -5
        bad = good(2, 100, 70, 16)
        bad.dtype = 7
        assert call(bad) == -3
    long_ = P(1, 1 << 20, 1536, 16, 1, 1)
    nf = lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(long_))
    assert fwd_train(long_, ws=FAKE, wsb=nf - 1) == -6
    # the conv front end's training forward: mssm_conv_scan_fwd's checks plus the context's
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731

    def conv_train(pp, K=4, x=FAKE, w=FAKE, ctx=FAKE, ctxb=1 << 40, ws=FAKE, wsb=1 << 40):
        return lib.mssm_conv_scan_fwd_train(ctypes.byref(pp) if pp is not None else None, K, v(x), v(w), None, None,
                                            v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, None, None, None, v(FAKE),
                                            None, None, v(ctx), ctxb, v(ws), wsb, None)
    assert conv_train(None) == -1
    assert conv_train(p, K=5) == -2
    assert conv_train(good(N=65)) == -4
    assert conv_train(p, w=None) == -1
    assert conv_train(p, ctx=None) == -1
    assert conv_train(p, ctx=MIS) == -5
    assert conv_train(p, ctxb=nctx - 1) == -6
    assert conv_train(long_, wsb=nf - 1) == -6
    assert bwd_saved(p, ws=None) == -6
    assert bwd_saved(p, wsb=nws - 1) == -6
    assert bwd_saved(p, dy=None) == -1
    assert bwd_saved(p, z=FAKE, dz=None) == -1
    assert bwd_saved(p, dC=None) == -1


def fwd_noalloc(p, u=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dskip=None, z=None, dt_bias=None, h0=None,
                y=FAKE, hf=None):
    pp = ctypes.byref(p) if p is not None else None
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.mssm_scan_fwd_noalloc(pp, v(u), v(delta), v(A), v(Bm), v(Cm), v(Dskip), v(z), v(dt_bias), v(h0),
                                     v(y), v(hf), None)


def test_noalloc_forward_validation():
    """mssm_scan_fwd_noalloc: the forward's checks, then the fixed scratch's
    limit -- all on the host, before the scratch array is looked up."""
    assert fwd_noalloc(None) == -1
    assert fwd_noalloc(good(dtype=3)) == -3
    assert fwd_noalloc(good(L=0)) == -2
    assert fwd_noalloc(good(N=80)) == -4
    for k in ("u", "delta", "A", "Bm", "Cm", "y"):
        assert fwd_noalloc(good(), **{k: None}) == -1, k
    for k in ("u", "Dskip", "h0", "y", "hf"):
        assert fwd_noalloc(good(), **{k: MIS}) == -5, k
    limit = 32 << 20
    # 8,192 channel blocks at dstate 64: the balanced schedule's published states alone take 128 MiB
    big = P(64, 4096, 8192, 64, 1, 1)
    assert lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(big)) > limit
    assert fwd_noalloc(big) == -6
    # the largest time-chunked plans (1M steps, dstate 64) fit
    for prob in (P(1, 1 << 20, 1536, 64, 1, 1), P(2, 1 << 20, 1536, 64, 0, 1), P(1, 1 << 20, 3072, 64, 1, 1)):
        assert 0 < lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(prob)) <= limit


def test_binding_rejects_cpu_tensors_and_bad_shapes():
    import torch
    u = torch.zeros(1, 8, 4)
    A = torch.zeros(4, 16)
    Bm = torch.zeros(1, 8, 16)
    with pytest.raises(ValueError):
        mssm.scan_fwd(u, u, A, Bm, Bm)          # CPU tensors: no fallback path exists
    with pytest.raises(ValueError):
        mssm.conv_scan_fwd(u, torch.zeros(4, 4), u, A, Bm, Bm)
    with pytest.raises(ValueError):
        mssm.conv_scan_fwd(u, torch.zeros(4, 5), u, A, Bm, Bm)   # d_conv 5 > the widest built
    with pytest.raises(TypeError):
        mssm.binding._dtype_code(torch.zeros(1, dtype=torch.float16))


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "selective_state_space_mssm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in src and "liboracle" not in src and "oracle_" not in src, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            src = open(os.path.join(ROOT, "oracle", f), encoding="utf-8").read()
            assert not re.search(r"^\s*(import|from)\s+selective_state_space_mssm_amd", src, re.M), f
            assert '#include "mssm.h"' not in src and "libmssm" not in src, f
