"""GPU parity of the forward behind the fused causal conv1d + SiLU front end
(mssm_conv_scan_fwd) against the float64 oracle (oracle.conv_scan_fwd: the
convolution written out tap by tap, SiLU, then the sequential scan).

u = silu(conv(x)) is formed inside the kernels; with u_out requested it is
also compared, and the unfused scan run on that u must give the same y."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, STATE_TOL, fwd_err, gpu_inputs, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mssm():
    import selective_state_space_mssm_amd as m
    return m


def make(w, K):
    inp = workloads.make_inputs(w)
    inp.update(workloads.conv_front_end(w, K))
    return inp, gpu_inputs(inp)


def gpu_run(mssm, t, use=("x_prev", "conv_b", "z", "Dskip", "dt_bias"), h0=None, want_u=True, **kw):
    g = lambda k: t[k] if k in use else None  # noqa: E731
    return mssm.conv_scan_fwd(t["u"], t["conv_w"], t["delta"], t["A"], t["Bm"], t["Cm"], g("Dskip"), g("z"),
                              g("dt_bias"), h0, conv_b=g("conv_b"), x_prev=g("x_prev"), return_u=want_u, **kw)


def oracle_run(inp, use=("x_prev", "conv_b", "z", "Dskip", "dt_bias"), h0=None):
    f = workloads.as_float32(inp)
    g = lambda k: f[k] if k in use else None  # noqa: E731
    return oracle.conv_scan_fwd(f["u"], f["conv_w"], f["delta"], f["A"], f["Bm"], f["Cm"], g("Dskip"), g("z"),
                                g("dt_bias"), h0, bias=g("conv_b"), x_prev=g("x_prev"))


def check(out, ref, dtype, with_u=True):
    y, hf, u = out
    yr, hr, ur = ref
    tol = FWD_TOL[dtype]
    assert fwd_err(to_np(y), yr) <= tol
    assert fwd_err(to_np(hf), hr) <= STATE_TOL
    if with_u:
        assert fwd_err(to_np(u), ur) <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 4, 64])
@pytest.mark.parametrize("K", [4, 3, 1])
def test_parity(mssm, dtype, N, K):
    # 77 steps: four full 16-step tiles and a ragged one; 100 channels: a ragged second block
    w = workloads.custom(2, 77, 100, N, dtype, seed=70 + N + K)
    print(f"[conv] {w} d_conv={K}", flush=True)
    inp, t = make(w, K)
    h0 = np.random.default_rng(K).standard_normal((w.B, w.D, N)).astype(np.float32)
    out = gpu_run(mssm, t, h0=torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    check(out, oracle_run(inp, h0=h0), dtype)


@pytest.mark.parametrize("N", [1, 2, 8, 32])
def test_other_state_sizes(mssm, N):
    # every other layout the forward dispatches (1, 2, 8, 32 states), bf16, d_conv = 4
    w = workloads.custom(2, 50, 130, N, "bf16", seed=170 + N)
    print(f"[conv] {w}", flush=True)
    inp, t = make(w, 4)
    check(gpu_run(mssm, t), oracle_run(inp), "bf16")


@pytest.mark.parametrize("use", [(), ("z",), ("x_prev",), ("conv_b", "Dskip"), ("dt_bias", "z", "conv_b")])
def test_optional_inputs(mssm, use):
    w = workloads.custom(1, 40, 70, 16, "f32", seed=80)
    print(f"[conv] {w} with {use}", flush=True)
    inp, t = make(w, 4)
    out = gpu_run(mssm, t, use=use)
    check(out, oracle_run(inp, use=use), "f32")


def test_short_sequences_reach_into_the_history(mssm):
    # L < d_conv - 1 and L = 1: every output row mixes x_prev and x
    for L in (1, 2, 3, 5):
        w = workloads.custom(2, L, 64, 16, "f32", seed=90 + L)
        print(f"[conv] {w}", flush=True)
        inp, t = make(w, 4)
        check(gpu_run(mssm, t), oracle_run(inp), "f32")


@pytest.mark.parametrize("B,L,D,N,dtype,K", [
    (5, 40, 4096, 16, "bf16", 4),    # 320 channel blocks: the balanced persistent schedule (split blocks)
    (1, 4200, 128, 16, "f32", 4),    # 2 blocks, long: time chunks (chunk-state kernel with the front end)
    (1, 2100, 64, 4, "f32", 2),
])
def test_schedules(mssm, B, L, D, N, dtype, K):
    w = workloads.custom(B, L, D, N, dtype, seed=100 + K)
    print(f"[conv] {w} d_conv={K}", flush=True)
    inp, t = make(w, K)
    out = gpu_run(mssm, t)
    torch.cuda.synchronize()
    check(out, oracle_run(inp), dtype)


def test_streaming_in_place(mssm):
    """Consecutive calls, each given the previous inputs' last d_conv - 1 rows
    as x_prev and the state in place (h0 == h_final), equal one call."""
    w = workloads.custom(2, 2200, 128, 16, "f32", seed=110)
    inp, t = make(w, 4)
    print(f"[conv] {w} streamed", flush=True)
    state = torch.zeros((w.B, w.D, 16), device="cuda")
    hist = t["x_prev"]
    ys, t0 = [], 0
    for n in (1, 2, 37, 2100, 60):
        sl = slice(t0, t0 + n)
        x = t["u"][:, sl].contiguous()
        y, hf, _ = mssm.conv_scan_fwd(x, t["conv_w"], t["delta"][:, sl].contiguous(), t["A"],
                                      t["Bm"][:, sl].contiguous(), t["Cm"][:, sl].contiguous(), t["Dskip"],
                                      t["z"][:, sl].contiguous(), t["dt_bias"], state, conv_b=t["conv_b"],
                                      x_prev=hist, h_final=state)
        assert hf is state
        ys.append(y)
        hist = torch.cat([hist, x], 1)[:, -3:].contiguous()
        t0 += n
    torch.cuda.synchronize()
    yr, hr, _ = oracle_run(inp)
    assert fwd_err(to_np(torch.cat(ys, 1)), yr) <= FWD_TOL["f32"]
    assert fwd_err(to_np(state), hr) <= FWD_TOL["f32"]


def test_fused_equals_unfused_scan_of_its_u(mssm):
    """float32: the fused front end feeds the scan exactly the u it reports,
    so the plain scan of that u gives bitwise the same y and final state."""
    w = workloads.custom(3, 300, 200, 16, "f32", seed=120)
    inp, t = make(w, 4)
    y, hf, u = gpu_run(mssm, t)
    y2, hf2 = mssm.scan_fwd(u, t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"])
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.equal(hf, hf2)


def test_full_size_2p8b(mssm):
    """The Mamba-2.8B layer shape (B=4, L=4096, D=5120, bf16) in the launch
    configuration of the benchmark: every element of y, h_final and u against
    the oracle."""
    w = workloads.WORKLOADS["2.8b"]
    inp, t = make(w, 4)
    print(f"[conv] {w} full size", flush=True)
    y, hf, u = gpu_run(mssm, t)
    torch.cuda.synchronize()
    out = (to_np(y), to_np(hf), to_np(u))
    del y, hf, u, t
    torch.cuda.empty_cache()
    yr, hr, ur = oracle_run(inp)
    print(f"2.8b conv: y err {fwd_err(out[0], yr):.2e}, h_final err {fwd_err(out[1], hr):.2e}, "
          f"u err {fwd_err(out[2], ur):.2e}", flush=True)
    check(out, (yr, hr, ur), "bf16")


# ---- backward of the front end (mssm_conv_bwd) --------------------------------------------------

from helpers import GRAD_TOL, grad_err  # noqa: E402


def conv_bwd_case(mssm, B, L, D, dtype, K, use=("x_prev", "conv_b"), seed=0):
    w = workloads.custom(B, L, D, 16, dtype, seed=seed)
    inp, t = make(w, K)
    du_np = np.random.default_rng(seed + 1).standard_normal((B, L, D)).astype(np.float32)
    du_st = workloads.bf16_bits(du_np) if dtype == "bf16" else du_np
    du = workloads.to_torch({"u": du_st, "dtype": dtype}, "cuda", keys=("u",))["u"]
    xp = t["x_prev"] if "x_prev" in use else None
    g = mssm.conv_bwd(t["u"], t["conv_w"], du, conv_b=t["conv_b"] if "conv_b" in use else None, x_prev=xp,
                      want_dx_prev=K > 1)
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    r = oracle.causal_conv_silu_bwd(f["u"], f["conv_w"], workloads.to_f32(du_st, dtype),
                                    f["conv_b"] if "conv_b" in use else None, f["x_prev"] if "x_prev" in use else None)
    return g, r


def check_conv_grads(g, r, dtype, K):
    tol = GRAD_TOL[dtype]
    assert grad_err(to_np(g["dx"]), r["dx"]) <= tol
    assert grad_err(to_np(g["dconv_w"]), r["dweight"]) <= tol
    if g["dconv_b"] is not None:
        assert grad_err(to_np(g["dconv_b"]), r["dbias"]) <= tol
    if K > 1:
        assert grad_err(to_np(g["dx_prev"]), r["dx_prev"]) <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [4, 3, 2, 1])
def test_conv_backward_parity(mssm, dtype, K):
    # 300 channels: a ragged second block of 256; 200 steps: four 64-step chunks, the last one short
    print(f"[conv bwd] dtype={dtype} d_conv={K}", flush=True)
    g, r = conv_bwd_case(mssm, 2, 200, 300, dtype, K, seed=130 + K)
    check_conv_grads(g, r, dtype, K)


@pytest.mark.parametrize("use", [(), ("x_prev",), ("conv_b",)])
def test_conv_backward_optional_inputs(mssm, use):
    print(f"[conv bwd] with {use}", flush=True)
    g, r = conv_bwd_case(mssm, 1, 70, 64, "f32", 4, use=use, seed=140)
    check_conv_grads(g, r, "f32", 4)


@pytest.mark.parametrize("B,L,D", [(1, 3, 40), (3, 1, 64), (1, 70000, 64), (2, 100, 77)])
def test_conv_backward_edge_shapes(mssm, B, L, D):
    # shorter than the window; a single step; long chunks (70,000 steps: 69 per chunk, 1,015 chunks);
    # an odd channel count (one channel per thread instead of pairs)
    print(f"[conv bwd] B={B} L={L} D={D}", flush=True)
    g, r = conv_bwd_case(mssm, B, L, D, "f32", 4, seed=150)
    check_conv_grads(g, r, "f32", 4)


def test_conv_backward_full_size_2p8b(mssm):
    """The 2.8B layer shape (B=4, L=4096, D=5120, bf16): every element of dx,
    dconv_w, dconv_b and dx_prev against the oracle."""
    w = workloads.WORKLOADS["2.8b"]
    inp, t = make(w, 4)
    print(f"[conv bwd] {w} full size", flush=True)
    du_st = workloads.bf16_bits(np.random.default_rng(7).standard_normal((w.B, w.L, w.D)).astype(np.float32))
    du = workloads.to_torch({"u": du_st, "dtype": "bf16"}, "cuda", keys=("u",))["u"]
    g = mssm.conv_bwd(t["u"], t["conv_w"], du, conv_b=t["conv_b"], x_prev=t["x_prev"], want_dx_prev=True)
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    r = oracle.causal_conv_silu_bwd(f["u"], f["conv_w"], workloads.to_f32(du_st, "bf16"), f["conv_b"], f["x_prev"])
    check_conv_grads(g, r, "bf16", 4)


def test_training_chain_through_the_front_end(mssm):
    """Forward with the fused front end (u_out), the scan's backward on that
    u, then the front end's backward: every gradient against the oracle's
    chain (conv + SiLU, scan adjoint, conv adjoint)."""
    w = workloads.custom(2, 150, 130, 16, "f32", seed=160, backward=True)
    inp, t = make(w, 4)
    print(f"[conv chain] {w}", flush=True)
    y, hf, u = gpu_run(mssm, t)
    gs = mssm.scan_bwd(u, t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["z"], t["dt_bias"])
    gc = mssm.conv_bwd(t["u"], t["conv_w"], gs["du"], conv_b=t["conv_b"], x_prev=t["x_prev"], want_dx_prev=True)
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    ur = oracle.causal_conv_silu(f["u"], f["conv_w"], f["conv_b"], f["x_prev"])
    rs = oracle.scan_bwd(ur, f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], f["Dskip"], f["z"], f["dt_bias"])
    rc = oracle.causal_conv_silu_bwd(f["u"], f["conv_w"], rs["du"], f["conv_b"], f["x_prev"])
    for k in ("ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias"):
        assert grad_err(to_np(gs[k]), rs[k]) <= GRAD_TOL["f32"], k
    check_conv_grads(gc, rc, "f32", 4)


@pytest.mark.parametrize("shape,dtype,K", [((2, 150, 130), "f32", 4), ((2, 150, 130), "bf16", 3),
                                           ((1, 600, 100), "f32", 4), ((3, 48, 5760), "f32", 2)])
def test_training_pair_through_the_front_end(mssm, shape, dtype, K):
    """The training pair behind the front end: mssm_conv_scan_fwd_train (y,
    h_final and u bit for bit those of mssm_conv_scan_fwd; it also saves the
    context), mssm_scan_bwd_saved on its u, mssm_conv_bwd on that du: every
    gradient against the oracle's chain.  (1, 600, 100): the time-chunked
    forward; (3, 48, 5760): 270 channel blocks, the balanced schedule."""
    B, L, D = shape
    w = workloads.custom(B, L, D, 16, dtype, seed=L + D + K, backward=True)
    inp, t = make(w, K)
    print(f"[conv train pair] {w} d_conv={K}", flush=True)
    xp = t["x_prev"] if K > 1 else None
    y, hf, u, ctx = mssm.conv_scan_fwd_train(t["u"], t["conv_w"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"],
                                             t["z"], t["dt_bias"], conv_b=t["conv_b"], x_prev=xp)
    y0, hf0, u0 = mssm.conv_scan_fwd(t["u"], t["conv_w"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"],
                                     t["dt_bias"], conv_b=t["conv_b"], x_prev=xp, return_u=True)
    assert torch.equal(y, y0) and torch.equal(hf, hf0) and torch.equal(u, u0)
    gs = mssm.scan_bwd_saved(u, t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx, t["Dskip"], t["z"], t["dt_bias"])
    gc = mssm.conv_bwd(t["u"], t["conv_w"], gs["du"], conv_b=t["conv_b"], x_prev=xp, want_dx_prev=K > 1)
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    fxp = f["x_prev"] if K > 1 else None
    ur = oracle.causal_conv_silu(f["u"], f["conv_w"], f["conv_b"], fxp)
    rs = oracle.scan_bwd(ur, f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], f["Dskip"], f["z"], f["dt_bias"])
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dh0"):
        assert grad_err(to_np(gs[k]), rs[k]) <= GRAD_TOL[dtype], k
    # the front end's backward against the oracle's on the du it was given: with bfloat16 activations du is
    # rounded to bfloat16 before it, and the rounding of du and then of dx compounds beyond one rounding's bar
    du_in = rs["du"] if dtype == "f32" else to_np(gs["du"]).astype(np.float64)
    rc = oracle.causal_conv_silu_bwd(f["u"], f["conv_w"], du_in, f["conv_b"], fxp)
    check_conv_grads(gc, rc, dtype, K)


# ---- decode through the front end (mssm_conv_step) ----------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,K", [(16, 4), (4, 3), (64, 2), (2, 4), (16, 1)])
def test_conv_step_decode(mssm, dtype, N, K):
    """Token by token through mssm_conv_step equals the oracle's one scan
    behind the conv over the whole sequence; the conv state ends as the last
    d_conv - 1 inputs (exactly: it only moves stored values)."""
    w = workloads.custom(3, 24, 100, N, dtype, seed=180 + N + K)
    inp, t = make(w, K)
    print(f"[conv step] {w} d_conv={K}", flush=True)
    h0 = np.random.default_rng(9).standard_normal((w.B, w.D, N)).astype(np.float32)
    state = torch.from_numpy(h0).cuda()
    cst = t["x_prev"].clone() if K > 1 else None
    ys = []
    for i in range(w.L):
        ys.append(mssm.conv_step(t["u"][:, i].contiguous(), t["conv_w"], cst, t["delta"][:, i].contiguous(), t["A"],
                                 t["Bm"][:, i].contiguous(), t["Cm"][:, i].contiguous(), state, t["Dskip"],
                                 t["z"][:, i].contiguous(), t["dt_bias"], conv_b=t["conv_b"]))
    torch.cuda.synchronize()
    yr, hr, _ = oracle_run(inp, h0=h0)
    tol = FWD_TOL[dtype]
    assert fwd_err(to_np(torch.stack(ys, 1)), yr) <= tol
    assert fwd_err(to_np(state), hr) <= STATE_TOL
    if K > 1:
        assert torch.equal(cst, torch.cat([t["x_prev"], t["u"]], 1)[:, -(K - 1):])


def test_prefill_then_decode(mssm):
    """A prefill with mssm_conv_scan_fwd (state in place), the conv state taken
    from its inputs, then decode steps: equal to one scan over all tokens."""
    w = workloads.custom(2, 40, 192, 16, "bf16", seed=190)
    inp, t = make(w, 4)
    print(f"[conv prefill+decode] {w}", flush=True)
    state = torch.zeros((w.B, w.D, 16), device="cuda")
    P = 30
    y0, _, _ = mssm.conv_scan_fwd(t["u"][:, :P].contiguous(), t["conv_w"], t["delta"][:, :P].contiguous(), t["A"],
                                  t["Bm"][:, :P].contiguous(), t["Cm"][:, :P].contiguous(), t["Dskip"],
                                  t["z"][:, :P].contiguous(), t["dt_bias"], state, conv_b=t["conv_b"],
                                  x_prev=t["x_prev"], h_final=state)
    cst = torch.cat([t["x_prev"], t["u"][:, :P]], 1)[:, -3:].contiguous()
    ys = [y0]
    for i in range(P, w.L):
        ys.append(mssm.conv_step(t["u"][:, i].contiguous(), t["conv_w"], cst, t["delta"][:, i].contiguous(), t["A"],
                                 t["Bm"][:, i].contiguous(), t["Cm"][:, i].contiguous(), state, t["Dskip"],
                                 t["z"][:, i].contiguous(), t["dt_bias"], conv_b=t["conv_b"])[:, None])
    torch.cuda.synchronize()
    yr, hr, _ = oracle_run(inp)
    assert fwd_err(to_np(torch.cat(ys, 1)), yr) <= FWD_TOL["bf16"]
    assert fwd_err(to_np(state), hr) <= STATE_TOL
