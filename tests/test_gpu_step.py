"""GPU parity of the recurrent step (mssm_step): one token at a time with the
state carried in place, against the float64 oracle's step and scan (the RNN
form / step function of the page "mamba.py: 一个简单高效的Mamba实现",
updates section)."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, STATE_TOL, fwd_err, gpu_inputs, run_oracle_fwd, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mssm():
    import selective_state_space_mssm_amd as m
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 4, 64, 2])
def test_steps_equal_scan(mssm, dtype, N):
    w = workloads.custom(3, 40, 100, N, dtype, seed=30 + N)
    print(f"[step] {w}", flush=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0 = np.random.default_rng(1).standard_normal((w.B, w.D, N)).astype(np.float32)
    state = torch.from_numpy(h0).cuda()
    ys = []
    for i in range(w.L):
        ys.append(mssm.step(t["u"][:, i].contiguous(), t["delta"][:, i].contiguous(), t["A"],
                            t["Bm"][:, i].contiguous(), t["Cm"][:, i].contiguous(), state,
                            t["Dskip"], t["z"][:, i].contiguous(), t["dt_bias"]))
    y = torch.stack(ys, 1)
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, h0)
    tol = FWD_TOL[dtype]
    assert fwd_err(to_np(y), yr) <= tol
    assert fwd_err(to_np(state), hr) <= STATE_TOL
    # and the GPU scan from the same state agrees with the GPU steps
    ysc, hsc = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"],
                             t["dt_bias"], torch.from_numpy(h0).cuda())
    assert fwd_err(to_np(ysc), to_np(y)) <= tol
    assert fwd_err(to_np(hsc), to_np(state)) <= STATE_TOL


def test_step_without_optional_inputs(mssm):
    w = workloads.custom(2, 6, 70, 16, "f32", seed=40)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    state = torch.zeros((2, 70, 16), device="cuda")
    ys = [mssm.step(t["u"][:, i].contiguous(), t["delta"][:, i].contiguous(), t["A"],
                    t["Bm"][:, i].contiguous(), t["Cm"][:, i].contiguous(), state) for i in range(6)]
    y = torch.stack(ys, 1)
    yr, hr = run_oracle_fwd(oracle, inp, None, use=())
    assert fwd_err(to_np(y), yr) <= 1e-4
    assert fwd_err(to_np(state), hr) <= 1e-4


def test_batched_decode_shape(mssm):
    # large-batch decode: B=256 sequences, D=1536 channels, one token
    w = workloads.custom(256, 1, 1536, 16, "bf16", seed=41)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0 = np.random.default_rng(2).standard_normal((256, 1536, 16)).astype(np.float32)
    state = torch.from_numpy(h0).cuda()
    y = mssm.step(t["u"][:, 0].contiguous(), t["delta"][:, 0].contiguous(), t["A"],
                  t["Bm"][:, 0].contiguous(), t["Cm"][:, 0].contiguous(), state, t["Dskip"],
                  t["z"][:, 0].contiguous(), t["dt_bias"])
    yr, hr = run_oracle_fwd(oracle, inp, h0)
    assert fwd_err(to_np(y), yr[:, 0]) <= FWD_TOL["bf16"]
    assert fwd_err(to_np(state), hr) <= 1e-5   # state stays float32


@pytest.mark.parametrize("B,D,segments,dtype", [
    (2, 100, [1, 3, 16, 17, 40], "f32"),          # one workgroup per channel block
    (5, 4096, [1, 16, 31], "bf16"),               # 320 blocks: the balanced persistent schedule
    (1, 128, [2100, 5, 2048], "f32"),             # few blocks, long segments: time chunks + carry
])
def test_multi_token_steps_in_place(mssm, B, D, segments, dtype):
    """The forward scan with h0 and h_final the same buffer advances the state
    in place: a chain of calls over consecutive segments equals one scan over
    the whole sequence (the oracle's)."""
    L = sum(segments)
    w = workloads.custom(B, L, D, 16, dtype, seed=60 + len(segments))
    print(f"[multi-token] {w} segments {segments}", flush=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0 = np.random.default_rng(3).standard_normal((B, D, 16)).astype(np.float32)
    state = torch.from_numpy(h0).cuda()
    ys, t0 = [], 0
    for n in segments:
        sl = slice(t0, t0 + n)
        y, hf = mssm.scan_fwd(t["u"][:, sl].contiguous(), t["delta"][:, sl].contiguous(), t["A"],
                              t["Bm"][:, sl].contiguous(), t["Cm"][:, sl].contiguous(), t["Dskip"],
                              t["z"][:, sl].contiguous(), t["dt_bias"], state, h_final=state)
        assert hf is state
        ys.append(y)
        t0 += n
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, h0)
    tol = FWD_TOL[dtype]
    assert fwd_err(to_np(torch.cat(ys, 1)), yr) <= tol
    assert fwd_err(to_np(state), hr) <= STATE_TOL


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_short_sequence_path(mssm, N, dtype):
    """Short sequences take the short path (the state in registers across the
    steps; here, over 260 (b, d) rows, up to 64 steps): against the oracle at
    lengths around the switch (1, 7, 64) and the tiled path just above it (65)."""
    for L in (1, 7, 64, 65):
        w = workloads.custom(2, L, 130, N, dtype, seed=200 + N + L)
        print(f"[short] {w}", flush=True)
        inp = workloads.make_inputs(w)
        t = gpu_inputs(inp)
        h0 = np.random.default_rng(L).standard_normal((w.B, w.D, N)).astype(np.float32)
        y, hf = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"],
                              torch.from_numpy(h0).cuda())
        torch.cuda.synchronize()
        yr, hr = run_oracle_fwd(oracle, inp, h0)
        tol = FWD_TOL[dtype]
        assert fwd_err(to_np(y), yr) <= tol
        assert fwd_err(to_np(hf), hr) <= STATE_TOL


@pytest.mark.parametrize("use,softplus", [((), True), (("z",), False), (("Dskip", "dt_bias"), True)])
def test_short_sequence_optional_inputs(mssm, use, softplus):
    # 20 steps over 600 (b, d) rows: the short path
    w = workloads.custom(3, 20, 200, 16, "f32", seed=210)
    inp = workloads.make_inputs(w)
    if not softplus:  # flag off: Delta used as is; keep it a positive step so the recurrence stays contractive
        inp["delta"] = (0.05 * np.abs(inp["delta"])).astype(np.float32)
    t = gpu_inputs(inp)
    y, hf = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"] if "Dskip" in use else None,
                          t["z"] if "z" in use else None, t["dt_bias"] if "dt_bias" in use else None, None,
                          delta_softplus=softplus)
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, None, use=use, softplus=softplus)
    assert fwd_err(to_np(y), yr) <= FWD_TOL["f32"]
    assert fwd_err(to_np(hf), hr) <= FWD_TOL["f32"]


def test_short_path_many_rows(mssm):
    """Up to 8 steps the short path runs at any row count: 64 x 1,536 rows, 1
    and 8 steps, against the oracle; 9 steps take the tiled kernel."""
    for L in (1, 8, 9):
        w = workloads.custom(64, L, 1536, 16, "bf16", seed=220 + L)
        print(f"[short] {w}", flush=True)
        inp = workloads.make_inputs(w)
        t = gpu_inputs(inp)
        y, hf = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"])
        torch.cuda.synchronize()
        yr, hr = run_oracle_fwd(oracle, inp)
        assert fwd_err(to_np(y), yr) <= FWD_TOL["bf16"]
        assert fwd_err(to_np(hf), hr) <= STATE_TOL


@pytest.mark.parametrize("shape,dtype", [((2, 20, 2048), "bf16"), ((1, 33, 4097), "f32"), ((1, 64, 32), "f32"),
                                         ((3, 17, 5), "bf16"), ((1, 9, 64), "f32")])
def test_short_path_few_rows(mssm, shape, dtype):
    """Few (b, d) rows (at most 4,096) over 9 to 64 steps: the short path loads
    16 tokens' inputs at a time (here 1, 2, 3 or 4 groups of 16, the last one
    partial); 4,097 rows keep the one-token prefetch."""
    B, L, D = shape
    w = workloads.custom(B, L, D, 16, dtype, seed=230 + L + D)
    print(f"[short few rows] {w}", flush=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0 = np.random.default_rng(D).standard_normal((B, D, 16)).astype(np.float32)
    y, hf = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"],
                          torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, h0)
    assert fwd_err(to_np(y), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(hf), hr) <= STATE_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stepper_over_bound_buffers_and_in_a_graph(mssm, dtype):
    # Stepper: the step over buffers bound once, each token's inputs copied into them in place.  Eager calls
    # equal step(); a captured graph of 4 steps over the bound buffers, replayed 3 times (new inputs each time)
    # with eager work and checks between replays, equals 4 eager steps from the same state, bit for bit
    w = workloads.custom(4, 16, 96, 16, dtype, seed=91)
    print(f"[stepper] {w}", flush=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    tok = lambda k, i: t[k][:, i].contiguous()  # noqa: E731
    ref_state = torch.zeros((w.B, w.D, w.N), device="cuda")
    ref = [mssm.step(tok("u", i), tok("delta", i), t["A"], tok("Bm", i), tok("Cm", i), ref_state, t["Dskip"],
                     tok("z", i), t["dt_bias"]).clone() for i in range(4)]
    bufs = {k: torch.empty_like(tok(k, 0)) for k in ("u", "delta", "Bm", "Cm", "z")}
    state = torch.zeros((w.B, w.D, w.N), device="cuda")

    def feed(i):
        for k, b in bufs.items():
            b.copy_(tok(k, i))

    def bound():
        return mssm.Stepper(bufs["u"], bufs["delta"], t["A"], bufs["Bm"], bufs["Cm"], state, t["Dskip"],
                            bufs["z"], t["dt_bias"])

    st = bound()
    for i in range(4):
        feed(i)
        assert torch.equal(st(), ref[i]), i
    assert torch.equal(state, ref_state)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    outs = [torch.empty_like(ref[0]) for _ in range(4)]
    with torch.cuda.graph(g, stream=side):
        gs = bound()  # binds the capture stream
        for j in range(4):
            outs[j].copy_(gs())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        feed(4 + r)
        check_state = state.clone()
        check = [mssm.step(bufs["u"], bufs["delta"], t["A"], bufs["Bm"], bufs["Cm"], check_state, t["Dskip"],
                           bufs["z"], t["dt_bias"]).clone() for _ in range(4)]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j in range(4):
            assert torch.equal(outs[j], check[j]), (r, j)
        assert torch.equal(state, check_state), r
