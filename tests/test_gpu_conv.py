"""GPU parity of the forward behind the fused causal conv1d + SiLU front end
(mssm_conv_scan_fwd) against the float64 oracle (oracle.conv_scan_fwd: the
convolution written out tap by tap, SiLU, then the sequential scan).

u = silu(conv(x)) is formed inside the kernels; with u_out requested it is
also compared, and the unfused scan run on that u must give the same y."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, fwd_err, gpu_inputs, to_np

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
    assert fwd_err(to_np(hf), hr) <= tol
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


def test_full_size_2p8b_sampled(mssm):
    """The Mamba-2.8B layer shape (B=4, L=4096, D=5120, bf16) in the launch
    configuration of the benchmark, checked on a sample of channels (first,
    last, and spread over the blocks) against the oracle on those channels."""
    w = workloads.WORKLOADS["2.8b"]
    inp, t = make(w, 4)
    print(f"[conv] {w} full size", flush=True)
    y, hf, u = gpu_run(mssm, t)
    torch.cuda.synchronize()
    ch = np.unique(np.concatenate([[0, 63, 64, 5119], np.random.default_rng(5).choice(w.D, 44, replace=False)]))
    sub = workloads.select_channels(inp, ch)
    yr, hr, ur = oracle_run(sub)
    cht = torch.from_numpy(ch).cuda()
    check((y[:, :, cht], hf[:, cht], u[:, :, cht]), (yr, hr, ur), "bf16")
