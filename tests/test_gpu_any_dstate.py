"""GPU parity for state sizes that are not a power of two (3, 12, 24, 48):
forward (short-sequence path, tiled grid, time-chunked and balanced
schedules), backward, the fused conv front end, the decode step and its conv
form, and the forward without a workspace, against the float64 oracle (which
takes any N).  The library runs such N at the next power of two with the extra
states inert (A, Bm, Cm, h0 zero for them), so the results must be those of
the N-state scan: y at the activation type's bar, the float32 state at 1e-4,
gradients at 1e-3 (2e-2 for bfloat16)."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, GRAD_TOL, STATE_TOL, fwd_err, gpu_inputs, grad_err, run_oracle_fwd, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mssm():
    import selective_state_space_mssm_amd as m
    return m


def fwd_case(mssm, B, L, D, N, dtype, seed, noalloc=False):
    w = workloads.custom(B, L, D, N, dtype, seed=seed)
    print(f"[any N fwd] {w} noalloc={noalloc}", flush=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0 = np.random.default_rng(seed).standard_normal((B, D, N)).astype(np.float32)
    args = (t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"], torch.from_numpy(h0).cuda())
    y, hf = (mssm.scan_fwd_noalloc if noalloc else mssm.scan_fwd)(*args)
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, h0)
    assert fwd_err(to_np(y), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(hf), hr) <= STATE_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [3, 12, 24, 48])
def test_forward(mssm, N, dtype):
    fwd_case(mssm, 2, 37, 70, N, dtype, seed=N)          # short-sequence path
    fwd_case(mssm, 2, 133, 100, N, dtype, seed=N + 1)    # tiled grid, ragged tile and block
    fwd_case(mssm, 1, 700, 64, N, dtype, seed=N + 2)     # time chunks joined by the carry


def test_forward_balanced_schedule(mssm):
    fwd_case(mssm, 3, 90, 5760, 12, "bf16", seed=5)      # 270 channel blocks: balanced persistent schedule


def test_forward_in_place_state(mssm):
    """h_final the same buffer as h0 (the state advanced in place) with padding."""
    w = workloads.custom(2, 150, 96, 24, "f32", seed=8)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0 = np.random.default_rng(3).standard_normal((2, 96, 24)).astype(np.float32)
    st = torch.from_numpy(h0).cuda()
    y, hf = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"], st,
                          h_final=st)
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, h0)
    assert hf is st
    assert fwd_err(to_np(y), yr) <= FWD_TOL["f32"] and fwd_err(to_np(st), hr) <= STATE_TOL


@pytest.mark.parametrize("N", [12, 48])
def test_forward_noalloc(mssm, N):
    fwd_case(mssm, 2, 133, 100, N, "bf16", seed=N + 3, noalloc=True)
    fwd_case(mssm, 1, 20, 30, N, "f32", seed=N + 4, noalloc=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [3, 12, 48])
def test_backward(mssm, N, dtype):
    for (B, L, D) in ((2, 40, 70), (1, 300, 70)):   # one pass; reverse walk cut into time chunks
        w = workloads.custom(B, L, D, N, dtype, seed=N + L)
        print(f"[any N bwd] {w}", flush=True)
        inp = workloads.make_inputs(w, with_dy=True)
        t = gpu_inputs(inp)
        rng = np.random.default_rng(N)
        h0 = rng.standard_normal((B, D, N)).astype(np.float32)
        dhf = rng.standard_normal((B, D, N)).astype(np.float32)
        g = mssm.scan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["z"], t["dt_bias"],
                          torch.from_numpy(h0).cuda(), torch.from_numpy(dhf).cuda())
        torch.cuda.synchronize()
        f = workloads.as_float32(inp)
        r = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], Dskip=f["Dskip"], z=f["z"],
                            dt_bias=f["dt_bias"], h0=h0, dh_final=dhf)
        for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dh0"):
            assert tuple(g[k].shape) == r[k].shape, k
            assert grad_err(to_np(g[k]), r[k]) <= GRAD_TOL[dtype], k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [3, 12, 48])
def test_step(mssm, N, dtype):
    w = workloads.custom(3, 10, 100, N, dtype, seed=N + 30)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0 = np.random.default_rng(1).standard_normal((3, 100, N)).astype(np.float32)
    state = torch.from_numpy(h0).cuda()
    ys = [mssm.step(t["u"][:, i].contiguous(), t["delta"][:, i].contiguous(), t["A"], t["Bm"][:, i].contiguous(),
                    t["Cm"][:, i].contiguous(), state, t["Dskip"], t["z"][:, i].contiguous(), t["dt_bias"])
          for i in range(w.L)]
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, h0)
    assert fwd_err(to_np(torch.stack(ys, 1)), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(state), hr) <= STATE_TOL


@pytest.mark.parametrize("K", [4, 2, 1])
def test_conv_forward_and_step(mssm, K):
    """The fused conv front end at N = 12: the forward over 90 steps, and the
    same sequence token by token through the conv decode step."""
    N = 12
    w = workloads.custom(2, 90, 100, N, "f32", seed=K + 40)
    inp = workloads.make_inputs(w)
    inp.update(workloads.conv_front_end(w, K))
    t = gpu_inputs(inp)
    y, hf, u = mssm.conv_scan_fwd(t["u"], t["conv_w"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"],
                                  t["dt_bias"], None, conv_b=t["conv_b"], x_prev=t.get("x_prev"), return_u=True)
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    yr, hr, ur = oracle.conv_scan_fwd(f["u"], f["conv_w"], f["delta"], f["A"], f["Bm"], f["Cm"], f["Dskip"], f["z"],
                                      f["dt_bias"], None, bias=f["conv_b"], x_prev=f.get("x_prev"))
    assert fwd_err(to_np(y), yr) <= FWD_TOL["f32"] and fwd_err(to_np(hf), hr) <= STATE_TOL
    assert fwd_err(to_np(u), ur) <= FWD_TOL["f32"]
    state = torch.zeros((2, 100, N), device="cuda")
    cst = t["x_prev"].clone() if K > 1 else None
    ys = [mssm.conv_step(t["u"][:, i].contiguous(), t["conv_w"], cst, t["delta"][:, i].contiguous(), t["A"],
                         t["Bm"][:, i].contiguous(), t["Cm"][:, i].contiguous(), state, t["Dskip"],
                         t["z"][:, i].contiguous(), t["dt_bias"], conv_b=t["conv_b"]) for i in range(w.L)]
    torch.cuda.synchronize()
    assert fwd_err(to_np(torch.stack(ys, 1)), yr) <= FWD_TOL["f32"]
    assert fwd_err(to_np(state), hr) <= STATE_TOL
    if K > 1:
        assert torch.equal(cst, torch.cat([t["x_prev"], t["u"]], 1)[:, -(K - 1):])
