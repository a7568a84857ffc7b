"""GPU test of mssm_scan_fwd_noalloc, the forward for callers that cannot
allocate: through the C ABI it must give exactly (bit for bit) what
mssm_scan_fwd gives with a workspace of its own, call after call, whatever an
earlier call left in the shared scratch array -- each sequence below runs a
larger problem first and smaller ones after it -- and agree with the float64
oracle at the usual bars."""
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


def run_pair(mssm, w, h0=True, with_oracle=False):
    print(f"[noalloc] {w}", flush=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0n = np.random.default_rng(w.seed).standard_normal((w.B, w.D, w.N)).astype(np.float32) if h0 else None
    h0t = torch.from_numpy(h0n).cuda() if h0 else None
    args = (t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"], h0t)
    y_ref, h_ref = mssm.scan_fwd(*args)
    y = torch.full_like(y_ref, float("nan"))
    hf = torch.full_like(h_ref, float("nan"))
    y2, hf2 = mssm.scan_fwd_noalloc(*args, y=y, h_final=hf)
    torch.cuda.synchronize()
    assert y2 is y and hf2 is hf
    assert torch.equal(y, y_ref), "y differs from mssm_scan_fwd's"
    assert torch.equal(hf, h_ref), "h_final differs from mssm_scan_fwd's"
    if with_oracle:
        yr, hr = run_oracle_fwd(oracle, inp, h0n)
        assert fwd_err(to_np(y), yr) <= FWD_TOL[w.dtype]
        assert fwd_err(to_np(hf), hr) <= STATE_TOL


def test_larger_then_smaller_balanced_first(mssm):
    # 270 channel blocks on a 256-CU GPU: the balanced schedule's hand-over
    # flags and published states in the scratch; then 260 blocks (fewer flags,
    # the first ones still set by the previous call); then one block of 5,000
    # steps, time-chunked, its chunk states over the same bytes; then a plain
    # grid that uses no scratch at all
    run_pair(mssm, workloads.custom(3, 333, 5760, 16, "bf16", seed=1), with_oracle=True)
    run_pair(mssm, workloads.custom(4, 101, 4160, 16, "f32", seed=2))
    run_pair(mssm, workloads.custom(1, 5000, 40, 16, "f32", seed=3), with_oracle=True)
    run_pair(mssm, workloads.custom(2, 100, 70, 16, "f32", seed=4), h0=False)


def test_larger_then_smaller_chunked_first(mssm):
    # 2 blocks of 20,000 steps (19 chunks), then 1 block of 2,100 steps in
    # bf16, then the balanced schedule over what the chunk states left
    run_pair(mssm, workloads.custom(1, 20000, 128, 16, "f32", seed=5), with_oracle=True)
    run_pair(mssm, workloads.custom(1, 2100, 40, 64, "bf16", seed=6), with_oracle=True)
    run_pair(mssm, workloads.custom(3, 104, 5760, 8, "bf16", seed=7))


def test_repeated_calls_same_problem(mssm):
    # the same problem twice in a row (flags left set by the first call)
    w = workloads.custom(5, 100, 3840, 16, "f32", seed=8)
    run_pair(mssm, w)
    run_pair(mssm, w)


def test_too_large_rejected(mssm):
    # a problem whose scratch exceeds the fixed array is refused before anything runs
    w = workloads.custom(2, 70, 1 << 20, 64, "bf16", seed=9)   # 32,768 channel blocks at dstate 64
    assert mssm.fwd_workspace_bytes(w.B, w.L, w.D, w.N, torch.bfloat16) > (32 << 20)
    u = torch.zeros((w.B, w.L, w.D), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((w.D, w.N), device="cuda")
    bc = torch.zeros((w.B, w.L, w.N), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros_like(u)
    with pytest.raises(mssm.MssmError) as ei:
        mssm.scan_fwd_noalloc(u, u, A, bc, bc, y=y, return_final_state=False)
    assert ei.value.status == -6
    assert not torch.any(y)
