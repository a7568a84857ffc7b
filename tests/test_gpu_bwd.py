"""GPU parity of the backward scan (mssm_scan_bwd) against the oracle's
analytic adjoint: du, ddelta, dA, dB, dC, dD, dz, ddt_bias, dh0, element by
element with the relative criterion of helpers.grad_err.

Covers the training workload (B=8, L=2048, D=1536, N=16, fp32) in full, ragged
small shapes with every optional input (h0, dh_final, z, Dskip, dt_bias), the
ungated path, every supported state size, bfloat16 activations, the reverse
walk cut into time chunks joined by the adjoint carry (one walk per chunk, or
one long walk per block and its last chunk walked apart), the forward pre-pass
under its chunked and its balanced schedules, and bitwise reproducibility
(the reductions have a fixed order, no atomics)."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import GRAD_TOL, grad_err, gpu_inputs, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GRADS = ["du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dh0"]


@pytest.fixture(scope="module")
def mssm():
    import selective_state_space_mssm_amd as m
    return m


def run_both(mssm, w, h0=True, dhf=True, gate=True, softplus=True):
    print(f"[bwd] {w} h0={h0} dhf={dhf} gate={gate}", flush=True)
    inp = workloads.make_inputs(w, with_dy=True)
    t = gpu_inputs(inp)
    rng = np.random.default_rng(w.seed + 7)
    h0n = rng.standard_normal((w.B, w.D, w.N)).astype(np.float32) if h0 else None
    dhn = rng.standard_normal((w.B, w.D, w.N)).astype(np.float32) if dhf else None
    cu = lambda a: None if a is None else torch.from_numpy(a).cuda()  # noqa: E731
    g = mssm.scan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"],
                      t["z"] if gate else None, t["dt_bias"], cu(h0n), cu(dhn), delta_softplus=softplus)
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    r = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], Dskip=f["Dskip"],
                        z=f["z"] if gate else None, dt_bias=f["dt_bias"], h0=h0n, dh_final=dhn,
                        softplus=softplus)
    return g, r


def assert_grads(g, r, tol, skip=()):
    errs = {}
    for k in GRADS:
        if k in skip or r.get(k) is None:
            continue
        errs[k] = grad_err(to_np(g[k]), r[k])
    print("grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"gradients over tolerance {tol}: {bad}"


@pytest.mark.parametrize("shape", [(2, 37, 70), (1, 16, 64), (2, 100, 130), (1, 1, 5)])
def test_ragged_all_options(mssm, shape):
    B, L, D = shape
    g, r = run_both(mssm, workloads.custom(B, L, D, 16, "f32", seed=L * 3 + D))
    assert_grads(g, r, GRAD_TOL["f32"])


def test_no_gate_no_state_inputs(mssm):
    g, r = run_both(mssm, workloads.custom(2, 50, 80, 16, "f32", seed=3), h0=False, dhf=False, gate=False)
    assert g["dz"] is None
    assert_grads(g, r, GRAD_TOL["f32"])


@pytest.mark.parametrize("N", [1, 2, 4, 8, 32, 64])
def test_state_sizes(mssm, N):
    g, r = run_both(mssm, workloads.custom(2, 40, 70, N, "f32", seed=N + 50))
    assert_grads(g, r, GRAD_TOL["f32"])


def test_bf16(mssm):
    g, r = run_both(mssm, workloads.custom(2, 64, 96, 16, "bf16", seed=60))
    assert_grads(g, r, GRAD_TOL["bf16"])


@pytest.mark.parametrize("L", [23, 46])
def test_bf16_ragged(mssm, L):
    # the pre-pass's readout groups end inside a group in the last tile
    g, r = run_both(mssm, workloads.custom(2, L, 96, 16, "bf16", seed=L + 61))
    assert_grads(g, r, GRAD_TOL["bf16"])


@pytest.mark.parametrize("N", [4, 8, 64])
def test_state_sizes_bf16(mssm, N):
    g, r = run_both(mssm, workloads.custom(2, 43, 70, N, "bf16", seed=N + 70))
    assert_grads(g, r, GRAD_TOL["bf16"])


@pytest.mark.parametrize("shape,dtype", [((1, 300, 70), "f32"), ((1, 300, 70), "bf16"), ((2, 1000, 40), "f32")])
def test_chunked_reverse(mssm, shape, dtype):
    # few channel blocks: the reverse walk is cut into time chunks (L = 300:
    # 4 chunks of 5, 5, 5, 4 tiles, the last tile ragged; L = 1000: 13 chunks)
    # joined by the adjoint carry; dh_final enters the last chunk, dh0 leaves the first
    B, L, D = shape
    g, r = run_both(mssm, workloads.custom(B, L, D, 16, dtype, seed=L + D + 7))
    assert_grads(g, r, GRAD_TOL[dtype])


def test_chunked_reverse_plain(mssm):
    # no dh_final (the last chunk starts from zero), no gate, no h0, softplus off
    w = workloads.custom(1, 300, 70, 16, "f32", seed=17)
    g, r = run_both(mssm, w, h0=False, dhf=False, gate=False)
    assert_grads(g, r, GRAD_TOL["f32"])
    inp = workloads.make_inputs(w, with_dy=True)
    inp["delta"] = (0.05 * np.abs(inp["delta"])).astype(np.float32)
    inp["dt_bias"] = np.full(w.D, 0.01, np.float32)
    t = gpu_inputs(inp)
    g = mssm.scan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["z"], t["dt_bias"],
                      None, None, delta_softplus=False)
    f = workloads.as_float32(inp)
    r = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], Dskip=f["Dskip"], z=f["z"],
                        dt_bias=f["dt_bias"], softplus=False)
    assert_grads(g, r, GRAD_TOL["f32"])


def test_chunked_reverse_many_chunks(mssm):
    # 24 channel blocks: 32 chunks of 8 tiles
    g, r = run_both(mssm, workloads.custom(1, 4096, 1536, 16, "f32", seed=77))
    assert_grads(g, r, GRAD_TOL["f32"])


@pytest.mark.parametrize("N", [1, 4, 64])
def test_chunked_reverse_state_sizes(mssm, N):
    g, r = run_both(mssm, workloads.custom(1, 200, 50, N, "f32", seed=N + 300))
    assert_grads(g, r, GRAD_TOL["f32"])


@pytest.mark.parametrize("shape,N,dtype", [
    ((3, 300, 3200), 16, "f32"),    # 150 blocks: 3 chunks of 7, 7, 5 tiles; walks [0, 2) and 2, last tile ragged
    ((2, 260, 6144), 16, "bf16"),   # 192 blocks: 4 chunks of 5, 5, 5, 2 tiles; walks [0, 3) and 3
    ((1, 400, 12800), 4, "f32"),    # 200 blocks: 5 chunks of 5 tiles; walks [0, 4) and 4
    ((1, 200, 8960), 64, "f32"),    # 140 blocks: 3 chunks of 5, 5, 3 tiles
    ((1, 300, 9600), 8, "f32"),     # 150 blocks, two states per wave
    ((2, 300, 5120), 32, "bf16"),   # 160 blocks, four states per wave
])
def test_tail_walk_reverse(mssm, shape, N, dtype):
    # more channel blocks than half the CUs of a 256-CU MI355X but fewer than all: each block's reverse walk
    # covers all chunks but the last, whose own walk runs on an otherwise idle CU from dh_final; the walk
    # before it starts from the adjoint the carry forms from the last chunk's Q
    B, L, D = shape
    g, r = run_both(mssm, workloads.custom(B, L, D, N, dtype, seed=L + D + N))
    assert_grads(g, r, GRAD_TOL[dtype])


def test_tail_walk_reverse_plain(mssm):
    # the same plan with no dh_final (the last chunk's walk starts from zero), no gate, no h0
    g, r = run_both(mssm, workloads.custom(3, 300, 3200, 16, "f32", seed=91), h0=False, dhf=False, gate=False)
    assert_grads(g, r, GRAD_TOL["f32"])


def test_tail_walk_backward_in_a_graph(mssm):
    # the tail-walk plan (pre-pass, the last chunk's Q pass, the long and short reverse walks, the
    # reductions) captured in a graph, replayed 3 times with a new dy each time (eager calls between the
    # replays): every replay equals the eager call on the same inputs bit for bit
    w = workloads.custom(3, 300, 3200, 16, "f32", seed=5)
    print(f"[bwd graph] {w}", flush=True)
    inp = workloads.make_inputs(w, with_dy=True)
    t = gpu_inputs(inp)
    dy = t["dy"].clone()

    def call():
        return mssm.scan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], dy, t["Dskip"], t["z"], t["dt_bias"])

    call()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        out = call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for r in range(3):
        dy.copy_(torch.from_numpy(rng.standard_normal(tuple(dy.shape)).astype(np.float32)).cuda())
        ref = {k: v.clone() for k, v in call().items() if v is not None}
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(out[k], v), (r, k)


@pytest.mark.parametrize("shape,dtype", [((1, 600, 100), "f32"), ((2, 1024, 64), "bf16")])
def test_chunked_prepass_short(mssm, shape, dtype):
    # few channel blocks and 512 <= L < 2048: the pre-pass runs the time-chunked forward schedule
    B, L, D = shape
    assert mssm.fwd_workspace_bytes(B, L, D, 16) > 0
    g, r = run_both(mssm, workloads.custom(B, L, D, 16, dtype, seed=L + 43))
    assert_grads(g, r, GRAD_TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_prepass(mssm, dtype):
    # one channel block and L >= 2048: the forward pre-pass runs the chunked
    # schedule (chunk end states, carry, rescan), the last chunk ragged
    B, L, D = 1, 4500, 40
    assert mssm.fwd_workspace_bytes(B, L, D, 16) > 0
    g, r = run_both(mssm, workloads.custom(B, L, D, 16, dtype, seed=41))
    assert_grads(g, r, GRAD_TOL[dtype])


@pytest.mark.parametrize("shape,dtype", [((3, 48, 5760), "f32"), ((5, 37, 3840), "bf16")])
def test_balanced_prepass(mssm, shape, dtype):
    # more channel blocks than CUs but not a multiple of them (270 and 300 on
    # a 256-CU MI355X): the forward pre-pass runs the balanced persistent
    # schedule, handing split blocks' states over through the workspace
    B, L, D = shape
    g, r = run_both(mssm, workloads.custom(B, L, D, 16, dtype, seed=B * L + 1), dhf=False)
    assert_grads(g, r, GRAD_TOL[dtype])


def test_training_workload_full(mssm):
    w = workloads.WORKLOADS["train"]
    g, r = run_both(mssm, w, h0=False, dhf=False)
    assert_grads(g, r, GRAD_TOL["f32"], skip=("dh0",))


def test_bitwise_reproducible(mssm):
    w = workloads.custom(2, 96, 200, 16, "f32", seed=70)
    inp = workloads.make_inputs(w, with_dy=True)
    t = gpu_inputs(inp)
    args = (t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["z"], t["dt_bias"])
    g1 = mssm.scan_bwd(*args)
    g2 = mssm.scan_bwd(*args)
    for k in GRADS:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k
