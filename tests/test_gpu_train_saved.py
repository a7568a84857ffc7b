"""GPU parity of the training pair: mssm_scan_fwd_train (the forward that
saves the state before every 16-step tile and the readout before the gate)
and mssm_scan_bwd_saved (the backward that starts from that context, with no
pre-pass).

* the forward's y and h_final equal mssm_scan_fwd's bit for bit (same
  kernels), on every schedule the forward uses: one workgroup per channel
  block, the balanced persistent schedule, the time-chunked schedule;
* the gradients du, ddelta, dA, dB, dC, dD, dz, ddt_bias, dh0 match the
  oracle's analytic adjoint element by element (helpers.grad_err, 1e-3 for
  float32 activations, 2e-2 for bfloat16) and mssm_scan_bwd's to 1e-6;
* shapes: ragged, every optional input, no gate, every state size, bfloat16,
  the reverse walk cut into chunks (few channel blocks) and into tail walks
  (between half and all of the CUs), short sequences (which mssm_scan_fwd runs
  on its short-sequence path, the training forward on the tiled one), the
  training workload in full, and bitwise reproducibility."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, GRAD_TOL, fwd_err, grad_err, gpu_inputs, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GRADS = ["du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dh0"]


@pytest.fixture(scope="module")
def mssm():
    import selective_state_space_mssm_amd as m
    return m


def short_path(w):  # the sequences mssm_scan_fwd runs on its short-sequence path
    return w.L <= 8 or (w.L <= 64 and w.B * w.D <= 32768)


def run_pair(mssm, w, h0=True, dhf=True, gate=True, with_oracle=True):
    print(f"[train pair] {w} h0={h0} dhf={dhf} gate={gate}", flush=True)
    inp = workloads.make_inputs(w, with_dy=True)
    t = gpu_inputs(inp)
    rng = np.random.default_rng(w.seed + 7)
    h0n = rng.standard_normal((w.B, w.D, w.N)).astype(np.float32) if h0 else None
    dhn = rng.standard_normal((w.B, w.D, w.N)).astype(np.float32) if dhf else None
    cu = lambda a: None if a is None else torch.from_numpy(a).cuda()  # noqa: E731
    z = t["z"] if gate else None
    y, hf, ctx = mssm.scan_fwd_train(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], z, t["dt_bias"],
                                     cu(h0n))
    y0, hf0 = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], z, t["dt_bias"], cu(h0n))
    if short_path(w):  # other kernels than the training forward's: equal up to rounding
        assert fwd_err(to_np(y), to_np(y0)) <= FWD_TOL[w.dtype] and fwd_err(to_np(hf), to_np(hf0)) <= 1e-5
    else:
        assert torch.equal(y, y0) and torch.equal(hf, hf0), "training forward differs from mssm_scan_fwd"
    g = mssm.scan_bwd_saved(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx, t["Dskip"], z,
                            t["dt_bias"], cu(dhn))
    ref = mssm.scan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], z, t["dt_bias"],
                        cu(h0n), cu(dhn))
    torch.cuda.synchronize()
    for k in GRADS:
        if ref[k] is not None:
            e = grad_err(to_np(g[k]), to_np(ref[k]))
            assert e <= 1e-6, f"{k}: {e:.2e} from mssm_scan_bwd"
    if not with_oracle:
        return g, None
    f = workloads.as_float32(inp)
    r = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], Dskip=f["Dskip"],
                        z=f["z"] if gate else None, dt_bias=f["dt_bias"], h0=h0n, dh_final=dhn)
    return g, r


def assert_grads(g, r, tol, skip=()):
    errs = {k: grad_err(to_np(g[k]), r[k]) for k in GRADS if k not in skip and r.get(k) is not None}
    print("grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"gradients over tolerance {tol}: {bad}"


@pytest.mark.parametrize("shape", [(2, 37, 70), (1, 16, 64), (2, 100, 130), (1, 1, 5), (2, 300, 200)])
def test_ragged_all_options(mssm, shape):
    B, L, D = shape
    g, r = run_pair(mssm, workloads.custom(B, L, D, 16, "f32", seed=L * 5 + D))
    assert_grads(g, r, GRAD_TOL["f32"])


def test_no_gate_no_state_inputs(mssm):
    g, r = run_pair(mssm, workloads.custom(2, 150, 80, 16, "f32", seed=13), h0=False, dhf=False, gate=False)
    assert g["dz"] is None
    assert_grads(g, r, GRAD_TOL["f32"])


@pytest.mark.parametrize("N", [1, 2, 4, 8, 32, 64, 3, 12, 24, 48])
def test_state_sizes(mssm, N):
    # 3, 12, 24, 48: the next power of two's kernels with inert extra states, its context
    g, r = run_pair(mssm, workloads.custom(2, 90, 70, N, "f32", seed=N + 150))
    assert_grads(g, r, GRAD_TOL["f32"])


@pytest.mark.parametrize("N,L", [(16, 96), (16, 46), (4, 83), (64, 70)])
def test_bf16(mssm, N, L):
    g, r = run_pair(mssm, workloads.custom(2, L, 96, N, "bf16", seed=N + L + 160))
    assert_grads(g, r, GRAD_TOL["bf16"])


@pytest.mark.parametrize("shape,dtype", [((1, 300, 70), "f32"), ((1, 600, 100), "bf16"), ((1, 4500, 40), "f32")])
def test_chunked(mssm, shape, dtype):
    # few channel blocks: the reverse walk in time chunks joined by the adjoint carry; from L = 512 the
    # training forward runs the time-chunked schedule and writes each chunk's checkpoints in its rescan
    B, L, D = shape
    g, r = run_pair(mssm, workloads.custom(B, L, D, 16, dtype, seed=L + D + 17))
    assert_grads(g, r, GRAD_TOL[dtype])


@pytest.mark.parametrize("shape,N,dtype", [
    ((3, 300, 3200), 16, "f32"),   # 150 blocks: walks [0, 2) and 2, the last tile ragged
    ((2, 260, 6144), 16, "bf16"),  # 192 blocks
    ((1, 200, 8960), 64, "f32"),   # 140 blocks
])
def test_tail_walks(mssm, shape, N, dtype):
    # the last chunk's Q pass forms sbar from dy and z itself
    B, L, D = shape
    g, r = run_pair(mssm, workloads.custom(B, L, D, N, dtype, seed=L + D + N + 1))
    assert_grads(g, r, GRAD_TOL[dtype])


def test_tail_walks_no_gate(mssm):
    g, r = run_pair(mssm, workloads.custom(3, 300, 3200, 16, "f32", seed=92), h0=False, gate=False)
    assert_grads(g, r, GRAD_TOL["f32"])


@pytest.mark.parametrize("shape,dtype", [((3, 48, 5760), "f32"), ((5, 37, 3840), "bf16")])
def test_balanced_forward(mssm, shape, dtype):
    # 270 and 300 channel blocks on a 256-CU MI355X: the training forward's balanced schedule writes the
    # checkpoints of blocks split between two workers
    B, L, D = shape
    g, r = run_pair(mssm, workloads.custom(B, L, D, 16, dtype, seed=B * L + 3), dhf=False)
    assert_grads(g, r, GRAD_TOL[dtype])


def test_training_workload_full(mssm):
    w = workloads.WORKLOADS["train"]
    g, r = run_pair(mssm, w, h0=False, dhf=False)
    assert_grads(g, r, GRAD_TOL["f32"], skip=("dh0",))


def test_bitwise_reproducible_and_ctx_reuse(mssm):
    w = workloads.custom(2, 96, 200, 16, "f32", seed=71)
    inp = workloads.make_inputs(w, with_dy=True)
    t = gpu_inputs(inp)
    fa = (t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"])
    _, _, ctx = mssm.scan_fwd_train(*fa)
    g1 = mssm.scan_bwd_saved(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx, t["Dskip"], t["z"],
                             t["dt_bias"])
    ctx2 = torch.full_like(ctx, 0xFF)  # a used context buffer is overwritten, not read
    mssm.scan_fwd_train(*fa, ctx=ctx2)
    nck = w.B * ((w.L + 15) // 16) * w.N * w.D * 4  # the checkpoints, then (256-byte aligned) the readouts
    s0 = (nck + 255) // 256 * 256
    ns = w.B * w.L * w.D * 4
    assert torch.equal(ctx[:nck], ctx2[:nck]) and torch.equal(ctx[s0:s0 + ns], ctx2[s0:s0 + ns])
    g2 = mssm.scan_bwd_saved(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx2, t["Dskip"], t["z"],
                             t["dt_bias"])
    for k in GRADS:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_training_pair_in_a_graph(mssm):
    # the forward saving its context and the backward from it (tail-walk plan: the last chunk's Q pass, the long
    # and short walks, the reductions) captured in one graph, replayed 3 times with new u and dy (eager calls
    # between the replays): every replay equals the eager calls on the same inputs bit for bit
    w = workloads.custom(3, 300, 3200, 16, "f32", seed=6)
    print(f"[train pair graph] {w}", flush=True)
    inp = workloads.make_inputs(w, with_dy=True)
    t = gpu_inputs(inp)
    u, dy = t["u"].clone(), t["dy"].clone()

    def call():
        y, hf, ctx = mssm.scan_fwd_train(u, t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"])
        g = mssm.scan_bwd_saved(u, t["delta"], t["A"], t["Bm"], t["Cm"], dy, ctx, t["Dskip"], t["z"], t["dt_bias"])
        return dict(g, y=y, h_final=hf)

    call()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        out = call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    for r in range(3):
        u.copy_(torch.from_numpy(rng.standard_normal(tuple(u.shape)).astype(np.float32)).cuda())
        dy.copy_(torch.from_numpy(rng.standard_normal(tuple(dy.shape)).astype(np.float32)).cuda())
        ref = {k: v.clone() for k, v in call().items() if v is not None}
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(out[k], v), (r, k)
