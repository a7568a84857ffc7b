"""GPU parity of the Mamba-2 (SSD) forward, mssm_ssd_fwd, against the float64
oracle (the selective scan over channels (head, p) with one decay and step
per head).  Shapes span several 64-step chunks with a ragged last chunk, one
step, both built state sizes, every optional input, and streaming in place."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, STATE_TOL, fwd_err, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
TOL = FWD_TOL["f32"]


@pytest.fixture(scope="module")
def lib():
    import selective_state_space_mssm_amd as m
    return m


def gpu(inp):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}


CASES = [  # B, L, H, N
    (2, 200, 3, 64),
    (1, 64, 2, 128),
    (2, 1, 2, 64),
    (1, 257, 4, 128),
    (3, 130, 2, 64),
    (1, 1000, 5, 128),
]


@pytest.mark.parametrize("B,L,H,N", CASES)
@pytest.mark.parametrize("opts", ["all", "none", "h0_nosoftplus"])
def test_ssd_forward_parity(lib, B, L, H, N, opts):
    print(f"[ssd fwd] B={B} L={L} H={H} N={N} {opts}", flush=True)
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=B * 1000 + L + N)
    t = gpu(inp)
    h0n = np.random.default_rng(L).standard_normal((B, H, 64, N)).astype(np.float32) if opts.startswith("h0") else None
    sp = opts != "h0_nosoftplus"
    dt = inp["dt"] if sp else np.abs(inp["dt"]) * np.float32(0.05)  # without softplus the raw step must be >= 0
    use = opts != "none"
    y, hf = lib.ssd_fwd(t["x"], torch.from_numpy(dt).cuda(), t["A"], t["Bm"], t["Cm"],
                        t["Dskip"] if use else None, t["dt_bias"] if use and sp else None,
                        torch.from_numpy(h0n).cuda() if h0n is not None else None, delta_softplus=sp)
    torch.cuda.synchronize()
    yr, hr = oracle.ssd_fwd(inp["x"], dt, inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"] if use else None,
                            inp["dt_bias"] if use and sp else None, h0n, softplus=sp)
    assert fwd_err(to_np(y), yr) <= TOL
    assert fwd_err(to_np(hf), hr) <= TOL


def test_ssd_streaming_in_place(lib):
    # two calls over [0, 100) and [100, 300) with h_final == h0 equal one call over [0, 300)
    B, L, H, N = 2, 300, 3, 128
    print(f"[ssd streaming] B={B} L={L} H={H} N={N}", flush=True)
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=77)
    t = gpu(inp)
    state = torch.zeros((B, H, 64, N), device="cuda")
    ys = []
    for a, b in ((0, 100), (100, 300)):
        sl = lambda k: t[k][:, a:b].contiguous()  # noqa: E731
        y, _ = lib.ssd_fwd(sl("x"), sl("dt"), t["A"], sl("Bm"), sl("Cm"), t["Dskip"], t["dt_bias"], state,
                           h_final=state)
        ys.append(y)
    torch.cuda.synchronize()
    yr, hr = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["dt_bias"])
    assert fwd_err(to_np(torch.cat(ys, 1)), yr) <= TOL
    assert fwd_err(to_np(state), hr) <= TOL


def test_ssd_no_final_state_and_validation(lib):
    inp = workloads.ssd_inputs(1, 70, 2, 64, 64, seed=5)
    t = gpu(inp)
    y, hf = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], return_final_state=False)
    torch.cuda.synchronize()
    assert hf is None
    yr, _ = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"])
    assert fwd_err(to_np(y), yr) <= TOL
    with pytest.raises(lib.MssmError):  # head dimension 32 is not built
        lib.ssd_fwd(t["x"][..., :32].contiguous(), t["dt"], t["A"], t["Bm"], t["Cm"])


def test_ssd_mamba2_layer_sampled(lib):
    # a Mamba-2 2.7B-shaped layer (d_inner 5120 = 80 heads of 64, d_state 128) at L = 2048, checked on a
    # sample of heads: the kernel runs all 80, the oracle recomputes heads {0, 37, 79} in full
    B, L, H, N = 2, 2048, 80, 128
    print(f"[ssd 2.7B layer] B={B} L={L} H={H} N={N}", flush=True)
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=2048)
    t = gpu(inp)
    y, hf = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"])
    torch.cuda.synchronize()
    heads = [0, 37, 79]
    sub = lambda k: inp[k][:, :, heads]  # noqa: E731
    yr, hr = oracle.ssd_fwd(sub("x"), sub("dt"), inp["A"][heads], inp["Bm"], inp["Cm"], inp["Dskip"][heads],
                            inp["dt_bias"][heads])
    assert fwd_err(to_np(y[:, :, heads]), yr) <= TOL
    assert fwd_err(to_np(hf[:, heads]), hr) <= TOL


@pytest.mark.parametrize("B,L,H,N", [(1, 2048, 24, 128), (1, 700, 3, 64), (2, 1100, 1, 64)])
def test_ssd_time_segments(lib, B, L, H, N):
    # few (batch, head) pairs: the sequence is cut into segments scanned in parallel, then a carry pass and a
    # correction pass (mssm_ssd_fwd_workspace_bytes > 0); with h0, the state advanced in place, every optional input
    import ctypes
    prob = lib.binding.SsdProblem(B, L, H, 64, N, 0, 1)
    assert lib.lib.mssm_ssd_fwd_workspace_bytes(ctypes.byref(prob)) > 0
    print(f"[ssd segments] B={B} L={L} H={H} N={N}", flush=True)
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=L + H)
    t = gpu(inp)
    h0n = np.random.default_rng(H).standard_normal((B, H, 64, N)).astype(np.float32)
    state = torch.from_numpy(h0n).cuda()
    y, _ = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"], state, h_final=state)
    torch.cuda.synchronize()
    yr, hr = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["dt_bias"], h0n)
    assert fwd_err(to_np(y), yr) <= TOL
    assert fwd_err(to_np(state), hr) <= TOL


@pytest.mark.parametrize("B,L,H,N", [(2, 200, 3, 64), (1, 257, 4, 128), (3, 130, 2, 64), (1, 1000, 5, 128),
                                     (8, 300, 20, 128)])
def test_ssd_bf16(lib, B, L, H, N):
    # bfloat16 x, dt, Bm, Cm and y, float32 arithmetic: the oracle takes the rounded inputs (exact in float32);
    # the first and fourth shapes take the segmented path, the last one workgroup per (batch, head)
    print(f"[ssd bf16] B={B} L={L} H={H} N={N}", flush=True)
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=5000 + L)
    t = gpu(inp)
    for k in ("x", "dt", "Bm", "Cm"):
        t[k] = t[k].to(torch.bfloat16)
    h0n = np.random.default_rng(N).standard_normal((B, H, 64, N)).astype(np.float32)
    y, hf = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"],
                        torch.from_numpy(h0n).cuda())
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    r = {k: t[k].float().cpu().numpy() for k in ("x", "dt", "Bm", "Cm")}
    yr, hr = oracle.ssd_fwd(r["x"], r["dt"], inp["A"], r["Bm"], r["Cm"], inp["Dskip"], inp["dt_bias"], h0n)
    assert fwd_err(to_np(y), yr) <= FWD_TOL["bf16"]
    assert fwd_err(to_np(hf), hr) <= STATE_TOL


@pytest.mark.parametrize("B,L,H,N,dtype", [(3, 300, 90, 64, "f32"), (5, 130, 60, 128, "f32"),
                                           (3, 200, 86, 64, "bf16")])
def test_ssd_balanced_schedule(lib, B, L, H, N, dtype):
    # at least as many (batch, head) pairs as CUs, not a multiple of them (270, 300, 258 on a 256-CU MI355X):
    # one persistent workgroup per CU scans an equal share of the chunks, pairs split between two workgroups
    # handing their state over through the workspace; with h0 and the state advanced in place
    import ctypes
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    prob = lib.binding.SsdProblem(B, L, H, 64, N, 1 if dtype == "bf16" else 0, 1)
    ws = lib.lib.mssm_ssd_fwd_workspace_bytes(ctypes.byref(prob))
    assert (ws > 0) == (B * H >= ncu and B * H % ncu != 0)
    print(f"[ssd balanced] B={B} L={L} H={H} N={N} {dtype} ws={ws}", flush=True)
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=B * H + L)
    t = gpu(inp)
    if dtype == "bf16":
        for k in ("x", "dt", "Bm", "Cm"):
            t[k] = t[k].to(torch.bfloat16)
    h0n = np.random.default_rng(H).standard_normal((B, H, 64, N)).astype(np.float32)
    state = torch.from_numpy(h0n).cuda()
    y, _ = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"], state, h_final=state)
    torch.cuda.synchronize()
    r = {k: t[k].float().cpu().numpy() for k in ("x", "dt", "Bm", "Cm")}
    yr, hr = oracle.ssd_fwd(r["x"], r["dt"], inp["A"], r["Bm"], r["Cm"], inp["Dskip"], inp["dt_bias"], h0n)
    assert fwd_err(to_np(y), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(state), hr) <= STATE_TOL


def test_ssd_mamba2_layer_batch8_sampled(lib):
    # the timed 80-head layer (B = 8, L = 2048, d_state 128): 640 (batch, head) pairs on the balanced
    # schedule (on 256 CUs, 2.5 pairs per workgroup; every pair with head = 2 mod 5 is split between two
    # workgroups); the oracle recomputes heads {0, 37, 79} of every batch in full
    B, L, H, N = 8, 2048, 80, 128
    print(f"[ssd 2.7B layer, batch 8] B={B} L={L} H={H} N={N}", flush=True)
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=4096)
    t = gpu(inp)
    h0n = np.random.default_rng(9).standard_normal((B, H, 64, N)).astype(np.float32)
    y, hf = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"],
                        torch.from_numpy(h0n).cuda())
    torch.cuda.synchronize()
    heads = [0, 37, 79]
    sub = lambda k: inp[k][:, :, heads]  # noqa: E731
    yr, hr = oracle.ssd_fwd(sub("x"), sub("dt"), inp["A"][heads], inp["Bm"], inp["Cm"], inp["Dskip"][heads],
                            inp["dt_bias"][heads], h0n[:, heads])
    assert fwd_err(to_np(y[:, :, heads]), yr) <= TOL
    assert fwd_err(to_np(hf[:, heads]), hr) <= STATE_TOL
