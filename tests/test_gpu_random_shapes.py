"""GPU parity on seeded random problems: shapes, state sizes, activation types
and optional inputs drawn at random, so that combinations the targeted tests
do not name (ragged channel blocks, short and long sequences, every layout and
schedule; the training pair of a forward saving its context and the backward
from it) are compared with the float64 oracle too.  Every case prints its
draw before it runs."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, STATE_TOL, GRAD_TOL, fwd_err, gpu_inputs, grad_err, run_oracle_fwd, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

STATES = [1, 2, 4, 8, 16, 32, 64]
OPTIONAL = ("Dskip", "z", "dt_bias")


def draw(i):
    rng = np.random.default_rng(1000 + i)
    B = int(rng.integers(1, 7))
    L = int(rng.choice([rng.integers(1, 65), rng.integers(65, 400), rng.integers(2048, 2600)], p=[0.4, 0.5, 0.1]))
    D = int(rng.integers(1, 700)) if rng.random() < 0.8 else int(rng.integers(3000, 4400))
    if L >= 2048:
        B, D = 1, int(rng.integers(1, 200))  # long sequences: few channel blocks (the chunked schedule)
    N = int(rng.choice(STATES))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    use = tuple(k for k in OPTIONAL if rng.random() < 0.7)
    h0 = bool(rng.random() < 0.5)
    K = int(rng.integers(1, 5))
    return B, L, D, N, dtype, use, h0, K


@pytest.mark.parametrize("i", range(24))
def test_random_forward(mssm_lib, i):
    B, L, D, N, dtype, use, h0, K = draw(i)
    print(f"[random fwd {i}] B={B} L={L} D={D} N={N} {dtype} use={use} h0={h0}", flush=True)
    w = workloads.custom(B, L, D, N, dtype, seed=3000 + i)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0n = np.random.default_rng(i).standard_normal((B, D, N)).astype(np.float32) if h0 else None
    g = lambda k: t[k] if k in use else None  # noqa: E731
    y, hf = mssm_lib.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], g("Dskip"), g("z"), g("dt_bias"),
                              torch.from_numpy(h0n).cuda() if h0 else None)
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, h0n, use=use)
    assert fwd_err(to_np(y), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(hf), hr) <= STATE_TOL


@pytest.mark.parametrize("i", range(12))
def test_random_conv_forward(mssm_lib, i):
    B, L, D, N, dtype, use, h0, K = draw(100 + i)
    print(f"[random conv fwd {i}] B={B} L={L} D={D} N={N} {dtype} use={use} d_conv={K}", flush=True)
    w = workloads.custom(B, L, D, N, dtype, seed=3100 + i)
    inp = workloads.make_inputs(w)
    inp.update(workloads.conv_front_end(w, K))
    t = gpu_inputs(inp)
    g = lambda k: t[k] if k in use else None  # noqa: E731
    y, hf, _ = mssm_lib.conv_scan_fwd(t["u"], t["conv_w"], t["delta"], t["A"], t["Bm"], t["Cm"], g("Dskip"), g("z"),
                                      g("dt_bias"), None, conv_b=t["conv_b"], x_prev=t["x_prev"] if K > 1 else None)
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    h = lambda k: f[k] if k in use else None  # noqa: E731
    yr, hr, _ = oracle.conv_scan_fwd(f["u"], f["conv_w"], f["delta"], f["A"], f["Bm"], f["Cm"], h("Dskip"), h("z"),
                                     h("dt_bias"), None, bias=f["conv_b"], x_prev=f["x_prev"] if K > 1 else None)
    assert fwd_err(to_np(y), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(hf), hr) <= STATE_TOL


@pytest.mark.parametrize("i", range(10))
def test_random_backward(mssm_lib, i):
    B, L, D, N, dtype, use, h0, K = draw(200 + i)
    L = min(L, 300)  # the float64 adjoint keeps the whole state history
    print(f"[random bwd {i}] B={B} L={L} D={D} N={N} {dtype} use={use} h0={h0}", flush=True)
    w = workloads.custom(B, L, D, N, dtype, seed=3200 + i, backward=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0n = np.random.default_rng(i).standard_normal((B, D, N)).astype(np.float32) if h0 else None
    g = lambda k: t[k] if k in use else None  # noqa: E731
    gg = mssm_lib.scan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], g("Dskip"), g("z"), g("dt_bias"),
                           torch.from_numpy(h0n).cuda() if h0 else None)
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    h = lambda k: f[k] if k in use else None  # noqa: E731
    r = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], h("Dskip"), h("z"), h("dt_bias"), h0n)
    tol = GRAD_TOL[dtype]
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "ddt_bias") + (("dz",) if "z" in use else ()) + \
            (("dh0",) if h0 else ()):
        assert grad_err(to_np(gg[k]), r[k]) <= tol, k


@pytest.mark.parametrize("i", range(10))
def test_random_training_pair(mssm_lib, i):
    # the forward saving its context and the backward from it, with the draws of the backward sweep
    B, L, D, N, dtype, use, h0, K = draw(250 + i)
    L = min(L, 300)
    print(f"[random train pair {i}] B={B} L={L} D={D} N={N} {dtype} use={use} h0={h0}", flush=True)
    w = workloads.custom(B, L, D, N, dtype, seed=3250 + i, backward=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0n = np.random.default_rng(i + 50).standard_normal((B, D, N)).astype(np.float32) if h0 else None
    g = lambda k: t[k] if k in use else None  # noqa: E731
    h0t = torch.from_numpy(h0n).cuda() if h0 else None
    y, hf, ctx = mssm_lib.scan_fwd_train(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], g("Dskip"), g("z"),
                                         g("dt_bias"), h0t)
    gg = mssm_lib.scan_bwd_saved(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx, g("Dskip"), g("z"),
                                 g("dt_bias"))
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, h0n, use=use)
    assert fwd_err(to_np(y), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(hf), hr) <= STATE_TOL
    f = workloads.as_float32(inp)
    h = lambda k: f[k] if k in use else None  # noqa: E731
    r = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], h("Dskip"), h("z"), h("dt_bias"), h0n)
    tol = GRAD_TOL[dtype]
    for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "ddt_bias", "dh0") + (("dz",) if "z" in use else ()):
        assert grad_err(to_np(gg[k]), r[k]) <= tol, k


@pytest.fixture(scope="module")
def mssm_lib():
    import selective_state_space_mssm_amd as m
    return m


@pytest.mark.parametrize("i", range(10))
def test_random_conv_backward(mssm_lib, i):
    B, L, D, N, dtype, use, h0, K = draw(300 + i)
    L = min(L, 3000)
    print(f"[random conv bwd {i}] B={B} L={L} D={D} {dtype} d_conv={K}", flush=True)
    w = workloads.custom(B, L, D, 16, dtype, seed=3300 + i)
    inp = workloads.make_inputs(w)
    inp.update(workloads.conv_front_end(w, K))
    t = gpu_inputs(inp)
    du = t["z"]  # any (B, L, D) activations of the same type serve as du
    with_prev = K > 1 and i % 2 == 0
    g = mssm_lib.conv_bwd(t["u"], t["conv_w"], du, conv_b=t["conv_b"], x_prev=t["x_prev"] if with_prev else None,
                          want_dx_prev=K > 1)
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    r = oracle.causal_conv_silu_bwd(f["u"], f["conv_w"], f["z"], f["conv_b"], f["x_prev"] if with_prev else None)
    tol = GRAD_TOL[dtype]
    assert grad_err(to_np(g["dx"]), r["dx"]) <= tol
    assert grad_err(to_np(g["dconv_w"]), r["dweight"]) <= tol
    assert grad_err(to_np(g["dconv_b"]), r["dbias"]) <= tol
    if K > 1:
        assert grad_err(to_np(g["dx_prev"]), r["dx_prev"]) <= tol


@pytest.mark.parametrize("i", range(6))
def test_random_conv_decode(mssm_lib, i):
    B, L, D, N, dtype, use, h0, K = draw(400 + i)
    L = min(L, 12)
    print(f"[random conv decode {i}] B={B} L={L} D={D} N={N} {dtype} d_conv={K}", flush=True)
    w = workloads.custom(B, L, D, N, dtype, seed=3400 + i)
    inp = workloads.make_inputs(w)
    inp.update(workloads.conv_front_end(w, K))
    t = gpu_inputs(inp)
    state = torch.zeros((B, D, N), device="cuda")
    cst = t["x_prev"].clone() if K > 1 else None
    # per-token slices as fresh (16-byte aligned) tensors: with B = 1 a slice is already "contiguous" and
    # would be passed at its offset inside the sequence, which the C ABI rejects as misaligned
    col = lambda a, s: a[:, s].clone()  # noqa: E731
    ys = [mssm_lib.conv_step(col(t["u"], s), t["conv_w"], cst, col(t["delta"], s), t["A"], col(t["Bm"], s),
                             col(t["Cm"], s), state, t["Dskip"], col(t["z"], s), t["dt_bias"], conv_b=t["conv_b"])
          for s in range(L)]
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    yr, hr, _ = oracle.conv_scan_fwd(f["u"], f["conv_w"], f["delta"], f["A"], f["Bm"], f["Cm"], f["Dskip"], f["z"],
                                     f["dt_bias"], None, bias=f["conv_b"], x_prev=f["x_prev"] if K > 1 else None)
    assert fwd_err(to_np(torch.stack(ys, 1)), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(state), hr) <= STATE_TOL


@pytest.mark.parametrize("i", range(12))
def test_random_ssd(mssm_lib, i):
    # Mamba-2 (SSD) forward: shapes on both sides of the segmented path (fewer than 128 (batch, head) pairs and at
    # least 4 chunks), both state sizes and activation types, optional inputs, h0 and the softplus flag drawn
    rng = np.random.default_rng(5000 + i)
    B, H = int(rng.integers(1, 5)), int(rng.integers(1, 48))
    L = int(rng.choice([rng.integers(1, 65), rng.integers(65, 700), rng.integers(700, 2600)]))
    L = min(L, max(1, 400000 // (B * H)))  # keeps the float64 oracle to a few seconds
    N = int(rng.choice([64, 128]))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    use_d, use_bias, h0, sp = (bool(rng.random() < 0.6) for _ in range(4))
    P = int(rng.choice([64, 64, 64, 128, 256]))  # head dim (drawn last: the draws above are those of P = 64 only)
    L = min(L, max(1, 400000 * 64 // (B * H * P)))
    print(f"[random ssd {i}] B={B} L={L} H={H} P={P} N={N} {dtype} D={use_d} bias={use_bias} h0={h0} softplus={sp}",
          flush=True)
    inp = workloads.ssd_inputs(B, L, H, P, N, seed=6000 + i)
    if not sp:  # without softplus the raw step dt + dt_bias must be >= 0: no (negative) bias, |dt| scaled down
        inp["dt"] = np.abs(inp["dt"]) * np.float32(0.05)
        use_bias = False
    t = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    if dtype == "bf16":
        for k in ("x", "dt", "Bm", "Cm"):
            t[k] = t[k].to(torch.bfloat16)
    h0n = rng.standard_normal((B, H, P, N)).astype(np.float32) if h0 else None
    y, hf = mssm_lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"] if use_d else None,
                             t["dt_bias"] if use_bias else None, torch.from_numpy(h0n).cuda() if h0 else None,
                             delta_softplus=sp)
    torch.cuda.synchronize()
    r = {k: t[k].float().cpu().numpy() for k in ("x", "dt", "Bm", "Cm")}
    yr, hr = oracle.ssd_fwd(r["x"], r["dt"], inp["A"], r["Bm"], r["Cm"], inp["Dskip"] if use_d else None,
                            inp["dt_bias"] if use_bias else None, h0n, softplus=sp)
    assert fwd_err(to_np(y), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(hf), hr) <= STATE_TOL


@pytest.mark.parametrize("i", range(10))
def test_random_ssd_backward(mssm_lib, i):
    # Mamba-2 (SSD) backward: head dims 64..256, both state sizes and activation types, optional inputs, h0,
    # dh_final and the softplus flag drawn; sequences long enough for the chains' time segments (few pairs)
    # and the head groups of the chunk pass (few (batch, chunk) pairs) to come up
    rng = np.random.default_rng(7000 + i)
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 20))
    P = int(rng.choice([64, 64, 128, 192, 256]))
    L = int(rng.choice([rng.integers(1, 65), rng.integers(65, 400), rng.integers(400, 1500)]))
    L = min(L, max(1, 60000 * 64 // (B * H * P)))  # the float64 adjoint keeps the whole state history
    N = int(rng.choice([64, 128]))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    use_d, use_bias, h0, dhf, sp = (bool(rng.random() < 0.6) for _ in range(5))
    print(f"[random ssd bwd {i}] B={B} L={L} H={H} P={P} N={N} {dtype} D={use_d} bias={use_bias} h0={h0} "
          f"dh_final={dhf} softplus={sp}", flush=True)
    inp = workloads.ssd_inputs(B, L, H, P, N, seed=7100 + i)
    inp["Dskip"] = rng.uniform(-2.0, 2.0, size=H).astype(np.float32)
    if not sp:
        inp["dt"] = np.abs(inp["dt"]) * np.float32(0.05)
        use_bias = False
    inp["dy"] = rng.standard_normal((B, L, H, P)).astype(np.float32)
    t = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    if dtype == "bf16":
        for k in ("x", "dt", "Bm", "Cm", "dy"):
            t[k] = t[k].to(torch.bfloat16)
    h0n = rng.standard_normal((B, H, P, N)).astype(np.float32) if h0 else None
    dhn = rng.standard_normal((B, H, P, N)).astype(np.float32) if dhf else None
    cu = lambda a: None if a is None else torch.from_numpy(a).cuda()  # noqa: E731
    g = mssm_lib.ssd_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"] if use_d else None,
                         t["dt_bias"] if use_bias else None, cu(h0n), cu(dhn), delta_softplus=sp)
    torch.cuda.synchronize()
    r = {k: t[k].float().cpu().numpy() for k in ("x", "dt", "Bm", "Cm", "dy")}
    ref = oracle.ssd_bwd(r["x"], r["dt"], inp["A"], r["Bm"], r["Cm"], r["dy"], Dskip=inp["Dskip"] if use_d else None,
                         dt_bias=inp["dt_bias"] if use_bias else None, h0=h0n, dh_final=dhn, softplus=sp)
    tol = GRAD_TOL[dtype]
    keys = ["dx", "ddt", "dA", "dB", "dC", "dD", "ddt_bias", "dh0"]
    if L == 1 and not h0:
        keys.remove("dA")  # exactly 0 in the oracle, a difference of equal sums on the GPU (judged in test_gpu_ssd_bwd)
    errs = {k: grad_err(to_np(g[k]), ref[k]) for k in keys}
    print("grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= tol for v in errs.values()), errs
