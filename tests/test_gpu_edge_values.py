"""GPU parity at the edges of the method's value ranges: forward, backward and
the recurrent step against the float64 oracle, plus two invariants asserted on
the GPU outputs themselves (not through the oracle).

The workloads' own draws (delta = 0.5 N(0,1) + dt_bias, z ~ N(0,1), A = -(n+1))
keep every transcendental in its comfortable range.  Here:

* raw delta uniform on [-30, 30] (flag on): softplus deep in both tails --
  x = delta + dt_bias from about -37 (Delta ~ 1e-16) to +28 (Delta = x);
* a quarter of the channels with delta = -1024: softplus underflows to an
  exact 0 step (the Delta -> 0 limit), in float32 and float64 alike;
* A = -10^U(-3, 2) per (d, n) and every seventh channel's row of A zero: decays
  from exp(-3000) (exp2 underflow to 0) to 1 exactly;
* z uniform on [-100, 100]: silu's exp overflows to inf on one side (the
  reciprocal then gives 0) and silu(z) = z on the other.

Invariants (the benchmark spec's pins, here on the GPU): A = 0 makes the state a
prefix sum, h_t = h0 + sum_{s<=t} Delta_s Bm_s u_s, checked against numpy's
float64 cumsum; Delta = 0 leaves the state at h0 bit for bit and makes
y = (Cm . h0 + Dskip u) silu(z).

Tolerances: the float32 state at 1e-4 and gradients at 1e-3 relative with the
per-tensor rms floor (2e-2 for bfloat16 activations), as everywhere.  y is
judged at the activation type's bar relative to max(1, |y|, scale), where
scale = |silu(z)| (sum_n |Cm_n h_n| + |Dskip u|) is the size of the terms the
readout adds.  With these inputs the readout often cancels (terms of 1e3
summing to 1e-1), and then no float32 evaluation meets an elementwise 1e-4 of
|y| -- a plain float32 loop of the same formulas misses it by 18x on the
(2, 150, 100) case -- while the forward error bound of a float32 sum of N
products, about N 2^-24 of the terms' size, is far inside 1e-4 of `scale`.
The plain elementwise error is printed next to it."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, GRAD_TOL, STATE_TOL, fwd_err, gpu_inputs, grad_err, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mssm():
    import selective_state_space_mssm_amd as m
    return m


def _store(x, dtype):
    x = np.ascontiguousarray(x, np.float32)
    return workloads.bf16_bits(x) if dtype == "bf16" else x


def edge_inputs(B, L, D, N, dtype, seed, softplus=True, with_dy=False):
    """Inputs in storage form with the edge-value draws above (u, Bm, Cm, dy
    from the workload generator)."""
    w = workloads.custom(B, L, D, N, dtype, seed=seed)
    inp = workloads.make_inputs(w, with_dy=with_dy)
    rng = np.random.default_rng(seed + 1000)
    if softplus:
        delta = rng.uniform(-30.0, 30.0, (B, L, D))
        delta[:, :, rng.permutation(D)[: max(1, D // 4)]] = -1024.0   # Delta = softplus(-1024 + bias) = 0
    else:
        delta = rng.uniform(0.0, 30.0, (B, L, D))                     # Delta = delta + bias >= 0
    inp["delta"] = _store(delta, dtype)
    inp["z"] = _store(rng.uniform(-100.0, 100.0, (B, L, D)), dtype)
    A = -(10.0 ** rng.uniform(-3.0, 2.0, (D, N)))
    A[::7] = 0.0
    inp["A"] = A.astype(np.float32)
    if not softplus:
        inp["dt_bias"] = np.abs(inp["dt_bias"]).astype(np.float32)
    return inp


def readout_scale(inp, h0, softplus):
    """|silu(z)| (sum_n |Cm_n h_n| + |Dskip u|) per (b, t, d) in float64, the
    size of the terms of y (not a reference value: y itself comes from the
    oracle)."""
    f = {k: np.asarray(v, np.float64) for k, v in workloads.as_float32(inp).items() if k != "dtype"}
    x = f["delta"] + f["dt_bias"]
    dt = np.logaddexp(0.0, x) if softplus else x
    B, L, D = f["u"].shape
    h = np.zeros((B, D, f["A"].shape[1])) if h0 is None else np.asarray(h0, np.float64).copy()
    sc = np.empty((B, L, D))
    for t in range(L):
        h = np.exp(dt[:, t, :, None] * f["A"]) * h + (dt[:, t] * f["u"][:, t])[..., None] * f["Bm"][:, t, None, :]
        sc[:, t] = np.sum(np.abs(f["Cm"][:, t, None, :] * h), axis=-1) + np.abs(f["Dskip"] * f["u"][:, t])
    z = f["z"]
    return sc * np.abs(z / (1.0 + np.exp(-z)))


def y_err(g, r, scale):
    g = np.asarray(g, np.float64)
    return float(np.max(np.abs(g - r) / np.maximum(np.maximum(1.0, np.abs(r)), scale)))


def oracle_fwd(inp, h0, softplus):
    f = workloads.as_float32(inp)
    return oracle.scan_fwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"], f["Dskip"], f["z"], f["dt_bias"], h0,
                           softplus=softplus)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("shape", [(2, 150, 100), (1, 2100, 40)])
def test_forward_edge_values(mssm, shape, softplus, dtype):
    # (2, 150, 100): one workgroup per channel block, a ragged tile and block;
    # (1, 2100, 40): one block, so time is cut into chunks joined by the carry,
    # whose chunk decays exp(A * sum Delta) underflow to 0 here
    B, L, D = shape
    print(f"[edge fwd] shape={shape} softplus={softplus} dtype={dtype}", flush=True)
    inp = edge_inputs(B, L, D, 16, dtype, seed=B * L + D, softplus=softplus)
    h0 = np.random.default_rng(3).standard_normal((B, D, 16)).astype(np.float32)
    t = gpu_inputs(inp)
    y, hf = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"],
                          torch.from_numpy(h0).cuda(), delta_softplus=softplus)
    torch.cuda.synchronize()
    yr, hr = oracle_fwd(inp, h0, softplus)
    yg = to_np(y)
    assert np.all(np.isfinite(yg))
    ey, eh = y_err(yg, yr, readout_scale(inp, h0, softplus)), fwd_err(to_np(hf), hr)
    print(f"  y err {ey:.2e} against the terms' size (elementwise {fwd_err(yg, yr):.2e}, max |y| "
          f"{np.max(np.abs(yr)):.2e}), h_final err {eh:.2e}", flush=True)
    assert ey <= FWD_TOL[dtype] and eh <= STATE_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 150, 100), (1, 300, 70)])
def test_backward_edge_values(mssm, shape, dtype):
    # (1, 300, 70): few channel blocks, so the reverse walk is cut into time chunks joined by the adjoint carry
    B, L, D = shape
    print(f"[edge bwd] shape={shape} dtype={dtype}", flush=True)
    inp = edge_inputs(B, L, D, 16, dtype, seed=B * L + D + 1, with_dy=True)
    rng = np.random.default_rng(4)
    h0 = rng.standard_normal((B, D, 16)).astype(np.float32)
    dhf = rng.standard_normal((B, D, 16)).astype(np.float32)
    t = gpu_inputs(inp)
    g = mssm.scan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["z"], t["dt_bias"],
                      torch.from_numpy(h0).cuda(), torch.from_numpy(dhf).cuda())
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    r = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], Dskip=f["Dskip"], z=f["z"],
                        dt_bias=f["dt_bias"], h0=h0, dh_final=dhf)
    errs = {k: grad_err(to_np(g[k]), r[k]) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias",
                                                     "dh0")}
    print("  grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k in errs:
        assert np.all(np.isfinite(to_np(g[k]))), k
    bad = {k: v for k, v in errs.items() if not v <= GRAD_TOL[dtype]}
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 150, 100), (1, 600, 70)])
def test_training_pair_edge_values(mssm, shape, dtype):
    # the training pair: the backward from the saved context forms sbar and dz from dy, z and the saved
    # readout itself (silu' at |z| up to 100); (1, 600, 70): chunked forward and chunked reverse
    B, L, D = shape
    print(f"[edge train pair] shape={shape} dtype={dtype}", flush=True)
    inp = edge_inputs(B, L, D, 16, dtype, seed=B * L + D + 5, with_dy=True)
    rng = np.random.default_rng(5)
    h0 = rng.standard_normal((B, D, 16)).astype(np.float32)
    dhf = rng.standard_normal((B, D, 16)).astype(np.float32)
    t = gpu_inputs(inp)
    _, _, ctx = mssm.scan_fwd_train(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"],
                                    t["dt_bias"], torch.from_numpy(h0).cuda())
    g = mssm.scan_bwd_saved(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx, t["Dskip"], t["z"],
                            t["dt_bias"], torch.from_numpy(dhf).cuda())
    torch.cuda.synchronize()
    f = workloads.as_float32(inp)
    r = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"], f["dy"], Dskip=f["Dskip"], z=f["z"],
                        dt_bias=f["dt_bias"], h0=h0, dh_final=dhf)
    errs = {k: grad_err(to_np(g[k]), r[k]) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias",
                                                     "dh0")}
    print("  grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k in errs:
        assert np.all(np.isfinite(to_np(g[k]))), k
    bad = {k: v for k, v in errs.items() if not v <= GRAD_TOL[dtype]}
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_edge_values(mssm, dtype):
    B, L, D, N = 3, 12, 100, 16
    print(f"[edge step] dtype={dtype}", flush=True)
    inp = edge_inputs(B, L, D, N, dtype, seed=77)
    h0 = np.random.default_rng(5).standard_normal((B, D, N)).astype(np.float32)
    t = gpu_inputs(inp)
    state = torch.from_numpy(h0).cuda()
    ys = [mssm.step(t["u"][:, i].contiguous(), t["delta"][:, i].contiguous(), t["A"], t["Bm"][:, i].contiguous(),
                    t["Cm"][:, i].contiguous(), state, t["Dskip"], t["z"][:, i].contiguous(), t["dt_bias"])
          for i in range(L)]
    torch.cuda.synchronize()
    yr, hr = oracle_fwd(inp, h0, True)
    assert y_err(to_np(torch.stack(ys, 1)), yr, readout_scale(inp, h0, True)) <= FWD_TOL[dtype]
    assert fwd_err(to_np(state), hr) <= STATE_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [150, 2100])
def test_invariant_A_zero_is_prefix_sum(mssm, L, dtype):
    """A = 0: every decay is 1 and the state is h0 plus the running sum of
    Delta Bm u -- computed here with numpy's float64 cumsum, independent of the
    oracle.  (L = 2100 with one channel block runs the time-chunked schedule.)"""
    B, D, N = (2, 100, 16) if L < 1000 else (1, 40, 16)
    print(f"[invariant A=0] L={L} dtype={dtype}", flush=True)
    w = workloads.custom(B, L, D, N, dtype, seed=L + 9)
    inp = workloads.make_inputs(w)
    inp["A"] = np.zeros((D, N), np.float32)
    h0 = np.random.default_rng(6).standard_normal((B, D, N)).astype(np.float32)
    t = gpu_inputs(inp)
    y, hf = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"],
                          torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    f = {k: np.asarray(v, np.float64) for k, v in workloads.as_float32(inp).items() if k != "dtype"}
    dt = np.logaddexp(0.0, f["delta"] + f["dt_bias"])                      # softplus, (B, L, D)
    h = h0[:, None, :, :] + np.cumsum((dt * f["u"])[..., None] * f["Bm"][:, :, None, :], axis=1)  # (B, L, D, N)
    s = np.einsum("bln,bldn->bld", f["Cm"], h) + f["Dskip"] * f["u"]
    yr = s * f["z"] / (1.0 + np.exp(-f["z"]))
    ey, eh = fwd_err(to_np(y), yr), fwd_err(to_np(hf), h[:, -1])
    print(f"  y err {ey:.2e}, h_final err {eh:.2e}", flush=True)
    assert ey <= FWD_TOL[dtype] and eh <= STATE_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("softplus", [True, False])
def test_invariant_delta_zero(mssm, softplus, dtype):
    """Delta = 0 (flag off: delta = -dt_bias = 0; flag on: delta = -1024, whose
    softplus underflows to 0): every decay is exp(0) = 1 and every input 0, so
    the state stays h0 bit for bit and y = (Cm . h0 + Dskip u) silu(z)."""
    B, L, D, N = 2, 90, 130, 16
    print(f"[invariant Delta=0] softplus={softplus} dtype={dtype}", flush=True)
    w = workloads.custom(B, L, D, N, dtype, seed=91)
    inp = workloads.make_inputs(w)
    inp["delta"] = _store(np.full((B, L, D), -1024.0 if softplus else 0.0), dtype)
    if not softplus:
        inp["dt_bias"] = np.zeros(D, np.float32)
    h0 = np.random.default_rng(7).standard_normal((B, D, N)).astype(np.float32)
    t = gpu_inputs(inp)
    h0t = torch.from_numpy(h0).cuda()
    y, hf = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"], h0t,
                          delta_softplus=softplus)
    y0, hf0 = mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["z"], t["dt_bias"], None,
                            delta_softplus=softplus)
    torch.cuda.synchronize()
    assert torch.equal(hf, h0t), "the state moved although every step is 0"
    assert not torch.any(hf0), "the state left zero although every step is 0"
    f = {k: np.asarray(v, np.float64) for k, v in workloads.as_float32(inp).items() if k != "dtype"}
    gate = f["z"] / (1.0 + np.exp(-f["z"]))
    skip = f["Dskip"] * f["u"]
    yr = (np.einsum("bln,bdn->bld", f["Cm"], h0.astype(np.float64)) + skip) * gate
    assert fwd_err(to_np(y), yr) <= FWD_TOL[dtype]
    assert fwd_err(to_np(y0), skip * gate) <= FWD_TOL[dtype]
