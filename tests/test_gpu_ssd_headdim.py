"""GPU parity of the Mamba-2 (SSD) forward and backward at head dims above 64
(128, 192, 256) against the float64 oracle, which takes any head dim.  The
kernels run such a head as head_dim / 64 parts of 64 channels that share the
head's dt, A, Dskip and dt_bias; the cases give every head its own Dskip (the
generator's are all 1) so that a part reading another head's parameters
fails, and cover the one-workgroup-per-pair grid, the time-segmented path
(few pairs) and the balanced persistent schedule of the forward, and the
backward's summing of ddt, dA, dDskip and ddt_bias over a head's parts."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, GRAD_TOL, fwd_err, grad_err, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GRADS = ["dx", "ddt", "dA", "dB", "dC", "dD", "ddt_bias", "dh0"]


@pytest.fixture(scope="module")
def lib():
    import selective_state_space_mssm_amd as m
    return m


def inputs(B, L, H, P, N, seed):
    inp = workloads.ssd_inputs(B, L, H, P, N, seed=seed)
    inp["Dskip"] = np.random.default_rng(seed + 3).uniform(-2.0, 2.0, size=H).astype(np.float32)
    return inp


def gpu(inp, dtype="f32"):
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    if dtype == "bf16":
        for k in ("x", "dt", "Bm", "Cm", "dy"):
            if k in t:
                t[k] = t[k].to(torch.bfloat16)
                inp[k] = t[k].float().cpu().numpy()  # the oracle takes the rounded values, exact in float32
    return t


@pytest.mark.parametrize("B,L,H,P,N,dtype", [
    (2, 130, 3, 128, 64, "f32"),     # grid: 12 pairs, 3 chunks
    (1, 200, 2, 256, 128, "f32"),    # segmented: 4 chunks, 8 pairs
    (2, 300, 3, 192, 64, "f32"),     # segmented, ragged last segment
    (3, 130, 45, 128, 64, "f32"),    # balanced: 270 pairs on the CUs
    (2, 257, 2, 128, 128, "bf16"),
])
def test_ssd_forward_wide_heads(lib, B, L, H, P, N, dtype):
    print(f"[ssd fwd headdim] B={B} L={L} H={H} P={P} N={N} {dtype}", flush=True)
    inp = inputs(B, L, H, P, N, seed=B * 7 + L + P)
    h0 = np.random.default_rng(L + 1).standard_normal((B, H, P, N)).astype(np.float32)
    t = gpu(inp, dtype)
    y, hf = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"],
                        torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    yr, hr = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["dt_bias"], h0)
    tol = FWD_TOL[dtype]
    assert fwd_err(to_np(y), yr) <= tol
    assert fwd_err(to_np(hf), hr) <= FWD_TOL["f32"]  # the state is float32 whatever the activations


@pytest.mark.parametrize("B,L,H,P,N,dtype", [
    (2, 150, 3, 128, 64, "f32"),
    (1, 130, 2, 256, 128, "f32"),
    (1, 200, 3, 192, 64, "f32"),
    (2, 100, 2, 128, 128, "bf16"),
])
def test_ssd_backward_wide_heads(lib, B, L, H, P, N, dtype):
    print(f"[ssd bwd headdim] B={B} L={L} H={H} P={P} N={N} {dtype}", flush=True)
    inp = inputs(B, L, H, P, N, seed=B * 11 + L + P)
    rng = np.random.default_rng(L + P)
    inp["dy"] = rng.standard_normal((B, L, H, P)).astype(np.float32)
    h0 = rng.standard_normal((B, H, P, N)).astype(np.float32)
    dhf = rng.standard_normal((B, H, P, N)).astype(np.float32)
    t = gpu(inp, dtype)
    g = lib.ssd_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["dt_bias"],
                    torch.from_numpy(h0).cuda(), torch.from_numpy(dhf).cuda())
    torch.cuda.synchronize()
    r = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["dy"], Dskip=inp["Dskip"],
                       dt_bias=inp["dt_bias"], h0=h0, dh_final=dhf)
    errs = {k: grad_err(to_np(g[k]), r[k]) for k in GRADS}
    print("grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    tol = GRAD_TOL[dtype]
    assert all(v <= tol for v in errs.values()), errs


def test_ssd_wide_head_equals_its_parts(lib):
    # a head of 128 channels gives, bit for bit, what two 64-channel heads with its dt, A, Dskip and dt_bias
    # give (the same kernels run the same sub-heads)
    B, L, H, P, N = 2, 200, 3, 128, 64
    inp = inputs(B, L, H, P, N, seed=5)
    t = gpu(inp)
    y, hf = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"])
    rep = lambda v: v.repeat_interleave(2, dim=-1).contiguous()  # noqa: E731
    y2, hf2 = lib.ssd_fwd(t["x"].reshape(B, L, 2 * H, 64), rep(t["dt"]), rep(t["A"]), t["Bm"], t["Cm"],
                          rep(t["Dskip"]), rep(t["dt_bias"]))
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(B, L, 2 * H, 64), y2)
    assert torch.equal(hf.reshape(B, 2 * H, 64, N), hf2)
