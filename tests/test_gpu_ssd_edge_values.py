"""GPU parity of the Mamba-2 (SSD) forward and backward at the edges of the
value ranges, against the float64 oracle, plus invariants asserted on the GPU
outputs themselves.  The generator's draws (dt = 0.5 N(0,1), A = -U(1, 16))
keep every exponential in its comfortable range; here, per head:

* head 0: raw dt uniform on [-30, 30] (softplus deep in both tails; the
  backward: on [-30, 8], see below);
* head 1: the same with A = -100 (decays down to exp(-3000), an exact 0);
* head 2: dt = -1024, so the step underflows to an exact 0 (the Delta -> 0
  limit): the state stays h0 bit for bit and y = Cm . h0 + Dskip x;
* head 3: A = 0, no decay: the state is a prefix sum,
  h_T = h0 + sum_t Delta_t x_t Bm_t^T, checked against numpy's float64 cumsum;
* head 4: dt = +30 with A = -16 (every step forgets the state);
* head 5: the generator's draw.

Tolerances as everywhere: outputs and states at the float32 bar, gradients at
1e-3 with the per-tensor rms floor.  The backward's dt, dA and ddt_bias come
from the reverse cumulative sum of dcum_i = C_i . dC_i - Delta_i x_i . V_i over
a chunk, in which the terms of every pair of steps (j, i) enter with both signs;
with steps up to 30 between steps of moderate decay those terms reach 1e4 and
their float32 rounding leaves dA about 1.3e-3 of its rms off (measured; ddt
5e-4).  The mixed-step heads of the backward therefore draw dt on [-30, 8]
(steps up to 8); the head with a constant step of 30 and a decay that leaves no
memory stays in (there the same-step terms, which cancel exactly, are kept out
of both sums by the kernel)."""
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


def edge_inputs(B, L, N, seed, dt_hi=30.0):
    H = 6
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=seed)
    rng = np.random.default_rng(seed + 1)
    dt, A = inp["dt"], inp["A"]
    dt[:, :, 0] = rng.uniform(-30.0, dt_hi, size=(B, L))
    dt[:, :, 1] = rng.uniform(-30.0, dt_hi, size=(B, L))
    A[1] = -100.0
    dt[:, :, 2] = -1024.0
    A[3] = 0.0
    dt[:, :, 4] = 30.0
    A[4] = -16.0
    inp["Dskip"] = rng.uniform(-2.0, 2.0, size=H).astype(np.float32)
    h0 = rng.standard_normal((B, H, 64, N)).astype(np.float32)
    return inp, h0


def test_ssd_forward_edge_values(lib):
    B, L, N = 2, 200, 64
    inp, h0 = edge_inputs(B, L, N, seed=17)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    y, hf = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"],
                        torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    yr, hr = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["dt_bias"], h0)
    y, hf = to_np(y), to_np(hf)
    print(f"ssd edge: y err {fwd_err(y, yr):.2e}, h_final err {fwd_err(hf, hr):.2e}", flush=True)
    assert fwd_err(y, yr) <= FWD_TOL["f32"]
    assert fwd_err(hf, hr) <= FWD_TOL["f32"]
    # head 2: a zero step leaves the state at h0 exactly, and the output is the readout of h0 plus the skip
    assert np.array_equal(hf[:, 2], h0[:, 2])
    y2 = np.einsum("bln,bpn->blp", inp["Cm"].astype(np.float64), h0[:, 2].astype(np.float64)) + \
        float(inp["Dskip"][2]) * inp["x"][:, :, 2].astype(np.float64)
    assert fwd_err(y[:, :, 2], y2) <= FWD_TOL["f32"]
    # head 3: no decay, the final state is h0 plus the prefix sum of the inputs Delta x Bm^T
    v = inp["dt"][:, :, 3].astype(np.float64) + float(inp["dt_bias"][3])
    delta = np.logaddexp(v, 0.0)
    sum3 = np.einsum("bl,blp,bln->bpn", delta, inp["x"][:, :, 3].astype(np.float64), inp["Bm"].astype(np.float64))
    assert fwd_err(hf[:, 3], h0[:, 3] + sum3) <= FWD_TOL["f32"]


@pytest.mark.parametrize("L", [150, 1000])
def test_ssd_backward_edge_values(lib, L):
    # 150 steps: one walk per pair; 1,000 steps, 6 pairs: the chains in time segments
    B, N = 1, 64
    inp, h0 = edge_inputs(B, L, N, seed=23 + L, dt_hi=8.0)
    rng = np.random.default_rng(L)
    inp["dy"] = rng.standard_normal(inp["x"].shape).astype(np.float32)
    dhf = rng.standard_normal(h0.shape).astype(np.float32)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    g = lib.ssd_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["dt_bias"],
                    torch.from_numpy(h0).cuda(), torch.from_numpy(dhf).cuda())
    torch.cuda.synchronize()
    r = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["dy"], Dskip=inp["Dskip"],
                       dt_bias=inp["dt_bias"], h0=h0, dh_final=dhf)
    errs = {k: grad_err(to_np(g[k]), r[k]) for k in GRADS}
    print("ssd edge grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= GRAD_TOL["f32"] for v in errs.values()), errs
    # head 2: a zero step passes no gradient to dt (softplus' slope is 0 there) and none to the decay
    assert float(np.abs(to_np(g["ddt"])[:, :, 2]).max()) == 0.0
    assert float(to_np(g["dA"])[2]) == 0.0
