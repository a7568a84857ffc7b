"""Pins of the float64 oracle's forward pass against things other than itself.

Each test uses a different arithmetic route or a case with a known answer, so
that a plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong softplus or gate) fails at least one of them:

* closed form of the unrolled recurrence (products of decays as exponentials
  of partial sums) -- wrong A sign, wrong Bm/Cm indexing, missing skip or gate;
* Blelloch up-/down-sweep scan over (decay, input) pairs (the parallel-scan
  route of the page "mamba.py: 一个简单高效的Mamba实现", repository layout
  section, pscan.py) -- wrong recurrence order;
* A = 0 reduces to a prefix sum (np.cumsum);
* Delta = 0 reduces to y = Dskip*u*silu(z); Cm = 0 likewise; z = 0 gives 0;
* the time-invariant case is a causal convolution (the "convolution mode"
  discussed in the Hacker News comments of the page "PyTorch 한 파일에서의
  Mamba 구현") -- np.convolve; constant input gives a geometric series;
* linearity in u and in h0;
* exact rational arithmetic on a tiny case with decays 1/2 and 1/4;
* streaming: a split scan and repeated single steps equal one scan (the RNN
  form / step function of the mamba.py page, updates section);
* the frozen Tiny-workload output under tests/golden (regression guard).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B=2, L=40, D=5, N=4, softplus=True):
    dt = np.exp(rng.uniform(np.log(1e-2), np.log(3e-1), size=D))
    return dict(
        u=rng.standard_normal((B, L, D)),
        delta=0.5 * rng.standard_normal((B, L, D)),
        A=-rng.uniform(0.2, 3.0, size=(D, N)),
        Bm=rng.standard_normal((B, L, N)),
        Cm=rng.standard_normal((B, L, N)),
        Dskip=rng.standard_normal(D),
        z=rng.standard_normal((B, L, D)),
        dt_bias=np.log(np.expm1(dt)),
        h0=rng.standard_normal((B, D, N)),
        softplus=softplus,
    )


def softplus_lib(x):
    return np.logaddexp(0.0, x)


def silu_lib(z):
    return z * expit(z)


def closed_form(inp):
    """h_{t,n} = exp(A_n S_t) h0_n + sum_{s<=t} exp(A_n (S_t - S_s)) Delta_s Bm_{s,n} u_s,
    S_t = sum_{r<=t} Delta_r; y = (Cm.h + Dskip u) silu(z).  O(L^2) per channel."""
    u, delta, A, Bm, Cm = inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"]
    B, L, D = u.shape
    N = A.shape[1]
    x = delta + inp["dt_bias"][None, None, :]
    dt = softplus_lib(x) if inp["softplus"] else x
    S = np.cumsum(dt, axis=1)                       # (B, L, D)
    y = np.empty_like(u)
    hf = np.empty((B, D, N))
    for b in range(B):
        for d in range(D):
            for t in range(L):
                dec = np.exp(A[d][None, :] * (S[b, t, d] - S[b, : t + 1, d])[:, None])  # (t+1, N)
                h = np.exp(A[d] * S[b, t, d]) * inp["h0"][b, d] + (
                    dec * (dt[b, : t + 1, d] * u[b, : t + 1, d])[:, None] * Bm[b, : t + 1]).sum(0)
                y[b, t, d] = (Cm[b, t] @ h + inp["Dskip"][d] * u[b, t, d]) * silu_lib(inp["z"][b, t, d])
                if t == L - 1:
                    hf[b, d] = h
    return y, hf


def run(inp, **over):
    kw = dict(inp)
    kw.update(over)
    return oracle.scan_fwd(kw["u"], kw["delta"], kw["A"], kw["Bm"], kw["Cm"],
                           Dskip=kw.get("Dskip"), z=kw.get("z"), dt_bias=kw.get("dt_bias"),
                           h0=kw.get("h0"), softplus=kw.get("softplus", True))


def rel(a, b):
    return np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b)))


@pytest.mark.parametrize("softplus", [True, False])
def test_closed_form(softplus):
    rng = np.random.default_rng(10)
    inp = rand_inputs(rng, softplus=softplus)
    if not softplus:  # keep Delta positive so the recurrence stays contractive
        inp["delta"] = np.abs(inp["delta"]) * 0.1
        inp["dt_bias"] = np.full(inp["u"].shape[2], 0.01)
    y, hf = run(inp)
    yc, hc = closed_form(inp)
    assert rel(y, yc) < 1e-12
    assert rel(hf, hc) < 1e-12


def blelloch_inclusive(a, g):
    """Inclusive scan of pairs e_t = (a_t, g_t) under the non-commutative
    operator (a1, g1) o (a2, g2) = (a1 a2, a2 g1 + g2) with identity (1, 0),
    by the Blelloch up-sweep / down-sweep (exclusive) scan on a power-of-two
    padded array, then one combine with the element itself."""
    L = a.shape[0]
    P = 1
    while P < L:
        P *= 2
    A_ = np.ones((P,) + a.shape[1:])
    G_ = np.zeros((P,) + a.shape[1:])
    A_[:L], G_[:L] = a, g
    step = 1
    while step < P:  # up-sweep
        for i in range(2 * step - 1, P, 2 * step):
            j = i - step
            A_[i], G_[i] = A_[j] * A_[i], A_[i] * G_[j] + G_[i]
        step *= 2
    A_[P - 1], G_[P - 1] = 1.0, 0.0
    step = P // 2
    while step >= 1:  # down-sweep
        for i in range(2 * step - 1, P, 2 * step):
            j = i - step
            tA, tG = A_[j].copy(), G_[j].copy()
            A_[j], G_[j] = A_[i], G_[i]
            # new right = (left prefix) o (left subtree total)
            A_[i], G_[i] = A_[i] * tA, tA * G_[i] + tG
        step //= 2
    # exclusive prefix o element -> inclusive
    return (A_[:L] * a, a * G_[:L] + g)


def test_blelloch_scan():
    rng = np.random.default_rng(11)
    inp = rand_inputs(rng, B=1, L=37, D=3, N=4)
    y, hf = run(inp)
    u, A = inp["u"][0], inp["A"]
    x = inp["delta"][0] + inp["dt_bias"]
    dt = softplus_lib(x)
    for d in range(3):
        a = np.exp(dt[:, d, None] * A[d][None, :])                   # (L, N)
        g = dt[:, d, None] * inp["Bm"][0] * u[:, d, None]
        g[0] += a[0] * inp["h0"][0, d]                                 # fold h0 into the first element
        _, h = blelloch_inclusive(a, g)
        s = (inp["Cm"][0] * h).sum(1) + inp["Dskip"][d] * u[:, d]
        yb = s * silu_lib(inp["z"][0, :, d])
        assert rel(y[0, :, d], yb) < 1e-12
        assert rel(hf[0, d], h[-1]) < 1e-12


def test_blelloch_matches_sequential_on_pairs():
    # the scan helper itself against a plain loop (so a broken helper cannot pass the test above)
    rng = np.random.default_rng(12)
    a, g = rng.uniform(0.1, 1, (13, 2)), rng.standard_normal((13, 2))
    _, h = blelloch_inclusive(a, g)
    ref = np.zeros(2)
    for t in range(13):
        ref = a[t] * ref + g[t]
        assert np.allclose(h[t], ref, rtol=1e-14, atol=1e-14)


def test_A_zero_is_prefix_sum():
    rng = np.random.default_rng(13)
    inp = rand_inputs(rng)
    inp["A"] = np.zeros_like(inp["A"])
    inp["z"] = None
    inp["Dskip"] = None
    y, hf = run(inp)
    x = inp["delta"] + inp["dt_bias"]
    dt = softplus_lib(x)
    g = (dt * inp["u"])[..., None] * inp["Bm"][:, :, None, :]         # (B, L, D, N)
    h = inp["h0"][:, None] + np.cumsum(g, axis=1)
    yr = np.einsum("bldn,bln->bld", h, inp["Cm"])
    assert rel(y, yr) < 1e-12
    assert rel(hf, h[:, -1]) < 1e-12


def test_delta_zero_flag_off():
    rng = np.random.default_rng(14)
    inp = rand_inputs(rng, softplus=False)
    inp["delta"] = np.broadcast_to(-inp["dt_bias"], inp["u"].shape).copy()  # x = 0 exactly
    y, hf = run(inp)
    expect = inp["Dskip"] * inp["u"] * silu_lib(inp["z"])
    assert np.array_equal(hf, inp["h0"])
    # h = h0 is carried unchanged, so y = (Cm.h0 + D u) silu(z)
    y_expect = (np.einsum("bln,bdn->bld", inp["Cm"], inp["h0"]) + inp["Dskip"] * inp["u"]) * silu_lib(inp["z"])
    assert rel(y, y_expect) < 1e-14
    y0, hf0 = run(inp, h0=None)
    assert np.all(hf0 == 0.0)
    assert rel(y0, expect) < 1e-15


def test_delta_zero_softplus_underflow():
    rng = np.random.default_rng(15)
    inp = rand_inputs(rng)
    inp["delta"] = np.full(inp["u"].shape, -900.0)   # softplus(-900+bias) == 0 in float64
    y, hf = run(inp, h0=None)
    assert np.all(hf == 0.0)
    assert rel(y, inp["Dskip"] * inp["u"] * silu_lib(inp["z"])) < 1e-15


def test_C_zero_and_z_zero():
    rng = np.random.default_rng(16)
    inp = rand_inputs(rng)
    y, _ = run(inp, Cm=np.zeros_like(inp["Cm"]), h0=None)
    assert rel(y, inp["Dskip"] * inp["u"] * silu_lib(inp["z"])) < 1e-15
    y, _ = run(inp, z=np.zeros_like(inp["z"]))
    assert np.all(y == 0.0)
    # no gate == gate with silu replaced by 1: compare against Dskip=0, Cm=0 pieces
    y_ng, _ = run(inp, z=None)
    y_g, _ = run(inp)
    assert rel(y_g, y_ng * silu_lib(inp["z"])) < 1e-14


def test_lti_is_causal_convolution():
    rng = np.random.default_rng(17)
    L, N = 64, 6
    A = -rng.uniform(0.2, 2.0, size=(1, N))
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    dtv = 0.07
    u = rng.standard_normal((1, L, 1))
    inp = dict(u=u, delta=np.full((1, L, 1), dtv), A=A,
               Bm=np.broadcast_to(Bv, (1, L, N)).copy(), Cm=np.broadcast_to(Cv, (1, L, N)).copy(),
               Dskip=None, z=None, dt_bias=None, h0=None, softplus=False)
    y, _ = run(inp)
    k = np.arange(L)
    K = (Cv[None, :] * np.exp(k[:, None] * dtv * A[0][None, :]) * dtv * Bv[None, :]).sum(1)
    yc = np.convolve(u[0, :, 0], K)[:L]
    assert rel(y[0, :, 0], yc) < 1e-12


def test_constant_input_geometric_series():
    L, N = 200, 3
    A = np.array([[-0.5, -1.0, -4.0]])
    dtv, uv = 0.03, 1.7
    Bv = np.array([0.3, -1.2, 2.0])
    inp = dict(u=np.full((1, L, 1), uv), delta=np.full((1, L, 1), dtv), A=A,
               Bm=np.broadcast_to(Bv, (1, L, N)).copy(), Cm=np.zeros((1, L, N)),
               Dskip=None, z=None, dt_bias=None, h0=None, softplus=False)
    _, hf = run(inp)
    a = np.exp(dtv * A[0])
    expect = dtv * Bv * uv * (1 - a ** L) / (1 - a)
    assert rel(hf[0, 0], expect) < 1e-12


def test_linearity_in_u_and_h0():
    rng = np.random.default_rng(18)
    inp = rand_inputs(rng)
    u1, u2 = rng.standard_normal(inp["u"].shape), rng.standard_normal(inp["u"].shape)
    h1, h2 = rng.standard_normal(inp["h0"].shape), rng.standard_normal(inp["h0"].shape)
    al, be = 0.7, -1.3
    # y is linear in (u, h0) jointly when delta is fixed
    ya, ha = run(inp, u=u1, h0=h1)
    yb, hb = run(inp, u=u2, h0=h2)
    yc, hc = run(inp, u=al * u1 + be * u2, h0=al * h1 + be * h2)
    assert rel(yc, al * ya + be * yb) < 1e-12
    assert rel(hc, al * ha + be * hb) < 1e-12


def exact_tiny_case():
    """Tiny case in exact rational arithmetic: flag off, no bias, Delta = ln 2,
    A = (-1, -2) so the decays are exactly 1/2 and 1/4; Delta*Bm*u is made
    rational by taking u_t = k_t / ln 2."""
    ln2 = float(np.log(2.0))
    L = 5
    Bm = [[1, 2], [-1, 3], [2, 0], [0, -2], [1, 1]]
    Cm = [[2, 1], [1, -1], [3, 2], [-1, 1], [1, 4]]
    k = [1, -2, 3, 1, 4]
    Dk = 2
    dec = [Fraction(1, 2), Fraction(1, 4)]
    h = [Fraction(0), Fraction(0)]
    ys = []
    for t in range(L):
        for n in range(2):
            h[n] = dec[n] * h[n] + Fraction(Bm[t][n]) * k[t]   # Delta*u_t = k_t
        # Dskip*u_t = Dk * k_t / ln 2 is irrational: keep it as a separate float term
        ys.append((sum(Fraction(Cm[t][n]) * h[n] for n in range(2)), Dk * k[t] / ln2))
    inp = dict(u=(np.array(k, float) / ln2).reshape(1, L, 1), delta=np.full((1, L, 1), ln2),
               A=np.array([[-1.0, -2.0]]), Bm=np.array(Bm, float)[None], Cm=np.array(Cm, float)[None],
               Dskip=np.array([float(Dk)]), z=None, dt_bias=None, h0=None, softplus=False)
    return inp, ys, h


def test_exact_rational_tiny_case():
    inp, ys, h = exact_tiny_case()
    y, hf = run(inp)
    for t, (frac, skip) in enumerate(ys):
        assert abs(y[0, t, 0] - (float(frac) + skip)) <= 1e-13 * max(1.0, abs(float(frac) + skip))
    assert np.allclose(hf[0, 0], [float(h[0]), float(h[1])], rtol=1e-14, atol=1e-14)


def test_split_scan_and_steps_equal_one_scan():
    rng = np.random.default_rng(19)
    inp = rand_inputs(rng, L=30)
    y, hf = run(inp)
    L1 = 11
    part1 = {k: (v[:, :L1] if k in ("u", "delta", "z", "Bm", "Cm") else v) for k, v in inp.items()}
    part2 = {k: (v[:, L1:] if k in ("u", "delta", "z", "Bm", "Cm") else v) for k, v in inp.items()}
    y1, h1 = run(part1)
    y2, h2 = run(part2, h0=h1)
    assert np.array_equal(np.concatenate([y1, y2], 1), y)
    assert np.array_equal(h2, hf)
    st = inp["h0"]
    for t in range(30):
        yt, st = oracle.step(inp["u"][:, t], inp["delta"][:, t], inp["A"], inp["Bm"][:, t],
                             inp["Cm"][:, t], st, Dskip=inp["Dskip"], z_t=inp["z"][:, t],
                             dt_bias=inp["dt_bias"])
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(st, hf)


def test_softplus_values():
    # softplus(0) = ln 2; softplus(x) - softplus(-x) = x; large x -> x
    y, _ = oracle.scan_fwd(np.ones((1, 1, 1)), np.zeros((1, 1, 1)), np.zeros((1, 1)),
                           np.ones((1, 1, 1)), np.ones((1, 1, 1)), softplus=True)
    assert abs(y[0, 0, 0] - np.log(2.0)) < 1e-16
    for xv in (-30.0, -3.0, 0.4, 5.0, 40.0):
        yp, _ = oracle.scan_fwd(np.ones((1, 1, 1)), np.full((1, 1, 1), xv), np.zeros((1, 1)),
                                np.ones((1, 1, 1)), np.ones((1, 1, 1)), softplus=True)
        ym, _ = oracle.scan_fwd(np.ones((1, 1, 1)), np.full((1, 1, 1), -xv), np.zeros((1, 1)),
                                np.ones((1, 1, 1)), np.ones((1, 1, 1)), softplus=True)
        assert abs((yp - ym)[0, 0, 0] - xv) < 1e-14 * max(1, abs(xv))
        assert abs(yp[0, 0, 0] - softplus_lib(xv)) <= 1e-15 * max(1e-14, softplus_lib(xv)) * 4


def test_dt_bias_recipe_maps_zero_delta_to_dt():
    # the workload recipe: with raw delta = 0, the step size equals the drawn dt
    w = workloads.custom(1, 1, 64, 1, seed=3)
    dt_bias, _, _ = workloads.channel_params(w)
    y, _ = oracle.scan_fwd(np.ones((1, 1, 64)), np.zeros((1, 1, 64)), np.zeros((64, 1)),
                           np.ones((1, 1, 1)), np.ones((1, 1, 1)), dt_bias=dt_bias, softplus=True)
    dt = y[0, 0]
    assert dt.min() > 0.9e-3 and dt.max() < 1.1e-1
    rng = np.random.Generator(np.random.PCG64(3))
    dt_drawn = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=64))
    assert np.max(np.abs(dt / dt_drawn - 1)) < 1e-6   # dt_bias is stored in float32


def test_golden_tiny_regression():
    """Frozen oracle output on the Tiny workload (written by
    tests/golden/make_golden.py, which calls only the oracle)."""
    with open(os.path.join(GOLDEN, "tiny_fwd.json")) as f:
        g = json.load(f)
    w = workloads.WORKLOADS["tiny"]
    inp = workloads.as_float32(workloads.make_inputs(w))
    y, hf = oracle.scan_fwd(inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"],
                            inp["z"], inp["dt_bias"], None, softplus=True)
    idx = np.array(g["y_index"])
    assert np.allclose(y.reshape(-1)[idx], np.array(g["y_values"]), rtol=1e-13, atol=1e-15)
    assert abs(float(np.sum(y)) - g["y_sum"]) < 1e-10
    assert abs(float(np.sum(hf * hf)) - g["h_final_sumsq"]) < 1e-10 * g["h_final_sumsq"]
