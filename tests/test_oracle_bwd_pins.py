"""Pins of the float64 oracle's analytic adjoint against independent routes.

* central finite differences of the oracle's own forward (float64, step 1e-6)
  for every input, with every optional input present;
* torch.autograd (CPU, float64) through a plain PyTorch loop of the forward
  definition -- reverse-mode derivatives from a library, not from the
  hand-derived adjoint;
* the adjoint dot-product identity <dy, J v> = <J^T dy, v> with J v from
  forward-mode differentiation (torch.func.jvp);
* invariants: ddt_bias = sum over (b, t) of ddelta; dD = sum of dy*silu(z)*u;
  with A = 0 and no gate, du has the closed form Dskip*dy + Delta * sum_{t'>=t} ...

The pages say the implementations they describe are meant to match the
official one numerically in forward and backward (page "PyTorch 한 파일에서의
Mamba 구현", project overview); no tolerance is printed there.
"""
import numpy as np
import pytest
import torch

import oracle

NAMES = ["u", "delta", "A", "Bm", "Cm", "Dskip", "z", "dt_bias", "h0"]
GRAD_OF = {"u": "du", "delta": "ddelta", "A": "dA", "Bm": "dB", "Cm": "dC", "Dskip": "dD",
           "z": "dz", "dt_bias": "ddt_bias", "h0": "dh0"}


def rand_case(seed, B=2, L=8, D=3, N=4):
    rng = np.random.default_rng(seed)
    dt = np.exp(rng.uniform(np.log(2e-2), np.log(3e-1), size=D))
    return dict(
        u=rng.standard_normal((B, L, D)), delta=0.5 * rng.standard_normal((B, L, D)),
        A=-rng.uniform(0.2, 3.0, size=(D, N)), Bm=rng.standard_normal((B, L, N)),
        Cm=rng.standard_normal((B, L, N)), Dskip=rng.standard_normal(D),
        z=rng.standard_normal((B, L, D)), dt_bias=np.log(np.expm1(dt)),
        h0=rng.standard_normal((B, D, N)),
    ), rng.standard_normal((B, L, D)), rng.standard_normal((B, D, N))


def fwd(inp, softplus=True):
    return oracle.scan_fwd(inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"],
                           inp["z"], inp["dt_bias"], inp["h0"], softplus=softplus)


def bwd(inp, dy, dhf, softplus=True):
    return oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                           Dskip=inp["Dskip"], z=inp["z"], dt_bias=inp["dt_bias"], h0=inp["h0"],
                           dh_final=dhf, softplus=softplus)


def loss(inp, dy, dhf, softplus=True):
    y, hf = fwd(inp, softplus)
    return float(np.sum(dy * y) + np.sum(dhf * hf))


@pytest.mark.parametrize("softplus", [True, False])
def test_finite_differences(softplus):
    inp, dy, dhf = rand_case(1)
    if not softplus:
        inp["delta"] = 0.02 + 0.05 * np.abs(inp["delta"])
        inp["dt_bias"] = np.full(3, 0.01)
    g = bwd(inp, dy, dhf, softplus)
    eps = 1e-6
    for name in NAMES:
        x = inp[name]
        fd = np.empty_like(x)
        flat = x.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            lp = loss(inp, dy, dhf, softplus)
            flat[i] = old - eps
            lm = loss(inp, dy, dhf, softplus)
            flat[i] = old
            fd.reshape(-1)[i] = (lp - lm) / (2 * eps)
        an = g[GRAD_OF[name]]
        err = np.max(np.abs(an - fd)) / max(1e-12, np.max(np.abs(fd)))
        assert err < 1e-6, (name, err)


def torch_loop(t, softplus=True):
    """Plain PyTorch loop of the forward definition (float64, CPU)."""
    u, delta, A, Bm, Cm, Dk, z, bias, h0 = (t[k] for k in NAMES)
    B, L, D = u.shape
    x = delta + bias
    dt = torch.nn.functional.softplus(x) if softplus else x
    h = h0
    ys = []
    for i in range(L):
        a = torch.exp(dt[:, i, :, None] * A[None])                          # (B, D, N)
        h = a * h + (dt[:, i, :, None] * u[:, i, :, None]) * Bm[:, i, None, :]
        s = (h * Cm[:, i, None, :]).sum(-1) + Dk * u[:, i]
        ys.append(s * torch.nn.functional.silu(z[:, i]))
    return torch.stack(ys, 1), h


def test_torch_autograd():
    inp, dy, dhf = rand_case(2, B=2, L=24, D=5, N=6)
    g = bwd(inp, dy, dhf)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp.items()}
    y, hf = torch_loop(t)
    (torch.sum(torch.tensor(dy) * y) + torch.sum(torch.tensor(dhf) * hf)).backward()
    for name in NAMES:
        ref = t[name].grad.numpy()
        err = np.linalg.norm(g[GRAD_OF[name]] - ref) / np.linalg.norm(ref)
        assert err < 1e-12, (name, err)
    # and the forward matches the torch loop
    yo, hfo = fwd(inp)
    assert np.max(np.abs(yo - y.detach().numpy())) < 1e-12 * np.max(np.abs(yo))


def test_adjoint_dot_identity():
    inp, dy, dhf = rand_case(3, B=2, L=16, D=4, N=5)
    g = bwd(inp, dy, dhf)
    rng = np.random.default_rng(33)
    v = {k: rng.standard_normal(np.shape(val)) for k, val in inp.items()}
    prim = tuple(torch.tensor(inp[k]) for k in NAMES)
    tang = tuple(torch.tensor(v[k]) for k in NAMES)

    def f(*args):
        return torch_loop(dict(zip(NAMES, args)))

    _, (jy, jh) = torch.func.jvp(f, prim, tang)
    lhs = float(np.sum(dy * jy.numpy()) + np.sum(dhf * jh.numpy()))
    rhs = float(sum(np.sum(g[GRAD_OF[k]] * v[k]) for k in NAMES))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_reduction_invariants():
    inp, dy, dhf = rand_case(4, B=3, L=20, D=4, N=3)
    g = bwd(inp, dy, dhf)
    # ddt_bias is the sum of ddelta over batch and time (bias enters additively)
    assert np.allclose(g["ddt_bias"], g["ddelta"].sum((0, 1)), rtol=1e-13, atol=1e-13)
    # dDskip = sum over (b, t) of (dy * silu(z)) * u
    z = inp["z"]
    sbar = dy * z / (1 + np.exp(-z))
    assert np.allclose(g["dD"], (sbar * inp["u"]).sum((0, 1)), rtol=1e-13, atol=1e-13)


def test_no_gate_A_zero_closed_form():
    """A = 0, no gate, no dh_final: lambda_t = sum_{t'>=t} dy_t' Cm_t', so
    du_t = Dskip dy_t + Delta_t sum_n Bm_{t,n} lambda_{t,n} and
    dB_{t,n} = sum_d lambda_{t,n}[d] Delta_t[d] u_t[d] in closed form."""
    inp, dy, _ = rand_case(5, B=2, L=12, D=3, N=4)
    inp["A"] = np.zeros_like(inp["A"])
    inp["z"] = None
    g = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                        Dskip=inp["Dskip"], z=None, dt_bias=inp["dt_bias"], h0=inp["h0"])
    x = inp["delta"] + inp["dt_bias"]
    dt = np.logaddexp(0.0, x)
    lam = np.flip(np.cumsum(np.flip(dy[..., None] * inp["Cm"][:, :, None, :], 1), 1), 1)  # (B,L,D,N)
    du = inp["Dskip"] * dy + dt * np.einsum("bldn,bln->bld", lam, inp["Bm"])
    dB = np.einsum("bldn,bld->bln", lam, dt * inp["u"])
    assert np.allclose(g["du"], du, rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dB"], dB, rtol=1e-12, atol=1e-12)
    assert g["dz"] is None
    # dh0 = lambda_0 (decay is 1 when A = 0)
    assert np.allclose(g["dh0"], lam[:, 0], rtol=1e-12, atol=1e-12)
