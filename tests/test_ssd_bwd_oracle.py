"""Pins of the float64 oracle's Mamba-2 (SSD) backward, ``oracle.ssd_bwd``.

The reading (the pages name Mamba-2 without equations): the selective scan
with one scalar decay A_h and one step size per head, shared by the head's P
channels and N states, and Bm, Cm shared by all heads.  The oracle's adjoint
is the scan's on the flattened channels with the tied gradients summed.
Pinned against routes that share nothing with it:

* central finite differences of the oracle's forward ``ssd_fwd`` (float64,
  step 1e-6), for every input, with every optional input present, with and
  without softplus;
* torch.autograd (CPU, float64) through a plain PyTorch loop of the per-head
  recurrence, written here from the definition;
* invariants: ddt_bias[h] = sum over (b, t) of ddt[b, t, h] (the step size and
  its bias enter only as their sum); dDskip[h] = sum of dy * x over (b, t, p);
  dh0 = 0 when no output depends on the state (dy = 0, no dh_final).

It also checks the chunked dual form of the backward -- the formulas the GPU
kernel computes chunk by chunk (``chunked_dual_bwd`` below) -- against the
oracle, so those formulas are pinned before any kernel runs.
"""
import numpy as np
import pytest
import torch

import oracle

NAMES = ["x", "dt", "A", "Bm", "Cm", "Dskip", "dt_bias", "h0"]
GRAD_OF = {"x": "dx", "dt": "ddt", "A": "dA", "Bm": "dB", "Cm": "dC", "Dskip": "dD",
           "dt_bias": "ddt_bias", "h0": "dh0"}


def rand_case(seed, B=2, L=9, H=2, P=3, N=4, softplus=True):
    rng = np.random.default_rng(seed)
    dtv = np.exp(rng.uniform(np.log(2e-2), np.log(3e-1), size=H))
    inp = dict(
        x=rng.standard_normal((B, L, H, P)),
        dt=0.5 * rng.standard_normal((B, L, H)) if softplus else rng.uniform(0.01, 0.3, size=(B, L, H)),
        A=-rng.uniform(0.2, 3.0, size=H), Bm=rng.standard_normal((B, L, N)), Cm=rng.standard_normal((B, L, N)),
        Dskip=rng.standard_normal(H), dt_bias=np.log(np.expm1(dtv)) if softplus else rng.uniform(0, 0.1, size=H),
        h0=rng.standard_normal((B, H, P, N)),
    )
    return inp, rng.standard_normal((B, L, H, P)), rng.standard_normal((B, H, P, N))


def loss(inp, dy, dhf, softplus=True):
    y, hf = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["Dskip"], inp["dt_bias"],
                           inp["h0"], softplus=softplus)
    return float((y * dy).sum() + (hf * dhf).sum())


def grads(inp, dy, dhf, softplus=True):
    return oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], dy, Dskip=inp["Dskip"],
                          dt_bias=inp["dt_bias"], h0=inp["h0"], dh_final=dhf, softplus=softplus)


@pytest.mark.parametrize("softplus", [True, False])
def test_finite_differences(softplus):
    inp, dy, dhf = rand_case(3 if softplus else 4, softplus=softplus)
    g = grads(inp, dy, dhf, softplus)
    eps = 1e-6
    for name in NAMES:
        a = inp[name]
        fd = np.empty_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + eps
            lp = loss(inp, dy, dhf, softplus)
            a[idx] = old - eps
            lm = loss(inp, dy, dhf, softplus)
            a[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        got = g[GRAD_OF[name]]
        scale = max(1.0, float(np.abs(fd).max()))
        assert np.abs(got - fd).max() <= 2e-6 * scale, name


def torch_ssd(t, softplus):
    """The per-head recurrence, written from its definition as a plain PyTorch loop."""
    x, A, Bm, Cm, D, h = t["x"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["h0"]
    v = t["dt"] + t["dt_bias"]
    delta = torch.logaddexp(v, torch.zeros_like(v)) if softplus else v  # softplus without a threshold
    ys = []
    for i in range(x.shape[1]):
        a = torch.exp(delta[:, i] * A)                                      # (B, H)
        h = a[:, :, None, None] * h + (delta[:, i, :, None] * x[:, i])[..., None] * Bm[:, i, None, None, :]
        ys.append((h * Cm[:, i, None, None, :]).sum(-1) + D[None, :, None] * x[:, i])
    return torch.stack(ys, 1), h


@pytest.mark.parametrize("softplus", [True, False])
def test_autograd(softplus):
    inp, dy, dhf = rand_case(11 if softplus else 12, L=13, H=3, softplus=softplus)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp.items()}
    y, hf = torch_ssd(t, softplus)
    ((y * torch.tensor(dy)).sum() + (hf * torch.tensor(dhf)).sum()).backward()
    g = grads(inp, dy, dhf, softplus)
    for name in NAMES:
        ref = t[name].grad.numpy()
        assert np.abs(g[GRAD_OF[name]] - ref).max() <= 1e-11 * max(1.0, float(np.abs(ref).max())), name


def test_invariants():
    inp, dy, dhf = rand_case(21, B=3, L=11, H=2, P=4, N=3)
    g = grads(inp, dy, dhf)
    np.testing.assert_allclose(g["ddt_bias"], g["ddt"].sum((0, 1)), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dD"], (dy * inp["x"]).sum((0, 1, 3)), rtol=1e-12, atol=1e-12)
    z = grads(inp, np.zeros_like(dy), None)
    assert np.abs(z["dh0"]).max() == 0.0 and np.abs(z["dx"]).max() == 0.0


def chunked_dual_bwd(x, dt, A, Bm, Cm, dy, Dh, bias, h0, dhf, Q, softplus=True):
    """The SSD backward in chunks of Q steps (float64 numpy), per (batch, head):
    a forward sweep forms the state entering each chunk; a reverse sweep carries
    dS (the adjoint of the state leaving the chunk) and per chunk, with local
    cum_i = sum_{s<=i} Delta_s A, G = C B^T, Lmask_ij = exp(cum_i - cum_j) Delta_j
    (j <= i), U_jk = exp(cum_k - cum_j) (k >= j), e_j = exp(cum_last - cum_j):
        dC   = diag(exp(cum)) dY S_in + ((dY X^T) o Lmask) B
        V    = (G^T o U) dY + diag(e) B dS^T          (V_j = lambda_j B_j)
        dX   = diag(Delta) V + D dY
        dB   = diag(Delta) [((X dY^T) o U) C + diag(e) X dS]
        r_i  = x_i . V_i ;  dcum_i = C_i . dC_i - Delta_i r_i  (+ <dS, S_out> at the last row)
        dDelta_t = A sum_{i >= t} dcum_i + r_t ;  dA += sum_i dcum_i sum_{s<=i} Delta_s
        dS_in = dY^T diag(exp(cum)) C + exp(cum_last) dS."""
    B, L, H, P = x.shape
    N = Bm.shape[2]
    v = dt + bias[None, None, :]
    delta = np.logaddexp(v, 0.0) if softplus else v
    sig = 1.0 / (1.0 + np.exp(-v)) if softplus else np.ones_like(v)
    out = {"dx": np.zeros_like(x), "ddt": np.zeros_like(dt), "dA": np.zeros(H), "dB": np.zeros_like(Bm),
           "dC": np.zeros_like(Cm), "dD": np.zeros(H), "dh0": np.zeros((B, H, P, N))}
    for b in range(B):
        for h in range(H):
            starts = list(range(0, L, Q))
            states = [h0[b, h].copy()]
            for t0 in starts:
                d = delta[b, t0:t0 + Q, h]
                cum = np.cumsum(d * A[h])
                X, Bc = x[b, t0:t0 + Q, h], Bm[b, t0:t0 + Q]
                w = np.exp(cum[-1] - cum) * d
                states.append(np.exp(cum[-1]) * states[-1] + (w[:, None] * X).T @ Bc)
            dS = dhf[b, h].copy()
            for c in reversed(range(len(starts))):
                t0 = starts[c]
                d = delta[b, t0:t0 + Q, h]
                n = len(d)
                cum = np.cumsum(d * A[h])
                X, Bc, Cc, dY = x[b, t0:t0 + n, h], Bm[b, t0:t0 + n], Cm[b, t0:t0 + n], dy[b, t0:t0 + n, h]
                S_in, S_out = states[c], states[c + 1]
                G = Cc @ Bc.T
                tri = np.tril(np.ones((n, n), bool))
                Lm = np.where(tri, np.exp(cum[:, None] - cum[None, :]), 0.0) * d[None, :]
                U = np.where(tri.T, np.exp(cum[None, :] - cum[:, None]), 0.0)
                e = np.exp(cum[-1] - cum)
                dYX = dY @ X.T
                dC = np.exp(cum)[:, None] * (dY @ S_in) + (dYX * Lm) @ Bc
                V = (G.T * U) @ dY + e[:, None] * (Bc @ dS.T)
                dX = d[:, None] * V + Dh[h] * dY
                dBc = d[:, None] * ((dYX.T * U) @ Cc + e[:, None] * (X @ dS))
                r = (X * V).sum(1)
                dcum = (Cc * dC).sum(1) - d * r
                dcum[-1] += (dS * S_out).sum()
                dDelta = A[h] * np.cumsum(dcum[::-1])[::-1] + r
                out["dA"][h] += (dcum * np.cumsum(d)).sum()
                out["dx"][b, t0:t0 + n, h] = dX
                out["ddt"][b, t0:t0 + n, h] = dDelta * sig[b, t0:t0 + n, h]
                out["dB"][b, t0:t0 + n] += dBc
                out["dC"][b, t0:t0 + n] += dC
                out["dD"][h] += (dY * X).sum()
                dS = dY.T @ (np.exp(cum)[:, None] * Cc) + np.exp(cum[-1]) * dS
            out["dh0"][b, h] = dS
    out["ddt_bias"] = out["ddt"].sum((0, 1))
    return out


@pytest.mark.parametrize("L,Q,softplus", [(1, 64, True), (64, 64, True), (150, 64, True), (37, 8, False),
                                          (40, 8, True)])
def test_chunked_dual_backward_equals_the_oracle(L, Q, softplus):
    inp, dy, dhf = rand_case(L + Q, B=2, L=L, H=3, P=4, N=5, softplus=softplus)
    r = grads(inp, dy, dhf, softplus)
    c = chunked_dual_bwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], dy, inp["Dskip"], inp["dt_bias"],
                         inp["h0"], dhf, Q, softplus)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "ddt_bias", "dh0"):
        ref = r[k]
        assert np.abs(c[k] - ref).max() <= 1e-10 * max(1.0, float(np.abs(ref).max())), k
