"""The Mamba-2 (SSD) reading and its chunked dual form, on the CPU.

Reading: the pages name Mamba-2 without defining it; the plainest reading
consistent with the selective scan they do define is the same recurrence with
one scalar decay per head (A[d, n] = A_h for every state n of every channel d
of head h), one step size per head (Delta shared by the head's P channels) and
Bm, Cm shared by all heads.  With channel d = (h, p) it is exactly the
selective scan, so the float64 scan oracle is its oracle (``oracle.ssd_fwd``
only rearranges arrays).

The GPU kernel computes it in the chunked dual form: per chunk of Q steps with
local cumulative log-decay cum_i = sum_{j <= i} Delta_j A_h,
    Y = (G o L) X + diag(exp(cum)) C S_in^T + D X,   G = C B^T,
        L_ij = exp(cum_i - cum_j) Delta_j for j <= i, else 0,
    S_out = exp(cum_{Q-1}) S_in + (w o X)^T B,  w_j = exp(cum_{Q-1} - cum_j) Delta_j.
``chunked_dual`` writes that out in float64 numpy; the test checks it against
the oracle, so the formulas the kernel implements are pinned to the
recurrence before any GPU runs.
"""
import numpy as np
import pytest

import oracle


def chunked_dual(x, dt, A, Bm, Cm, Dh, dt_bias, h0, Q, softplus=True):
    B, L, H, P = x.shape
    N = Bm.shape[2]
    xx = dt + dt_bias[None, None, :]
    delta = np.maximum(xx, 0) + np.log1p(np.exp(-np.abs(xx))) if softplus else xx
    y = np.zeros((B, L, H, P))
    hf = np.zeros((B, H, P, N))
    for b in range(B):
        for h in range(H):
            S = h0[b, h].copy()  # (P, N)
            for t0 in range(0, L, Q):
                n = min(Q, L - t0)
                d = delta[b, t0:t0 + n, h]
                cum = np.cumsum(d * A[h])
                X = x[b, t0:t0 + n, h]            # (n, P)
                Bc, Cc = Bm[b, t0:t0 + n], Cm[b, t0:t0 + n]  # (n, N)
                G = Cc @ Bc.T
                Lm = np.tril(np.exp(cum[:, None] - cum[None, :])) * d[None, :]
                Y = (G * Lm) @ X + np.exp(cum)[:, None] * (Cc @ S.T) + Dh[h] * X
                w = np.exp(cum[-1] - cum) * d
                S = np.exp(cum[-1]) * S + (w[:, None] * X).T @ Bc
                y[b, t0:t0 + n, h] = Y
            hf[b, h] = S
    return y, hf


@pytest.mark.parametrize("L,Q", [(1, 64), (64, 64), (150, 64), (37, 8)])
def test_chunked_dual_form_equals_the_recurrence(L, Q):
    rng = np.random.default_rng(L + Q)
    B, H, P, N = 2, 3, 4, 5
    x = rng.standard_normal((B, L, H, P))
    dt = 0.5 * rng.standard_normal((B, L, H))
    A = -np.exp(rng.standard_normal(H))
    Bm, Cm = rng.standard_normal((B, L, N)), rng.standard_normal((B, L, N))
    Dh, bias = rng.standard_normal(H), rng.standard_normal(H) - 2.0
    h0 = rng.standard_normal((B, H, P, N))
    yr, hr = oracle.ssd_fwd(x, dt, A, Bm, Cm, Dh, bias, h0)
    yc, hc = chunked_dual(x, dt, A, Bm, Cm, Dh, bias, h0, Q)
    np.testing.assert_allclose(yc, yr, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(hc, hr, rtol=1e-10, atol=1e-10)


def test_per_head_scalar_decay_is_the_scan_with_constant_A_rows():
    # the reduction itself: per channel d = (h, p) the oracle sees A[d, n] = A_h for every n, so each state's
    # decay over a step is the same exp(Delta A_h) -- the closed form of one step checks it
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 1, 2, 3))
    dt = np.array([[[0.3, -0.4]]])
    A = np.array([-0.7, -1.9])
    Bm, Cm = rng.standard_normal((1, 1, 4)), rng.standard_normal((1, 1, 4))
    h0 = rng.standard_normal((1, 2, 3, 4))
    y, hf = oracle.ssd_fwd(x, dt, A, Bm, Cm, None, None, h0, softplus=False)
    for h in range(2):
        a = np.exp(dt[0, 0, h] * A[h])
        want = a * h0[0, h] + dt[0, 0, h] * x[0, 0, h][:, None] * Bm[0, 0][None, :]
        np.testing.assert_allclose(hf[0, h], want, rtol=1e-14)
        np.testing.assert_allclose(y[0, 0, h], want @ Cm[0, 0], rtol=1e-13)
