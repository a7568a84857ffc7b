"""Pins of the oracle's causal conv1d + SiLU front end (CPU only).

The front end is the Mamba block's depthwise causal convolution over time
(kernel size d_conv, 4 in the configurations of the page "Mamba SSM 架构";
the mamba-minimal page "PyTorch 한 파일에서의 Mamba 구현" runs it as
torch.nn.Conv1d) followed by SiLU.  ``oracle.causal_conv_silu`` writes the
sum out tap by tap; each pin below reaches the same numbers by another route:

* numpy's full convolution (``np.convolve``) of each channel with the reversed
  kernel, sliced to the causal outputs;
* ``torch.nn.functional.conv1d`` in float64 on the CPU with groups = D and
  d_conv - 1 steps of left padding, truncated to L outputs -- the layer the
  pages name, as a library routine;
* SiLU against scipy's logistic function, and its special values;
* impulse kernels (identity and pure delay) and streaming continuity (a
  sequence cut in two, the second part given the first part's last inputs).

The last test plants plausible mistakes in a copy of the oracle's function and
checks that a pin catches each.
"""
import inspect
import textwrap

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(2024)


def case(B=2, L=13, D=5, K=4, prev=True):
    x = RNG.standard_normal((B, L, D))
    w = RNG.standard_normal((D, K))
    b = RNG.standard_normal(D)
    xp = RNG.standard_normal((B, K - 1, D)) if prev else None
    return x, w, b, xp


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("prev", [True, False])
def test_against_numpy_convolve(K, prev):
    x, w, b, xp = case(K=K, prev=prev)
    c = oracle.causal_conv_silu(x, w, b, xp, silu=False)
    B, L, D = x.shape
    xx = np.concatenate([xp if prev else np.zeros((B, K - 1, D)), x], axis=1)
    for bb in range(B):
        for d in range(D):
            full = np.convolve(xx[bb, :, d], w[d, ::-1])      # full[n] = sum_m xx[m] w[K-1-(n-m)]
            ref = full[K - 1:K - 1 + L] + b[d]
            np.testing.assert_allclose(c[bb, :, d], ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("K", [2, 4])
def test_against_torch_conv1d(K):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    x, w, b, xp = case(B=3, L=21, D=7, K=K)
    B, L, D = x.shape
    xt = torch.from_numpy(x).transpose(1, 2)                 # (B, D, L), as nn.Conv1d takes it
    wt = torch.from_numpy(w).reshape(D, 1, K)                # nn.Conv1d(D, D, K, groups=D).weight
    bt = torch.from_numpy(b)
    # zero history: the layer's own left padding, outputs truncated to L
    ref0 = F.conv1d(xt, wt, bt, padding=K - 1, groups=D)[..., :L].transpose(1, 2).numpy()
    np.testing.assert_allclose(oracle.causal_conv_silu(x, w, b, silu=False), ref0, rtol=0, atol=1e-13)
    # given history: the layer over the history and the sequence, no padding
    xxt = torch.from_numpy(np.concatenate([xp, x], axis=1)).transpose(1, 2)
    ref1 = F.conv1d(xxt, wt, bt, groups=D).transpose(1, 2).numpy()
    np.testing.assert_allclose(oracle.causal_conv_silu(x, w, b, xp, silu=False), ref1, rtol=0, atol=1e-13)
    # the (D, 1, K) weight layout is accepted as it is
    np.testing.assert_allclose(oracle.causal_conv_silu(x, wt.numpy(), b, xp), oracle.causal_conv_silu(x, w, b, xp),
                               rtol=0, atol=0)


def test_silu():
    from scipy.special import expit
    x, w, b, xp = case()
    c = oracle.causal_conv_silu(x, w, b, xp, silu=False)
    np.testing.assert_allclose(oracle.causal_conv_silu(x, w, b, xp), c * expit(c), rtol=1e-14, atol=1e-15)
    # special values of silu(c) = c * sigmoid(c): 0 at 0, c for large c, -> 0 for very negative c
    one = np.ones((1, 1))
    for cv, want in ((0.0, 0.0), (50.0, 50.0), (-50.0, -50.0 * np.exp(-50.0))):
        u = oracle.causal_conv_silu(np.zeros((1, 1, 1)), one, np.array([cv]))
        assert abs(u[0, 0, 0] - want) <= 1e-15 * max(1.0, abs(want)), (cv, u)


def test_impulse_kernels():
    x, _, b, xp = case(K=4)
    B, L, D = x.shape
    ident = np.zeros((D, 4))
    ident[:, 3] = 1.0                                        # tap on the current input
    np.testing.assert_array_equal(oracle.causal_conv_silu(x, ident, b, xp, silu=False), x + b)
    delay = np.zeros((D, 4))
    delay[:, 0] = 1.0                                        # tap on the input 3 steps back
    c = oracle.causal_conv_silu(x, delay, b, xp, silu=False)
    np.testing.assert_array_equal(c[:, 3:], x[:, :-3] + b)
    np.testing.assert_array_equal(c[:, :3], xp + b)
    np.testing.assert_array_equal(oracle.causal_conv_silu(x, delay, None, None, silu=False)[:, :3], 0.0)


def test_streaming_continuity():
    x, w, b, xp = case(L=30, K=4)
    whole = oracle.causal_conv_silu(x, w, b, xp)
    for cut in (1, 2, 3, 17):
        first = oracle.causal_conv_silu(x[:, :cut], w, b, xp)
        hist = np.concatenate([xp, x[:, :cut]], axis=1)[:, -3:]
        second = oracle.causal_conv_silu(x[:, cut:], w, b, hist)
        np.testing.assert_allclose(np.concatenate([first, second], axis=1), whole, rtol=0, atol=1e-15)


CONV_PINS = [lambda: test_against_numpy_convolve(4, True), lambda: test_against_numpy_convolve(3, False),
             lambda: test_against_torch_conv1d(4), test_silu, test_impulse_kernels]

MUTATIONS = {
    "kernel not reversed (convolution instead of correlation)": ("c += weight[:, k] * xx[:, k:k + L, :]",
                                                                 "c += weight[:, K - 1 - k] * xx[:, k:k + L, :]"),
    "off by one step": ("c += weight[:, k] * xx[:, k:k + L, :]", "c += weight[:, k] * xx[:, k - 1:k - 1 + L, :]"),
    "bias dropped": ("c = np.zeros((Bsz, L, D)) if bias is None else", "c = np.zeros((Bsz, L, D)) if True else"),
    "sigmoid instead of silu": ("return c / (1.0 + np.exp(-c))", "return 1.0 / (1.0 + np.exp(-c))"),
    "history ignored": ("xx = np.concatenate([x_prev, x], axis=1)",
                        "xx = np.concatenate([np.zeros_like(x_prev), x], axis=1)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_conv_mutation(name, monkeypatch):
    old, new = MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(oracle.causal_conv_silu))
    assert src.count(old) == 1, "mutation anchor not found: " + old
    ns = {"np": np, "_f64": oracle._f64}
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oracle, "causal_conv_silu", ns["causal_conv_silu"])
    failed = 0
    for pin in CONV_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed += 1
    assert failed >= 1, f"no pin caught the mutation '{name}'"


# ---- the adjoint (oracle.causal_conv_silu_bwd) -------------------------------------------------

@pytest.mark.parametrize("K,prev", [(4, True), (4, False), (3, True), (1, False)])
def test_backward_against_torch_autograd(K, prev):
    """torch.autograd in float64 through the layer the pages name
    (torch.nn.functional.conv1d, groups = D, over history + sequence) and
    SiLU: a library route to every gradient."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    x, w, b, xp = case(B=2, L=11, D=3, K=K, prev=prev)
    B, L, D = x.shape
    du = RNG.standard_normal((B, L, D))
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    xpt = torch.tensor(xp if prev else np.zeros((B, K - 1, D)), requires_grad=True)
    xx = torch.cat([xpt, xt], 1).transpose(1, 2)
    u = F.silu(F.conv1d(xx, wt.reshape(D, 1, K), bt, groups=D)).transpose(1, 2)
    (u * torch.tensor(du)).sum().backward()
    g = oracle.causal_conv_silu_bwd(x, w, du, b, xp if prev else None)
    np.testing.assert_allclose(g["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dweight"], wt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dbias"], bt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dx_prev"], xpt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_backward_finite_differences():
    x, w, b, xp = case(B=1, L=6, D=2, K=4)
    du = RNG.standard_normal(x.shape)
    g = oracle.causal_conv_silu_bwd(x, w, du, b, xp)
    loss = lambda x_, w_, b_, p_: float(np.sum(du * oracle.causal_conv_silu(x_, w_, b_, p_)))  # noqa: E731
    eps = 1e-6
    for name, arr, grad, pos in (("dx", x, g["dx"], lambda a: (a, w, b, xp)),
                                 ("dweight", w, g["dweight"], lambda a: (x, a, b, xp)),
                                 ("dbias", b, g["dbias"], lambda a: (x, w, a, xp)),
                                 ("dx_prev", xp, g["dx_prev"], lambda a: (x, w, b, a))):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            num[idx] = (loss(*pos(p)) - loss(*pos(m))) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_invariants():
    """dbias is the sum of dx over the sequence and history for an identity
    kernel scaled by one; with a pure delay, dx is g shifted back."""
    x, _, b, xp = case(K=4)
    du = RNG.standard_normal(x.shape)
    delay = np.zeros((x.shape[2], 4))
    delay[:, 0] = 1.0
    g = oracle.causal_conv_silu_bwd(x, delay, du, b, xp)
    c = oracle.causal_conv_silu(x, delay, b, xp, silu=False)
    from scipy.special import expit
    gg = du * (expit(c) * (1 + c * (1 - expit(c))))
    np.testing.assert_allclose(g["dx"][:, :-3], gg[:, 3:], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(g["dx"][:, -3:], 0.0)
    np.testing.assert_allclose(g["dx_prev"], gg[:, :3], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(g["dbias"], gg.sum(axis=(0, 1)), rtol=1e-13)


BWD_CONV_PINS = [lambda: test_backward_against_torch_autograd(4, True), test_backward_invariants]

BWD_MUTATIONS = {
    "silu derivative without the c term": ("g = du * s * (1.0 + c * (1.0 - s))", "g = du * s"),
    "dx stencil not transposed": ("dxx[:, k:k + L, :] += weight[:, k] * g", "dxx[:, k:k + L, :] += weight[:, K - 1 - k] * g"),
    "dweight against the wrong tap": ("dw[:, k] = np.sum(g * xx[:, k:k + L, :], axis=(0, 1))",
                                      "dw[:, k] = np.sum(g * xx[:, K - 1:K - 1 + L, :], axis=(0, 1))"),
    "history gradient dropped": ('"dx_prev": dxx[:, :K - 1]', '"dx_prev": 0.0 * dxx[:, :K - 1]'),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_pins_catch_conv_backward_mutation(name, monkeypatch):
    old, new = BWD_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(oracle.causal_conv_silu_bwd))
    assert src.count(old) == 1, "mutation anchor not found: " + old
    ns = {"np": np, "_f64": oracle._f64, "causal_conv_silu": oracle.causal_conv_silu}
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oracle, "causal_conv_silu_bwd", ns["causal_conv_silu_bwd"])
    failed = 0
    for pin in BWD_CONV_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed += 1
    assert failed >= 1, f"no pin caught the mutation '{name}'"
