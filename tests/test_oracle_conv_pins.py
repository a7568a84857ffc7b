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
