"""Float64 CPU oracle of the Mamba selective scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU product path
(``selective_state_space_mssm_amd``) never imports it, and this package imports
nothing from the product path: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, float64, sequential in time,
OpenMP over independent (batch, channel) rows).  This module only converts
arrays to float64 -- exactly, since every stored float32/bfloat16 value is a
float64 value -- and calls it.

What the oracle computes is the sequential loop of the mamba-minimal page
("PyTorch 한 파일에서의 Mamba 구현", Hacker News comments), with the
discretisation, skip term, gate and step-size transform of the selective SSM
(Mamba paper Section 3 / Algorithm 2, named on the page "Mamba SSM 架构");
``oracle.c`` states the formulas.

The Mamba block's causal conv1d + SiLU, which produces the scan's u (the
fused front end of ``mssm_conv_scan_fwd``), is ``causal_conv_silu`` below,
written out in numpy: a depthwise convolution of kernel size d_conv over
time, causal (output t sees inputs t - d_conv + 1 .. t), with bias, as
torch.nn.Conv1d(groups=D, padding=d_conv - 1) truncated to the first L
outputs -- the layer the mamba-minimal page runs in place of the CUDA conv,
with d_conv = 4 in the configurations of the page "Mamba SSM 架构".

Mamba-2's layer (``ssd_fwd``), which the pages name without equations, is
read as the same scan with one scalar decay and one step size per head,
shared by the head's channels and states, and Bm, Cm shared by all heads; the
oracle runs it through ``scan_fwd`` on the flattened channels.

Its backward (``ssd_bwd``) is the chain rule through that tying: the scan's
adjoint on the flattened channels, the gradients of the shared step size,
decay, skip and bias summed over the channels (and states) that share them.

Pinning (what checks this oracle against something other than itself) is in
``tests/test_oracle_fwd_pins.py``, ``tests/test_oracle_bwd_pins.py``,
``tests/test_oracle_conv_pins.py``, ``tests/test_ssd_dual_form.py`` and
``tests/test_ssd_bwd_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCE = os.path.join(_HERE, "oracle.c")

_lib = None


def build(verbose: bool = False, source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (-O2, no fast-math)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", out, source, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


def open_library(path: str):
    """Open a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_scan_fwd.argtypes = [i64, i64, i64, i64, i32] + [p] * 11
    lib.oracle_scan_fwd.restype = None
    lib.oracle_step.argtypes = [i64, i64, i64, i32] + [p] * 10
    lib.oracle_step.restype = None
    lib.oracle_scan_bwd.argtypes = [i64, i64, i64, i64, i32] + [p] * 20
    lib.oracle_scan_bwd.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = open_library(LIB_PATH)
    return _lib


def num_threads() -> int:
    """Threads the oracle's parallel loops use on this host."""
    return int(_load().oracle_num_threads())


def _f64(x):
    """Exact float64 copy of an input (numpy array or CPU/GPU torch tensor)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16/fp32 -> fp64 is exact
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan_fwd(u, delta, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, h0=None,
             softplus=True):
    """Return ``(y, h_final)`` in float64 for inputs of shapes
    u, delta, z: (B, L, D); Bm, Cm: (B, L, N); A: (D, N); Dskip, dt_bias: (D);
    h0: (B, D, N)."""
    u, delta, A, Bm, Cm = map(_f64, (u, delta, A, Bm, Cm))
    Dskip, z, dt_bias, h0 = map(_f64, (Dskip, z, dt_bias, h0))
    Bsz, L, D = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (D, N)
    assert Bm.shape == (Bsz, L, N) and Cm.shape == (Bsz, L, N)
    assert z is None or z.shape == u.shape
    assert h0 is None or h0.shape == (Bsz, D, N)
    y = np.empty((Bsz, L, D), np.float64)
    hf = np.empty((Bsz, D, N), np.float64)
    _load().oracle_scan_fwd(Bsz, L, D, N, int(bool(softplus)), _ptr(u), _ptr(delta),
                            _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
                            _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(hf))
    return y, hf


def causal_conv_silu(x, weight, bias=None, x_prev=None, silu=True):
    """u[b,t,d] = silu(bias[d] + sum_k weight[d,k] * x[b, t - K + 1 + k, d]) in
    float64, K = d_conv.  x: (B, L, D); weight: (D, K) (or (D, 1, K), the
    torch.nn.Conv1d layout); bias: (D); x_prev: (B, K - 1, D), the inputs at
    t = -(K - 1) .. -1, zeros when None (the left padding).  silu=False returns
    the convolution alone."""
    x, weight, bias, x_prev = map(_f64, (x, weight, bias, x_prev))
    Bsz, L, D = x.shape
    weight = weight.reshape(D, -1)
    K = weight.shape[1]
    if x_prev is None:
        x_prev = np.zeros((Bsz, K - 1, D))
    assert x_prev.shape == (Bsz, K - 1, D)
    xx = np.concatenate([x_prev, x], axis=1)          # time -(K-1) .. L-1
    c = np.zeros((Bsz, L, D)) if bias is None else np.broadcast_to(bias, (Bsz, L, D)).copy()
    for k in range(K):                                 # tap k sees input t - (K - 1) + k
        c += weight[:, k] * xx[:, k:k + L, :]
    if not silu:
        return c
    return c / (1.0 + np.exp(-c))


def causal_conv_silu_bwd(x, weight, du, bias=None, x_prev=None):
    """Adjoint of ``causal_conv_silu`` in float64: given du = dL/du, returns a
    dict with dx (B, L, D), dweight (D, K), dbias (D) and dx_prev (B, K - 1, D).
    With c the convolution and g = du * silu'(c), silu'(c) = s (1 + c (1 - s)),
    s = sigmoid(c): dbias = sum_{b,t} g, dweight[d,k] = sum_{b,t} g[t] xx[t+k]
    and dxx[tau] = sum_k weight[d,k] g[tau - k] over the history and the
    sequence together (xx, time -(K - 1) .. L - 1), split into dx_prev and dx."""
    x, weight, du, bias, x_prev = map(_f64, (x, weight, du, bias, x_prev))
    Bsz, L, D = x.shape
    weight = weight.reshape(D, -1)
    K = weight.shape[1]
    if x_prev is None:
        x_prev = np.zeros((Bsz, K - 1, D))
    xx = np.concatenate([x_prev, x], axis=1)
    c = causal_conv_silu(x, weight, bias, x_prev, silu=False)
    s = 1.0 / (1.0 + np.exp(-c))
    g = du * s * (1.0 + c * (1.0 - s))
    dxx = np.zeros_like(xx)
    dw = np.zeros((D, K))
    for k in range(K):                                 # c[t] took weight[:, k] * xx[t + k]
        dxx[:, k:k + L, :] += weight[:, k] * g
        dw[:, k] = np.sum(g * xx[:, k:k + L, :], axis=(0, 1))
    return {"dx": dxx[:, K - 1:], "dweight": dw, "dbias": g.sum(axis=(0, 1)), "dx_prev": dxx[:, :K - 1]}


def conv_scan_fwd(x, weight, delta, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, h0=None,
                  bias=None, x_prev=None, softplus=True):
    """The scan behind the conv front end: ``(y, h_final, u)`` in float64 with
    u = causal_conv_silu(x, weight, bias, x_prev) fed to ``scan_fwd``."""
    u = causal_conv_silu(x, weight, bias, x_prev)
    y, hf = scan_fwd(u, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, softplus=softplus)
    return y, hf, u


def ssd_fwd(x, dt, A, Bm, Cm, Dskip=None, dt_bias=None, h0=None, softplus=True):
    """Mamba-2 (state-space dual) forward in float64, as the selective scan
    over channels d = (h, p) with A[d, n] = A[h], delta[b,t,d] = dt[b,t,h],
    Dskip[d] = Dskip[h], dt_bias[d] = dt_bias[h] (the pages name Mamba-2 in the
    model list of "mamba.py: 一个简单高效的Mamba实现" and the versions paragraph
    of "Mamba SSM 架构"; this per-head scalar-decay reading is the library's).
    x (B, L, H, P); dt (B, L, H); A, Dskip, dt_bias (H); Bm, Cm (B, L, N);
    h0 (B, H, P, N).  Returns ``(y (B, L, H, P), h_final (B, H, P, N))``."""
    x, dt, A, Bm, Cm = _f64(x), _f64(dt), _f64(A), _f64(Bm), _f64(Cm)
    B, L, H, P = x.shape
    N = Bm.shape[2]
    rep = lambda v: None if v is None else np.repeat(_f64(v), P, axis=-1)  # noqa: E731
    y, hf = scan_fwd(x.reshape(B, L, H * P), rep(dt), np.repeat(A, P)[:, None] * np.ones((1, N)), Bm, Cm,
                     rep(Dskip), None, rep(dt_bias), None if h0 is None else _f64(h0).reshape(B, H * P, N),
                     softplus=softplus)
    return y.reshape(B, L, H, P), hf.reshape(B, H, P, N)


def step(u_t, delta_t, A, Bm_t, Cm_t, state, Dskip=None, z_t=None, dt_bias=None,
         softplus=True):
    """One recurrent step.  u_t, delta_t, z_t: (B, D); Bm_t, Cm_t: (B, N);
    state: (B, D, N).  Returns ``(y_t, new_state)`` (the input is not modified)."""
    u_t, delta_t, A, Bm_t, Cm_t = map(_f64, (u_t, delta_t, A, Bm_t, Cm_t))
    Dskip, z_t, dt_bias = map(_f64, (Dskip, z_t, dt_bias))
    st = _f64(state).copy()
    Bsz, D = u_t.shape
    N = A.shape[1]
    y = np.empty((Bsz, D), np.float64)
    _load().oracle_step(Bsz, D, N, int(bool(softplus)), _ptr(u_t), _ptr(delta_t),
                        _ptr(A), _ptr(Bm_t), _ptr(Cm_t), _ptr(Dskip), _ptr(z_t),
                        _ptr(dt_bias), _ptr(st), _ptr(y))
    return y, st


def scan_bwd(u, delta, A, Bm, Cm, dy, Dskip=None, z=None, dt_bias=None, h0=None,
             dh_final=None, softplus=True):
    """Analytic adjoint.  Returns a dict with du, ddelta, dA, dB, dC, dD, dz,
    ddt_bias, dh0 (float64; dz is None without a gate)."""
    u, delta, A, Bm, Cm, dy = map(_f64, (u, delta, A, Bm, Cm, dy))
    Dskip, z, dt_bias, h0, dh_final = map(_f64, (Dskip, z, dt_bias, h0, dh_final))
    Bsz, L, D = u.shape
    N = A.shape[1]
    out = {
        "du": np.empty((Bsz, L, D)), "ddelta": np.empty((Bsz, L, D)),
        "dA": np.empty((D, N)), "dB": np.empty((Bsz, L, N)), "dC": np.empty((Bsz, L, N)),
        "dD": np.empty((D,)), "dz": np.empty((Bsz, L, D)) if z is not None else None,
        "ddt_bias": np.empty((D,)), "dh0": np.empty((Bsz, D, N)),
    }
    _load().oracle_scan_bwd(
        Bsz, L, D, N, int(bool(softplus)), _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm),
        _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(dy),
        _ptr(dh_final), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
        _ptr(out["ddt_bias"]), _ptr(out["dh0"]))
    return out


def ssd_bwd(x, dt, A, Bm, Cm, dy, Dskip=None, dt_bias=None, h0=None, dh_final=None, softplus=True):
    """Mamba-2 (SSD) backward in float64: the adjoint of ``ssd_fwd`` (the same
    reading: the selective scan over channels d = (h, p) with A[d, n] = A[h],
    delta[b,t,d] = dt[b,t,h], Dskip[d] = Dskip[h], dt_bias[d] = dt_bias[h]).
    By the chain rule through that tying, ``scan_bwd`` on the flattened
    channels gives every gradient once the ones of tied parameters are summed
    over the entries that share them: ddt[b,t,h] = sum_p ddelta[b,t,(h,p)],
    dA[h] = sum_{p,n} dA[(h,p),n], dDskip[h] and ddt_bias[h] = sum_p.  dy
    (B, L, H, P); dh_final (B, H, P, N) optional.  Returns a dict with dx
    (B, L, H, P), ddt (B, L, H), dA, dD, ddt_bias (H), dB, dC (B, L, N) and
    dh0 (B, H, P, N), float64."""
    x, dt, A, Bm, Cm, dy = _f64(x), _f64(dt), _f64(A), _f64(Bm), _f64(Cm), _f64(dy)
    B, L, H, P = x.shape
    N = Bm.shape[2]
    rep = lambda v: None if v is None else np.repeat(_f64(v), P, axis=-1)  # noqa: E731
    flat = lambda v: None if v is None else _f64(v).reshape(B, H * P, N)  # noqa: E731
    g = scan_bwd(x.reshape(B, L, H * P), rep(dt), np.repeat(A, P)[:, None] * np.ones((1, N)), Bm, Cm,
                 dy.reshape(B, L, H * P), Dskip=rep(Dskip), z=None, dt_bias=rep(dt_bias), h0=flat(h0),
                 dh_final=flat(dh_final), softplus=softplus)
    return {
        "dx": g["du"].reshape(B, L, H, P),
        "ddt": g["ddelta"].reshape(B, L, H, P).sum(-1),
        "dA": g["dA"].reshape(H, P, N).sum((1, 2)),
        "dB": g["dB"],
        "dC": g["dC"],
        "dD": g["dD"].reshape(H, P).sum(-1),
        "ddt_bias": g["ddt_bias"].reshape(H, P).sum(-1),
        "dh0": g["dh0"].reshape(B, H, P, N),
    }
