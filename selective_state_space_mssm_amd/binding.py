"""ctypes binding of libmssm.so (C ABI in include/mssm.h).

Argument marshalling only: checks that tensors are on the GPU, contiguous and
of the expected dtype and shape, allocates outputs and workspace with torch,
and passes raw device pointers plus torch's current HIP stream to the C entry
points.  Every step of the scan runs in the library's HIP kernels; there is no
CPU or PyTorch fallback, and importing this module fails loudly when the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmssm.so")

MSSM_F32, MSSM_BF16 = 0, 1
STATUS = {0: "MSSM_OK", -1: "MSSM_ERR_NULL", -2: "MSSM_ERR_SHAPE", -3: "MSSM_ERR_DTYPE",
          -4: "MSSM_ERR_UNSUPPORTED", -5: "MSSM_ERR_ALIGN", -6: "MSSM_ERR_WORKSPACE",
          -7: "MSSM_ERR_HIP"}
EXPORTS = ["mssm_scan_fwd_workspace_bytes", "mssm_scan_bwd_workspace_bytes", "mssm_scan_fwd", "mssm_scan_fwd_noalloc",
           "mssm_conv_scan_fwd", "mssm_conv_bwd_workspace_bytes", "mssm_conv_bwd", "mssm_scan_bwd", "mssm_step",
           "mssm_conv_step", "mssm_ssd_fwd_workspace_bytes", "mssm_ssd_fwd", "mssm_ssd_bwd_workspace_bytes",
           "mssm_ssd_bwd", "mssm_scan_ctx_bytes", "mssm_scan_fwd_train", "mssm_conv_scan_fwd_train", "mssm_scan_bwd_saved_workspace_bytes",
           "mssm_scan_bwd_saved", "mssm_ssd_ctx_bytes", "mssm_ssd_fwd_train_workspace_bytes", "mssm_ssd_fwd_train",
           "mssm_ssd_bwd_saved_workspace_bytes", "mssm_ssd_bwd_saved", "mssm_status_string", "mssm_build_info"]
MAX_DCONV = 4


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("delta_softplus", ctypes.c_int32)]


class SsdProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("delta_softplus", ctypes.c_int32)]


class MssmError(RuntimeError):
    def __init__(self, status: int, lib):
        self.status = status
        msg = lib.mssm_status_string(status).decode()
        if status == -5:  # a slice such as x[:, t] of a batch-1 tensor is "contiguous" but starts mid-allocation
            msg += " (pass a fresh tensor, e.g. .clone(), instead of a view at an offset)"
        super().__init__(msg)


def _open(path: str):
    if not os.path.exists(path):
        raise ImportError(
            f"libmssm.so not found at {path}: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P, sz, st, vp = ctypes.POINTER(Problem), ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p
    lib.mssm_scan_fwd_workspace_bytes.argtypes = [P]
    lib.mssm_scan_fwd_workspace_bytes.restype = sz
    lib.mssm_scan_bwd_workspace_bytes.argtypes = [P]
    lib.mssm_scan_bwd_workspace_bytes.restype = sz
    lib.mssm_scan_fwd.argtypes = [P] + [vp] * 11 + [vp, sz, vp]
    lib.mssm_scan_fwd.restype = st
    lib.mssm_scan_fwd_noalloc.argtypes = [P] + [vp] * 11 + [vp]
    lib.mssm_scan_fwd_noalloc.restype = st
    lib.mssm_conv_scan_fwd.argtypes = [P, ctypes.c_int32] + [vp] * 15 + [vp, sz, vp]
    lib.mssm_conv_scan_fwd.restype = st
    lib.mssm_conv_bwd_workspace_bytes.argtypes = [P, ctypes.c_int32]
    lib.mssm_conv_bwd_workspace_bytes.restype = sz
    lib.mssm_conv_bwd.argtypes = [P, ctypes.c_int32] + [vp] * 9 + [vp, sz, vp]
    lib.mssm_conv_bwd.restype = st
    lib.mssm_scan_bwd.argtypes = [P] + [vp] * 20 + [vp, sz, vp]
    lib.mssm_scan_bwd.restype = st
    lib.mssm_step.argtypes = [P] + [vp] * 10 + [vp]
    lib.mssm_step.restype = st
    lib.mssm_conv_step.argtypes = [P, ctypes.c_int32] + [vp] * 13 + [vp]
    lib.mssm_conv_step.restype = st
    lib.mssm_ssd_fwd_workspace_bytes.argtypes = [ctypes.POINTER(SsdProblem)]
    lib.mssm_ssd_fwd_workspace_bytes.restype = sz
    lib.mssm_ssd_fwd.argtypes = [ctypes.POINTER(SsdProblem)] + [vp] * 10 + [vp, sz, vp]
    lib.mssm_ssd_fwd.restype = st
    lib.mssm_ssd_bwd_workspace_bytes.argtypes = [ctypes.POINTER(SsdProblem)]
    lib.mssm_ssd_bwd_workspace_bytes.restype = sz
    lib.mssm_ssd_bwd.argtypes = [ctypes.POINTER(SsdProblem)] + [vp] * 18 + [vp, sz, vp]
    lib.mssm_ssd_bwd.restype = st
    lib.mssm_scan_ctx_bytes.argtypes = [P]
    lib.mssm_scan_ctx_bytes.restype = sz
    lib.mssm_scan_fwd_train.argtypes = [P] + [vp] * 11 + [vp, sz, vp, sz, vp]
    lib.mssm_scan_fwd_train.restype = st
    lib.mssm_conv_scan_fwd_train.argtypes = [P, ctypes.c_int32] + [vp] * 15 + [vp, sz, vp, sz, vp]
    lib.mssm_conv_scan_fwd_train.restype = st
    lib.mssm_scan_bwd_saved_workspace_bytes.argtypes = [P]
    lib.mssm_scan_bwd_saved_workspace_bytes.restype = sz
    lib.mssm_scan_bwd_saved.argtypes = [P] + [vp] * 8 + [vp, sz] + [vp] * 11 + [vp, sz, vp]
    lib.mssm_scan_bwd_saved.restype = st
    SP = ctypes.POINTER(SsdProblem)
    for q in ("mssm_ssd_ctx_bytes", "mssm_ssd_fwd_train_workspace_bytes", "mssm_ssd_bwd_saved_workspace_bytes"):
        getattr(lib, q).argtypes = [SP]
        getattr(lib, q).restype = sz
    lib.mssm_ssd_fwd_train.argtypes = [SP] + [vp] * 10 + [vp, sz, vp, sz, vp]
    lib.mssm_ssd_fwd_train.restype = st
    lib.mssm_ssd_bwd_saved.argtypes = [SP] + [vp] * 7 + [vp, sz] + [vp] * 10 + [vp, sz, vp]
    lib.mssm_ssd_bwd_saved.restype = st
    lib.mssm_status_string.argtypes = [st]
    lib.mssm_status_string.restype = ctypes.c_char_p
    lib.mssm_build_info.argtypes = []
    lib.mssm_build_info.restype = ctypes.c_char_p
    return lib


lib = _open(LIB_PATH)


def _check(status: int):
    if status != 0:
        raise MssmError(status, lib)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MSSM_F32
    if t.dtype == torch.bfloat16:
        return MSSM_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _req(t: torch.Tensor, name: str, shape, dtype) -> torch.Tensor:
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, name, shape, dtype):
    return None if t is None else _req(t, name, shape, dtype)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def problem(B: int, L: int, D: int, N: int, dtype=torch.float32, delta_softplus=True) -> Problem:
    code = dtype if isinstance(dtype, int) else (MSSM_BF16 if dtype == torch.bfloat16 else MSSM_F32)
    return Problem(B, L, D, N, code, 1 if delta_softplus else 0)


def fwd_workspace_bytes(B, L, D, N, dtype=torch.float32) -> int:
    return int(lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(problem(B, L, D, N, dtype))))


def bwd_workspace_bytes(B, L, D, N, dtype=torch.float32) -> int:
    return int(lib.mssm_scan_bwd_workspace_bytes(ctypes.byref(problem(B, L, D, N, dtype))))


def _workspace(nbytes: int, device, workspace=None):
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def scan_fwd(u, delta, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, h0=None,
             delta_softplus=True, return_final_state=True, y=None, h_final=None, workspace=None):
    """Selective scan forward.  u, delta, z: (B, L, D); Bm, Cm: (B, L, N), all
    float32 or all bfloat16; A (D, N), Dskip, dt_bias (D), h0 (B, D, N):
    float32.  Returns (y, h_final) (h_final None unless requested)."""
    act = u.dtype
    B, L, D = u.shape
    N = A.shape[1]
    _req(u, "u", (B, L, D), act)
    _req(delta, "delta", (B, L, D), act)
    _req(A, "A", (D, N), torch.float32)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _opt(Dskip, "Dskip", (D,), torch.float32)
    _opt(z, "z", (B, L, D), act)
    _opt(dt_bias, "dt_bias", (D,), torch.float32)
    _opt(h0, "h0", (B, D, N), torch.float32)
    if y is None:
        y = torch.empty((B, L, D), dtype=act, device=u.device)
    _req(y, "y", (B, L, D), act)
    if return_final_state and h_final is None:
        h_final = torch.empty((B, D, N), dtype=torch.float32, device=u.device)
    _opt(h_final, "h_final", (B, D, N), torch.float32)
    prob = problem(B, L, D, N, _dtype_code(u), delta_softplus)
    nbytes = int(lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(prob)))
    ws = _workspace(nbytes, u.device, workspace)
    _check(lib.mssm_scan_fwd(ctypes.byref(prob), _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                             _ptr(Dskip), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final),
                             _ptr(ws), nbytes, _stream(u.device)))
    return y, h_final


def scan_fwd_noalloc(u, delta, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, h0=None,
                     delta_softplus=True, return_final_state=True, y=None, h_final=None):
    """scan_fwd through mssm_scan_fwd_noalloc: no workspace, the library's own
    fixed scratch array instead (calls on one GPU must not overlap).  Pass y
    (and h_final) to allocate nothing here either."""
    act = u.dtype
    B, L, D = u.shape
    N = A.shape[1]
    _req(u, "u", (B, L, D), act)
    _req(delta, "delta", (B, L, D), act)
    _req(A, "A", (D, N), torch.float32)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _opt(Dskip, "Dskip", (D,), torch.float32)
    _opt(z, "z", (B, L, D), act)
    _opt(dt_bias, "dt_bias", (D,), torch.float32)
    _opt(h0, "h0", (B, D, N), torch.float32)
    if y is None:
        y = torch.empty((B, L, D), dtype=act, device=u.device)
    _req(y, "y", (B, L, D), act)
    if return_final_state and h_final is None:
        h_final = torch.empty((B, D, N), dtype=torch.float32, device=u.device)
    _opt(h_final, "h_final", (B, D, N), torch.float32)
    prob = problem(B, L, D, N, _dtype_code(u), delta_softplus)
    _check(lib.mssm_scan_fwd_noalloc(ctypes.byref(prob), _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                                     _ptr(Dskip), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final),
                                     _stream(u.device)))
    return y, h_final


def conv_scan_fwd(x, conv_w, delta, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, h0=None, conv_b=None,
                  x_prev=None, delta_softplus=True, return_final_state=True, return_u=False, y=None,
                  h_final=None, u_out=None, workspace=None):
    """Selective scan forward behind the fused causal conv1d + SiLU front end:
    the scan's u = silu(conv_b + depthwise causal conv of x with conv_w) is
    formed inside the kernels.  x, delta, z: (B, L, D); conv_w (D, d_conv) or
    (D, 1, d_conv) float32 (the torch.nn.Conv1d layout), conv_b (D) float32;
    x_prev (B, d_conv - 1, D): the inputs before t = 0 (zeros when None).
    Returns (y, h_final, u): h_final None unless requested, u (B, L, D) only
    with return_u (or u_out)."""
    return _conv_fwd(x, conv_w, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, conv_b, x_prev, delta_softplus,
                     return_final_state, return_u, y, h_final, u_out, workspace, None, False)[:3]


def conv_scan_fwd_train(x, conv_w, delta, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, h0=None, conv_b=None,
                        x_prev=None, delta_softplus=True, return_final_state=True, y=None, h_final=None,
                        u_out=None, ctx=None, workspace=None):
    """conv_scan_fwd that also saves the training context for scan_bwd_saved
    (which takes the returned u).  Returns (y, h_final, u, ctx)."""
    return _conv_fwd(x, conv_w, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, conv_b, x_prev, delta_softplus,
                     return_final_state, True, y, h_final, u_out, workspace, ctx, True)


def _conv_fwd(x, conv_w, delta, A, Bm, Cm, Dskip, z, dt_bias, h0, conv_b, x_prev, delta_softplus,
              return_final_state, return_u, y, h_final, u_out, workspace, ctx, train):
    act = x.dtype
    B, L, D = x.shape
    N = A.shape[1]
    if conv_w is None or conv_w.dim() not in (2, 3) or conv_w.shape[0] != D:
        raise ValueError("conv_w must be (D, d_conv) or (D, 1, d_conv)")
    K = conv_w.shape[-1]
    if conv_w.dim() == 3:
        if conv_w.shape[1] != 1:
            raise ValueError("conv_w must be depthwise: (D, 1, d_conv)")
        _req(conv_w, "conv_w", (D, 1, K), torch.float32)
        conv_w = conv_w.view(D, K)
    if not 1 <= K <= MAX_DCONV:
        raise ValueError(f"d_conv = {K} not in 1..{MAX_DCONV}")
    _req(x, "x", (B, L, D), act)
    _req(conv_w, "conv_w", (D, K), torch.float32)
    _opt(conv_b, "conv_b", (D,), torch.float32)
    if K > 1:
        _opt(x_prev, "x_prev", (B, K - 1, D), act)
    else:
        x_prev = None
    _req(delta, "delta", (B, L, D), act)
    _req(A, "A", (D, N), torch.float32)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _opt(Dskip, "Dskip", (D,), torch.float32)
    _opt(z, "z", (B, L, D), act)
    _opt(dt_bias, "dt_bias", (D,), torch.float32)
    _opt(h0, "h0", (B, D, N), torch.float32)
    if y is None:
        y = torch.empty((B, L, D), dtype=act, device=x.device)
    _req(y, "y", (B, L, D), act)
    if return_final_state and h_final is None:
        h_final = torch.empty((B, D, N), dtype=torch.float32, device=x.device)
    _opt(h_final, "h_final", (B, D, N), torch.float32)
    if return_u and u_out is None:
        u_out = torch.empty((B, L, D), dtype=act, device=x.device)
    _opt(u_out, "u_out", (B, L, D), act)
    prob = problem(B, L, D, N, _dtype_code(x), delta_softplus)
    nbytes = int(lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(prob)))
    ws = _workspace(nbytes, x.device, workspace)
    if not train:
        _check(lib.mssm_conv_scan_fwd(ctypes.byref(prob), K, _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(x_prev),
                                      _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
                                      _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final), _ptr(u_out),
                                      _ptr(ws), nbytes, _stream(x.device)))
        return y, h_final, u_out, None
    cbytes = int(lib.mssm_scan_ctx_bytes(ctypes.byref(prob)))
    if cbytes == 0:
        raise MssmError(-4, lib)
    if ctx is None:
        ctx = torch.empty(cbytes, dtype=torch.uint8, device=x.device)
    _check(lib.mssm_conv_scan_fwd_train(ctypes.byref(prob), K, _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(x_prev),
                                        _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
                                        _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final), _ptr(u_out),
                                        _ptr(ctx), ctx.numel() * ctx.element_size(), _ptr(ws), nbytes,
                                        _stream(x.device)))
    return y, h_final, u_out, ctx


def conv_bwd(x, conv_w, du, conv_b=None, x_prev=None, want_dconv_b=True, want_dx_prev=False, workspace=None):
    """Backward of the conv1d + SiLU front end of conv_scan_fwd: given du
    (B, L, D), returns a dict with dx (B, L, D), dconv_w (D, d_conv) float32,
    dconv_b (D) float32 (None unless wanted) and dx_prev (B, d_conv - 1, D)
    (None unless wanted)."""
    act = x.dtype
    B, L, D = x.shape
    if conv_w is None or conv_w.dim() not in (2, 3) or conv_w.shape[0] != D:
        raise ValueError("conv_w must be (D, d_conv) or (D, 1, d_conv)")
    K = conv_w.shape[-1]
    if conv_w.dim() == 3:
        _req(conv_w, "conv_w", (D, 1, K), torch.float32)
        conv_w = conv_w.view(D, K)
    if not 1 <= K <= MAX_DCONV:
        raise ValueError(f"d_conv = {K} not in 1..{MAX_DCONV}")
    _req(x, "x", (B, L, D), act)
    _req(conv_w, "conv_w", (D, K), torch.float32)
    _opt(conv_b, "conv_b", (D,), torch.float32)
    if K > 1:
        _opt(x_prev, "x_prev", (B, K - 1, D), act)
    else:
        x_prev, want_dx_prev = None, False
    _req(du, "du", (B, L, D), act)
    dev = x.device
    g = {"dx": torch.empty((B, L, D), dtype=act, device=dev),
         "dconv_w": torch.empty((D, K), dtype=torch.float32, device=dev),
         "dconv_b": torch.empty((D,), dtype=torch.float32, device=dev) if want_dconv_b else None,
         "dx_prev": torch.empty((B, K - 1, D), dtype=act, device=dev) if want_dx_prev else None}
    prob = problem(B, L, D, 1, _dtype_code(x))
    nbytes = int(lib.mssm_conv_bwd_workspace_bytes(ctypes.byref(prob), K))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.mssm_conv_bwd(ctypes.byref(prob), K, _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(x_prev), _ptr(du),
                             _ptr(g["dx"]), _ptr(g["dconv_w"]), _ptr(g["dconv_b"]), _ptr(g["dx_prev"]),
                             _ptr(ws), nbytes, _stream(dev)))
    return g


def scan_bwd(u, delta, A, Bm, Cm, dy, Dskip=None, z=None, dt_bias=None, h0=None, dh_final=None,
             delta_softplus=True, want_dh0=True, workspace=None):
    """Gradients of sum(dy*y) + sum(dh_final*h_final).  Returns a dict with
    du, ddelta, dA, dB, dC, dD, dz (None without z), ddt_bias, dh0."""
    act = u.dtype
    B, L, D = u.shape
    N = A.shape[1]
    dev = u.device
    _req(u, "u", (B, L, D), act)
    _req(delta, "delta", (B, L, D), act)
    _req(A, "A", (D, N), torch.float32)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _req(dy, "dy", (B, L, D), act)
    _opt(Dskip, "Dskip", (D,), torch.float32)
    _opt(z, "z", (B, L, D), act)
    _opt(dt_bias, "dt_bias", (D,), torch.float32)
    _opt(h0, "h0", (B, D, N), torch.float32)
    _opt(dh_final, "dh_final", (B, D, N), torch.float32)
    g = {
        "du": torch.empty((B, L, D), dtype=act, device=dev),
        "ddelta": torch.empty((B, L, D), dtype=act, device=dev),
        "dA": torch.empty((D, N), dtype=torch.float32, device=dev),
        "dB": torch.empty((B, L, N), dtype=act, device=dev),
        "dC": torch.empty((B, L, N), dtype=act, device=dev),
        "dD": torch.empty((D,), dtype=torch.float32, device=dev),
        "dz": torch.empty((B, L, D), dtype=act, device=dev) if z is not None else None,
        "ddt_bias": torch.empty((D,), dtype=torch.float32, device=dev),
        "dh0": torch.empty((B, D, N), dtype=torch.float32, device=dev) if want_dh0 else None,
    }
    prob = problem(B, L, D, N, _dtype_code(u), delta_softplus)
    nbytes = int(lib.mssm_scan_bwd_workspace_bytes(ctypes.byref(prob)))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.mssm_scan_bwd(ctypes.byref(prob), _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                             _ptr(Dskip), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(dy), _ptr(dh_final),
                             _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                             _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddt_bias"]),
                             _ptr(g["dh0"]), _ptr(ws), nbytes, _stream(dev)))
    return g


def ctx_bytes(B, L, D, N, dtype=torch.float32) -> int:
    return int(lib.mssm_scan_ctx_bytes(ctypes.byref(problem(B, L, D, N, dtype))))


def scan_fwd_train(u, delta, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, h0=None,
                   delta_softplus=True, return_final_state=True, y=None, h_final=None, ctx=None, workspace=None):
    """The forward of scan_fwd that also saves the training context for
    scan_bwd_saved.  Returns (y, h_final, ctx); ctx is a uint8 device tensor
    of ctx_bytes(...) bytes (pass one to reuse it)."""
    act = u.dtype
    B, L, D = u.shape
    N = A.shape[1]
    _req(u, "u", (B, L, D), act)
    _req(delta, "delta", (B, L, D), act)
    _req(A, "A", (D, N), torch.float32)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _opt(Dskip, "Dskip", (D,), torch.float32)
    _opt(z, "z", (B, L, D), act)
    _opt(dt_bias, "dt_bias", (D,), torch.float32)
    _opt(h0, "h0", (B, D, N), torch.float32)
    if y is None:
        y = torch.empty((B, L, D), dtype=act, device=u.device)
    _req(y, "y", (B, L, D), act)
    if return_final_state and h_final is None:
        h_final = torch.empty((B, D, N), dtype=torch.float32, device=u.device)
    _opt(h_final, "h_final", (B, D, N), torch.float32)
    prob = problem(B, L, D, N, _dtype_code(u), delta_softplus)
    cbytes = int(lib.mssm_scan_ctx_bytes(ctypes.byref(prob)))
    if cbytes == 0:
        raise MssmError(-4, lib)
    if ctx is None:
        ctx = torch.empty(cbytes, dtype=torch.uint8, device=u.device)
    nbytes = int(lib.mssm_scan_fwd_workspace_bytes(ctypes.byref(prob)))
    ws = _workspace(nbytes, u.device, workspace)
    _check(lib.mssm_scan_fwd_train(ctypes.byref(prob), _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                                   _ptr(Dskip), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final),
                                   _ptr(ctx), ctx.numel() * ctx.element_size(), _ptr(ws), nbytes, _stream(u.device)))
    return y, h_final, ctx


def scan_bwd_saved(u, delta, A, Bm, Cm, dy, ctx, Dskip=None, z=None, dt_bias=None, dh_final=None,
                   delta_softplus=True, want_dh0=True, workspace=None):
    """scan_bwd from the context scan_fwd_train saved for the same inputs (no
    h0 argument: the context holds it).  Returns the dict of scan_bwd."""
    act = u.dtype
    B, L, D = u.shape
    N = A.shape[1]
    dev = u.device
    _req(u, "u", (B, L, D), act)
    _req(delta, "delta", (B, L, D), act)
    _req(A, "A", (D, N), torch.float32)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _req(dy, "dy", (B, L, D), act)
    _opt(Dskip, "Dskip", (D,), torch.float32)
    _opt(z, "z", (B, L, D), act)
    _opt(dt_bias, "dt_bias", (D,), torch.float32)
    _opt(dh_final, "dh_final", (B, D, N), torch.float32)
    if not ctx.is_cuda or not ctx.is_contiguous():
        raise ValueError("ctx must be a contiguous GPU tensor")
    g = {
        "du": torch.empty((B, L, D), dtype=act, device=dev),
        "ddelta": torch.empty((B, L, D), dtype=act, device=dev),
        "dA": torch.empty((D, N), dtype=torch.float32, device=dev),
        "dB": torch.empty((B, L, N), dtype=act, device=dev),
        "dC": torch.empty((B, L, N), dtype=act, device=dev),
        "dD": torch.empty((D,), dtype=torch.float32, device=dev),
        "dz": torch.empty((B, L, D), dtype=act, device=dev) if z is not None else None,
        "ddt_bias": torch.empty((D,), dtype=torch.float32, device=dev),
        "dh0": torch.empty((B, D, N), dtype=torch.float32, device=dev) if want_dh0 else None,
    }
    prob = problem(B, L, D, N, _dtype_code(u), delta_softplus)
    nbytes = int(lib.mssm_scan_bwd_saved_workspace_bytes(ctypes.byref(prob)))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.mssm_scan_bwd_saved(ctypes.byref(prob), _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm),
                                   _ptr(Dskip), _ptr(z), _ptr(dt_bias), _ptr(ctx),
                                   ctx.numel() * ctx.element_size(), _ptr(dy), _ptr(dh_final),
                                   _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                                   _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddt_bias"]),
                                   _ptr(g["dh0"]), _ptr(ws), nbytes, _stream(dev)))
    return g


def step(u_t, delta_t, A, Bm_t, Cm_t, state, Dskip=None, z_t=None, dt_bias=None,
         delta_softplus=True, y_t=None):
    """One recurrent step.  u_t, delta_t, z_t: (B, D); Bm_t, Cm_t: (B, N);
    state (B, D, N) float32 is updated in place.  Returns y_t (B, D)."""
    act = u_t.dtype
    B, D = u_t.shape
    N = A.shape[1]
    _req(u_t, "u_t", (B, D), act)
    _req(delta_t, "delta_t", (B, D), act)
    _req(A, "A", (D, N), torch.float32)
    _req(Bm_t, "Bm_t", (B, N), act)
    _req(Cm_t, "Cm_t", (B, N), act)
    _req(state, "state", (B, D, N), torch.float32)
    _opt(Dskip, "Dskip", (D,), torch.float32)
    _opt(z_t, "z_t", (B, D), act)
    _opt(dt_bias, "dt_bias", (D,), torch.float32)
    if y_t is None:
        y_t = torch.empty((B, D), dtype=act, device=u_t.device)
    prob = problem(B, 1, D, N, _dtype_code(u_t), delta_softplus)
    _check(lib.mssm_step(ctypes.byref(prob), _ptr(u_t), _ptr(delta_t), _ptr(A), _ptr(Bm_t), _ptr(Cm_t),
                         _ptr(Dskip), _ptr(z_t), _ptr(dt_bias), _ptr(state), _ptr(y_t),
                         _stream(u_t.device)))
    return y_t


class Stepper:
    """The recurrent step over fixed buffers, for decode loops: the buffers are
    checked and their addresses marshalled once, so that a call is one C call
    (mssm_step) on the stream current at construction.  The caller writes
    each token's inputs into u_t, delta_t, Bm_t, Cm_t (and z_t) in place; the
    step updates state and writes y_t.  Arguments as step(); the buffers must
    outlive the Stepper.  A call enqueues no allocation or memset, so it can
    be captured in a CUDA/HIP graph."""

    def __init__(self, u_t, delta_t, A, Bm_t, Cm_t, state, Dskip=None, z_t=None, dt_bias=None,
                 delta_softplus=True, y_t=None):
        act = u_t.dtype
        B, D = u_t.shape
        N = A.shape[1]
        _req(u_t, "u_t", (B, D), act)
        _req(delta_t, "delta_t", (B, D), act)
        _req(A, "A", (D, N), torch.float32)
        _req(Bm_t, "Bm_t", (B, N), act)
        _req(Cm_t, "Cm_t", (B, N), act)
        _req(state, "state", (B, D, N), torch.float32)
        _opt(Dskip, "Dskip", (D,), torch.float32)
        _opt(z_t, "z_t", (B, D), act)
        _opt(dt_bias, "dt_bias", (D,), torch.float32)
        if y_t is None:
            y_t = torch.empty((B, D), dtype=act, device=u_t.device)
        _req(y_t, "y_t", (B, D), act)
        self.y_t = y_t
        self._keep = (u_t, delta_t, A, Bm_t, Cm_t, state, Dskip, z_t, dt_bias, y_t)
        self._prob = problem(B, 1, D, N, _dtype_code(u_t), delta_softplus)
        self._args = (ctypes.byref(self._prob), _ptr(u_t), _ptr(delta_t), _ptr(A), _ptr(Bm_t), _ptr(Cm_t),
                      _ptr(Dskip), _ptr(z_t), _ptr(dt_bias), _ptr(state), _ptr(y_t), _stream(u_t.device))
        self._fn = lib.mssm_step

    def __call__(self):
        status = self._fn(*self._args)
        if status != 0:
            raise MssmError(status, lib)
        return self.y_t


def conv_step(x_t, conv_w, conv_state, delta_t, A, Bm_t, Cm_t, state, Dskip=None, z_t=None, dt_bias=None,
              conv_b=None, delta_softplus=True, y_t=None):
    """One token through the conv1d + SiLU front end and the recurrent step.
    x_t, delta_t, z_t: (B, D); Bm_t, Cm_t: (B, N); conv_w (D, d_conv) or
    (D, 1, d_conv) float32; conv_state (B, d_conv - 1, D) (the previous inputs,
    shifted in place), state (B, D, N) float32 updated in place.  Returns y_t."""
    act = x_t.dtype
    B, D = x_t.shape
    N = A.shape[1]
    if conv_w is None or conv_w.dim() not in (2, 3) or conv_w.shape[0] != D:
        raise ValueError("conv_w must be (D, d_conv) or (D, 1, d_conv)")
    K = conv_w.shape[-1]
    if conv_w.dim() == 3:
        _req(conv_w, "conv_w", (D, 1, K), torch.float32)
        conv_w = conv_w.view(D, K)
    if not 1 <= K <= MAX_DCONV:
        raise ValueError(f"d_conv = {K} not in 1..{MAX_DCONV}")
    _req(x_t, "x_t", (B, D), act)
    _req(conv_w, "conv_w", (D, K), torch.float32)
    _opt(conv_b, "conv_b", (D,), torch.float32)
    if K > 1:
        _req(conv_state, "conv_state", (B, K - 1, D), act)
    else:
        conv_state = None
    _req(delta_t, "delta_t", (B, D), act)
    _req(A, "A", (D, N), torch.float32)
    _req(Bm_t, "Bm_t", (B, N), act)
    _req(Cm_t, "Cm_t", (B, N), act)
    _req(state, "state", (B, D, N), torch.float32)
    _opt(Dskip, "Dskip", (D,), torch.float32)
    _opt(z_t, "z_t", (B, D), act)
    _opt(dt_bias, "dt_bias", (D,), torch.float32)
    if y_t is None:
        y_t = torch.empty((B, D), dtype=act, device=x_t.device)
    prob = problem(B, 1, D, N, _dtype_code(x_t), delta_softplus)
    _check(lib.mssm_conv_step(ctypes.byref(prob), K, _ptr(x_t), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state),
                              _ptr(delta_t), _ptr(A), _ptr(Bm_t), _ptr(Cm_t), _ptr(Dskip), _ptr(z_t),
                              _ptr(dt_bias), _ptr(state), _ptr(y_t), _stream(x_t.device)))
    return y_t


def ssd_fwd(x, dt, A, Bm, Cm, Dskip=None, dt_bias=None, h0=None, delta_softplus=True,
            return_final_state=True, y=None, h_final=None, workspace=None):
    """Mamba-2 (SSD) forward.  x: (B, L, H, P); dt: (B, L, H); Bm, Cm: (B, L, N),
    all float32 or all bfloat16; A, Dskip, dt_bias: (H); h0: (B, H, P, N):
    float32.  Returns (y, h_final) (y in x's dtype; h_final None unless requested)."""
    B, L, H, P = x.shape
    N = Bm.shape[2]
    f, act = torch.float32, x.dtype
    _req(x, "x", (B, L, H, P), act)
    _req(dt, "dt", (B, L, H), act)
    _req(A, "A", (H,), f)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _opt(Dskip, "Dskip", (H,), f)
    _opt(dt_bias, "dt_bias", (H,), f)
    _opt(h0, "h0", (B, H, P, N), f)
    if y is None:
        y = torch.empty((B, L, H, P), dtype=act, device=x.device)
    _req(y, "y", (B, L, H, P), act)
    if return_final_state and h_final is None:
        h_final = torch.empty((B, H, P, N), dtype=f, device=x.device)
    _opt(h_final, "h_final", (B, H, P, N), f)
    prob = SsdProblem(B, L, H, P, N, _dtype_code(x), 1 if delta_softplus else 0)
    nbytes = int(lib.mssm_ssd_fwd_workspace_bytes(ctypes.byref(prob)))
    ws = _workspace(nbytes, x.device, workspace)
    _check(lib.mssm_ssd_fwd(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip),
                            _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final), _ptr(ws), nbytes, _stream(x.device)))
    return y, h_final


def ssd_bwd(x, dt, A, Bm, Cm, dy, Dskip=None, dt_bias=None, h0=None, dh_final=None, delta_softplus=True,
            want_dD=True, want_ddt_bias=True, want_dh0=True, workspace=None):
    """Mamba-2 (SSD) backward.  Inputs as ssd_fwd, with dy (B, L, H, P) in x's dtype and dh_final
    (B, H, P, N) float32 optional.  Returns a dict with dx, ddt, dB, dC (x's dtype), dA and, unless
    switched off, dD, ddt_bias, dh0 (float32)."""
    B, L, H, P = x.shape
    N = Bm.shape[2]
    f, act = torch.float32, x.dtype
    _req(x, "x", (B, L, H, P), act)
    _req(dt, "dt", (B, L, H), act)
    _req(A, "A", (H,), f)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _req(dy, "dy", (B, L, H, P), act)
    _opt(Dskip, "Dskip", (H,), f)
    _opt(dt_bias, "dt_bias", (H,), f)
    _opt(h0, "h0", (B, H, P, N), f)
    _opt(dh_final, "dh_final", (B, H, P, N), f)
    dev = x.device
    g = {
        "dx": torch.empty((B, L, H, P), dtype=act, device=dev),
        "ddt": torch.empty((B, L, H), dtype=act, device=dev),
        "dA": torch.empty((H,), dtype=f, device=dev),
        "dB": torch.empty((B, L, N), dtype=act, device=dev),
        "dC": torch.empty((B, L, N), dtype=act, device=dev),
        "dD": torch.empty((H,), dtype=f, device=dev) if want_dD else None,
        "ddt_bias": torch.empty((H,), dtype=f, device=dev) if want_ddt_bias else None,
        "dh0": torch.empty((B, H, P, N), dtype=f, device=dev) if want_dh0 else None,
    }
    prob = SsdProblem(B, L, H, P, N, _dtype_code(x), 1 if delta_softplus else 0)
    nbytes = int(lib.mssm_ssd_bwd_workspace_bytes(ctypes.byref(prob)))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.mssm_ssd_bwd(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip),
                            _ptr(dt_bias), _ptr(h0), _ptr(dy), _ptr(dh_final), _ptr(g["dx"]), _ptr(g["ddt"]),
                            _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["ddt_bias"]),
                            _ptr(g["dh0"]), _ptr(ws), nbytes, _stream(dev)))
    return g


def ssd_fwd_train(x, dt, A, Bm, Cm, Dskip=None, dt_bias=None, h0=None, delta_softplus=True,
                  return_final_state=True, y=None, h_final=None, ctx=None, workspace=None):
    """ssd_fwd that also keeps the chunk states for ssd_bwd_saved.
    Returns (y, h_final, ctx); ctx a uint8 device tensor of mssm_ssd_ctx_bytes."""
    B, L, H, P = x.shape
    N = Bm.shape[2]
    f, act = torch.float32, x.dtype
    _req(x, "x", (B, L, H, P), act)
    _req(dt, "dt", (B, L, H), act)
    _req(A, "A", (H,), f)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _opt(Dskip, "Dskip", (H,), f)
    _opt(dt_bias, "dt_bias", (H,), f)
    _opt(h0, "h0", (B, H, P, N), f)
    if y is None:
        y = torch.empty((B, L, H, P), dtype=act, device=x.device)
    _req(y, "y", (B, L, H, P), act)
    if return_final_state and h_final is None:
        h_final = torch.empty((B, H, P, N), dtype=f, device=x.device)
    _opt(h_final, "h_final", (B, H, P, N), f)
    prob = SsdProblem(B, L, H, P, N, _dtype_code(x), 1 if delta_softplus else 0)
    cbytes = int(lib.mssm_ssd_ctx_bytes(ctypes.byref(prob)))
    if cbytes == 0:
        raise MssmError(-4, lib)
    if ctx is None:
        ctx = torch.empty(cbytes, dtype=torch.uint8, device=x.device)
    nbytes = int(lib.mssm_ssd_fwd_train_workspace_bytes(ctypes.byref(prob)))
    ws = _workspace(nbytes, x.device, workspace)
    _check(lib.mssm_ssd_fwd_train(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip),
                                  _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final), _ptr(ctx),
                                  ctx.numel() * ctx.element_size(), _ptr(ws), nbytes, _stream(x.device)))
    return y, h_final, ctx


def ssd_bwd_saved(x, dt, A, Bm, Cm, dy, ctx, Dskip=None, dt_bias=None, dh_final=None, delta_softplus=True,
                  want_dD=True, want_ddt_bias=True, want_dh0=True, workspace=None):
    """ssd_bwd from the context ssd_fwd_train kept for the same inputs (no h0 argument: the context
    holds it).  Returns the dict of ssd_bwd."""
    B, L, H, P = x.shape
    N = Bm.shape[2]
    f, act = torch.float32, x.dtype
    _req(x, "x", (B, L, H, P), act)
    _req(dt, "dt", (B, L, H), act)
    _req(A, "A", (H,), f)
    _req(Bm, "Bm", (B, L, N), act)
    _req(Cm, "Cm", (B, L, N), act)
    _req(dy, "dy", (B, L, H, P), act)
    _opt(Dskip, "Dskip", (H,), f)
    _opt(dt_bias, "dt_bias", (H,), f)
    _opt(dh_final, "dh_final", (B, H, P, N), f)
    if not ctx.is_cuda or not ctx.is_contiguous():
        raise ValueError("ctx must be a contiguous GPU tensor")
    dev = x.device
    g = {
        "dx": torch.empty((B, L, H, P), dtype=act, device=dev),
        "ddt": torch.empty((B, L, H), dtype=act, device=dev),
        "dA": torch.empty((H,), dtype=f, device=dev),
        "dB": torch.empty((B, L, N), dtype=act, device=dev),
        "dC": torch.empty((B, L, N), dtype=act, device=dev),
        "dD": torch.empty((H,), dtype=f, device=dev) if want_dD else None,
        "ddt_bias": torch.empty((H,), dtype=f, device=dev) if want_ddt_bias else None,
        "dh0": torch.empty((B, H, P, N), dtype=f, device=dev) if want_dh0 else None,
    }
    prob = SsdProblem(B, L, H, P, N, _dtype_code(x), 1 if delta_softplus else 0)
    nbytes = int(lib.mssm_ssd_bwd_saved_workspace_bytes(ctypes.byref(prob)))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib.mssm_ssd_bwd_saved(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip),
                                  _ptr(dt_bias), _ptr(ctx), ctx.numel() * ctx.element_size(), _ptr(dy),
                                  _ptr(dh_final), _ptr(g["dx"]), _ptr(g["ddt"]), _ptr(g["dA"]), _ptr(g["dB"]),
                                  _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["ddt_bias"]), _ptr(g["dh0"]), _ptr(ws),
                                  nbytes, _stream(dev)))
    return g
