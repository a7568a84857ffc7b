"""Shared helpers for the parity tests: run the HIP path through the C ABI
binding and the float64 oracle on the same seeded inputs, and compare.

Tolerances (float32 arithmetic on the GPU against the float64 oracle):
* forward outputs y, h_final: max_i |g - r| / max(1, |r|) <= 1e-4 for float32
  activations and <= 2e-2 for bfloat16 activations (abs-or-rel criterion);
* the float32 state (h_final, a decode state) at 1e-4 whatever the activation
  type: bfloat16 inputs widen to float32 exactly and the state is never
  rounded to bfloat16, so only float32 arithmetic separates it from the
  float64 oracle -- the bfloat16 bar would hide a carry defect of 1e-3;
* gradients: max_i |g - r| / max(|r|, rms(r)) <= 1e-3 per tensor (relative,
  with an rms floor so that entries near zero are judged on the tensor's
  scale), 2e-2 for bfloat16 activations.
"""
from __future__ import annotations

import numpy as np

import workloads

FWD_TOL = {"f32": 1e-4, "bf16": 2e-2}
STATE_TOL = 1e-4
GRAD_TOL = {"f32": 1e-3, "bf16": 2e-2}


def fwd_err(g, r) -> float:
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.max(np.abs(g - r) / np.maximum(1.0, np.abs(r)))) if r.size else 0.0


def grad_err(g, r) -> float:
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    floor = np.maximum(np.abs(r), max(rms, 1e-30))
    return float(np.max(np.abs(g - r) / floor)) if r.size else 0.0


def to_np(t):
    if t is None or isinstance(t, np.ndarray):
        return t
    return t.detach().float().cpu().numpy()


def gpu_inputs(inp, device="cuda"):
    return workloads.to_torch(inp, device)


def run_gpu_fwd(mssm, t, h0=None, use=("Dskip", "z", "dt_bias"), softplus=True):
    return mssm.scan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"],
                         t["Dskip"] if "Dskip" in use else None,
                         t["z"] if "z" in use else None,
                         t["dt_bias"] if "dt_bias" in use else None,
                         h0, delta_softplus=softplus)


def run_oracle_fwd(oracle, inp, h0=None, use=("Dskip", "z", "dt_bias"), softplus=True):
    f = workloads.as_float32(inp)
    return oracle.scan_fwd(f["u"], f["delta"], f["A"], f["Bm"], f["Cm"],
                           f["Dskip"] if "Dskip" in use else None,
                           f["z"] if "z" in use else None,
                           f["dt_bias"] if "dt_bias" in use else None,
                           h0, softplus=softplus)
