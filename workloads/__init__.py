"""Seeded synthetic inputs for the selective-scan workloads.

This module only draws random numbers and lays them out; it holds none of the
scan's arithmetic.  Both the HIP path (through its tests and benchmark) and
the float64 oracle consume what it produces.

The pages measure no dataset: the scan is benchmarked on one Mamba layer with
d_model=16, d_state=16 at batch 1 (page "mamba.py: 一个简单高效的Mamba实现",
overview figure caption and the performance section), and the pretrained
models all use d_state=16 (same page, d_state paragraph).  The five workloads
below are synthetic stand-ins of that layer and of the 130M / 2.8B layer
shapes, plus a 1M-step sequence and a training case.

Recipe (fixed draw order, numpy ``Generator(PCG64)``):

1. ``dt`` per channel, log-uniform on [1e-3, 1e-1], drawn in float64; then
   ``dt_bias = softplus^-1(dt) = dt + log(-expm1(-dt))`` so that a raw delta of
   0 maps to a step of exactly ``dt`` (stored float32);
2. ``A[d, n] = -(n + 1)`` (no draw);  3. ``Dskip = 1`` (no draw);
4. ``u ~ N(0,1)``;  5. ``delta = 0.5 * N(0,1)``;  6. ``z ~ N(0,1)``;
7. ``Bm ~ N(0,1)``; 8. ``Cm ~ N(0,1)``;  9. ``dy ~ N(0,1)`` (training only).

Causal conv1d front end (``conv_front_end``): the conv input x is the u
drawn above; taps (D, d_conv) and bias (D) uniform on [-1/sqrt(d_conv),
1/sqrt(d_conv)] (torch.nn.Conv1d's default initialisation for a depthwise
layer, whose fan-in is d_conv), and the history x_prev (B, d_conv - 1, D) ~
N(0,1), from ``SeedSequence(seed, spawn_key=(2**20, d_conv))``.

Normals are drawn in float32.  For bfloat16 workloads u, delta, z, Bm, Cm are
rounded to nearest-even bfloat16 and kept as uint16 bit patterns ("storage
form"); float32 workloads keep float32 arrays.  Steps 4-9 are drawn per block
of ``BLOCK_L`` time steps, each block from ``SeedSequence(seed,
spawn_key=(block,))``, so a block can be regenerated alone.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BLOCK_L = 65536


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    D: int
    N: int
    dtype: str          # "f32" or "bf16": storage type of u, delta, z, Bm, Cm, y
    seed: int
    backward: bool = False

    @property
    def elements(self) -> int:
        return self.B * self.L * self.D

    @property
    def elem_states(self) -> int:
        return self.B * self.L * self.D * self.N


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 32, 16, "f32", 1),
    "130m": Workload("130m", 8, 2048, 1536, 16, "f32", 2),
    "2.8b": Workload("2.8b", 4, 4096, 5120, 16, "bf16", 3),
    "long": Workload("long", 1, 1048576, 1536, 16, "bf16", 4),
    "train": Workload("train", 8, 2048, 1536, 16, "f32", 5, backward=True),
}

DESCRIPTIONS = {
    "tiny": "Tiny fwd scan B=1 L=64 D=32 N=16 fp32",
    "130m": "Mamba-130M-layer fwd scan B=8 L=2048 D=1536 N=16 fp32",
    "2.8b": "Mamba-2.8B-layer fwd scan B=4 L=4096 D=5120 N=16 bf16 act, fp32 A/D/state",
    "long": "Long-sequence fwd scan B=1 L=1048576 D=1536 N=16 bf16 act, fp32 state",
    "train": "Training fwd+bwd scan B=8 L=2048 D=1536 N=16 fp32",
}


def custom(B, L, D, N=16, dtype="f32", seed=0, backward=False, name="custom") -> Workload:
    return Workload(name, B, L, D, N, dtype, seed, backward)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + r) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form -> float32 values (exact)."""
    if x is None:
        return None
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


def channel_params(w: Workload):
    """dt_bias (D,), A (D, N), Dskip (D,) -- all float32."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=w.D))
    dt_bias = (dt + np.log(-np.expm1(-dt))).astype(np.float32)
    A = np.broadcast_to(-np.arange(1, w.N + 1, dtype=np.float32), (w.D, w.N)).copy()
    Dskip = np.ones(w.D, np.float32)
    return dt_bias, A, Dskip


def _draw_block(w: Workload, blk: int, l0: int, l1: int, out: dict):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(blk,))))
    lb = l1 - l0
    store = bf16_bits if w.dtype == "bf16" else (lambda a: a)
    out["u"][:, l0:l1] = store(rng.standard_normal((w.B, lb, w.D), dtype=np.float32))
    out["delta"][:, l0:l1] = store(np.float32(0.5) * rng.standard_normal((w.B, lb, w.D), dtype=np.float32))
    out["z"][:, l0:l1] = store(rng.standard_normal((w.B, lb, w.D), dtype=np.float32))
    out["Bm"][:, l0:l1] = store(rng.standard_normal((w.B, lb, w.N), dtype=np.float32))
    out["Cm"][:, l0:l1] = store(rng.standard_normal((w.B, lb, w.N), dtype=np.float32))
    if "dy" in out:
        out["dy"][:, l0:l1] = store(rng.standard_normal((w.B, lb, w.D), dtype=np.float32))


def make_inputs(w: Workload, with_dy: bool | None = None, threads: int = 8) -> dict:
    """All inputs of a workload in storage form (see module docstring).

    Keys: u, delta, z, Bm, Cm (+ dy), dt_bias, A, Dskip, and 'dtype'."""
    if with_dy is None:
        with_dy = w.backward
    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    out = {
        "u": np.empty((w.B, w.L, w.D), sdt), "delta": np.empty((w.B, w.L, w.D), sdt),
        "z": np.empty((w.B, w.L, w.D), sdt), "Bm": np.empty((w.B, w.L, w.N), sdt),
        "Cm": np.empty((w.B, w.L, w.N), sdt),
    }
    if with_dy:
        out["dy"] = np.empty((w.B, w.L, w.D), sdt)
    blocks = [(i, l0, min(l0 + BLOCK_L, w.L)) for i, l0 in enumerate(range(0, w.L, BLOCK_L))]
    if len(blocks) == 1:
        _draw_block(w, *blocks[0], out)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda b: _draw_block(w, *b, out), blocks))
    out["dt_bias"], out["A"], out["Dskip"] = channel_params(w)
    out["dtype"] = w.dtype
    return out


def conv_front_end(w: Workload, d_conv: int = 4) -> dict:
    """Seeded parameters of the causal conv1d front end of workload `w`:
    conv_w (D, d_conv) and conv_b (D) float32, x_prev (B, d_conv - 1, D) in
    the workload's storage form.  Merge into the dict of ``make_inputs``; its
    u then serves as the conv input x."""
    rng = np.random.default_rng(np.random.SeedSequence(w.seed, spawn_key=(1 << 20, d_conv)))
    bound = 1.0 / np.sqrt(d_conv)
    conv_w = rng.uniform(-bound, bound, (w.D, d_conv)).astype(np.float32)
    conv_b = rng.uniform(-bound, bound, w.D).astype(np.float32)
    xp = rng.standard_normal((w.B, d_conv - 1, w.D), dtype=np.float32)
    return {"conv_w": conv_w, "conv_b": conv_b, "x_prev": bf16_bits(xp) if w.dtype == "bf16" else xp}


def select_channels(inp: dict, channels) -> dict:
    """Inputs restricted to a subset of channels (channels are independent in
    the scan; Bm and Cm are shared by all channels and kept whole)."""
    ch = np.asarray(channels)
    out = dict(inp)
    for k in ("u", "delta", "z", "dy"):
        if k in inp and inp[k] is not None:
            out[k] = np.ascontiguousarray(inp[k][:, :, ch])
    for k in ("dt_bias", "Dskip", "conv_b"):
        if k in inp and inp[k] is not None:
            out[k] = np.ascontiguousarray(inp[k][ch])
    for k in ("A", "conv_w"):
        if k in inp and inp[k] is not None:
            out[k] = np.ascontiguousarray(inp[k][ch])
    if inp.get("x_prev") is not None:
        out["x_prev"] = np.ascontiguousarray(inp["x_prev"][:, :, ch])
    return out


def select_time(inp: dict, t0: int, t1: int) -> dict:
    """Inputs restricted to time steps [t0, t1)."""
    out = dict(inp)
    for k in ("u", "delta", "z", "dy", "Bm", "Cm"):
        if k in inp and inp[k] is not None:
            out[k] = np.ascontiguousarray(inp[k][:, t0:t1])
    return out


def as_float32(inp: dict) -> dict:
    """Storage form -> float32 arrays (exact)."""
    out = dict(inp)
    for k in ("u", "delta", "z", "dy", "Bm", "Cm", "x_prev"):
        if k in inp and inp[k] is not None:
            out[k] = to_f32(inp[k], inp["dtype"])
    return out


def to_torch(inp: dict, device="cuda", keys=("u", "delta", "z", "Bm", "Cm", "dy", "dt_bias", "A", "Dskip", "conv_w",
                                             "conv_b", "x_prev")) -> dict:
    """Storage form -> torch tensors on `device` (bfloat16 bits are
    reinterpreted, not converted, so values are exact)."""
    import torch

    out = {}
    for k in keys:
        if k not in inp or inp[k] is None:
            continue
        x = inp[k]
        if k in ("dt_bias", "A", "Dskip", "conv_w", "conv_b") or inp["dtype"] == "f32":
            out[k] = torch.from_numpy(np.ascontiguousarray(x)).to(device)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return out


def ssd_inputs(B: int, L: int, H: int, P: int, N: int, seed: int = 0) -> dict:
    """Seeded float32 inputs of a Mamba-2 (SSD) layer: x (B, L, H, P) ~ N(0,1);
    dt (B, L, H) = 0.5 * N(0,1); Bm, Cm (B, L, N) ~ N(0,1); per head, dt_bias =
    softplus^-1 of a step log-uniform on [1e-3, 1e-1] (as ``channel_params``),
    A = -U(1, 16) and Dskip = 1.  One ``Generator(PCG64(SeedSequence(seed,
    spawn_key=(2**21,))))`` in that order."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(1 << 21,))))
    dt_step = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=H))
    return {
        "dt_bias": (dt_step + np.log(-np.expm1(-dt_step))).astype(np.float32),
        "A": (-rng.uniform(1.0, 16.0, size=H)).astype(np.float32),
        "Dskip": np.ones(H, np.float32),
        "x": rng.standard_normal((B, L, H, P), dtype=np.float32),
        "dt": np.float32(0.5) * rng.standard_normal((B, L, H), dtype=np.float32),
        "Bm": rng.standard_normal((B, L, N), dtype=np.float32),
        "Cm": rng.standard_normal((B, L, N), dtype=np.float32),
    }
