"""GPU parity of the forward scan (HIP kernels through the C ABI) against the
float64 oracle, element by element, on seeded synthetic inputs.

Covers: the Tiny workload in full; ragged small shapes (channels not a
multiple of 64, sequence not a multiple of the 16-step tile) with every
optional input present and absent, softplus on and off; last tiles that end
inside a readout group; every supported state size in fp32 and bf16; the chunked (cross-chunk carry) schedule
with a ragged last chunk; the 130M and 2.8B layer workloads in full; the
1M-step workload in full, every channel, with the oracle run over batches of
64 channels (channels are independent, so the oracle can take them in any
grouping); bitwise determinism; and streaming (a split scan equals one scan).
y is judged at the activation type's bar, the float32 final state at 1e-4
(helpers.STATE_TOL) for every workload.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import FWD_TOL, STATE_TOL, fwd_err, gpu_inputs, run_gpu_fwd, run_oracle_fwd, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mssm():
    import selective_state_space_mssm_amd as m
    return m


def check(mssm, w, h0=False, use=("Dskip", "z", "dt_bias"), softplus=True, tol=None):
    print(f"[fwd] {w} h0={h0} use={use} softplus={softplus}", flush=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    h0n = None
    h0t = None
    if h0:
        h0n = np.random.default_rng(w.seed + 100).standard_normal((w.B, w.D, w.N)).astype(np.float32)
        h0t = torch.from_numpy(h0n).cuda()
    y, hf = run_gpu_fwd(mssm, t, h0t, use, softplus)
    torch.cuda.synchronize()
    yr, hr = run_oracle_fwd(oracle, inp, h0n, use, softplus)
    tol = tol or FWD_TOL[w.dtype]
    ey, eh = fwd_err(to_np(y), yr), fwd_err(to_np(hf), hr)
    assert np.all(np.isfinite(to_np(y)))
    print(f"  y err {ey:.2e}, h_final err {eh:.2e}", flush=True)
    assert ey <= tol, f"y err {ey:.3e} > {tol}"
    assert eh <= STATE_TOL, f"h_final err {eh:.3e} > {STATE_TOL}"
    return ey, eh


def test_tiny_workload(mssm):
    check(mssm, workloads.WORKLOADS["tiny"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 37, 70), (3, 16, 64), (1, 1, 1), (1, 200, 130), (2, 5, 200),
                                   (2, 101, 70), (3, 80, 64), (1, 65, 1), (2, 69, 200)])
def test_ragged_shapes_all_options(mssm, shape, dtype):
    # up to 64 steps the short-sequence path runs, above it the tiled kernel (the same remainders mod 16)
    B, L, D = shape
    check(mssm, workloads.custom(B, L, D, 16, dtype, seed=L + D), h0=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [82, 87, 94, 111])
def test_ragged_readout_groups(mssm, L, dtype):
    # the partial readouts of a tile are formed in groups of 2 (fp32) or 4
    # (bf16) steps: a last tile of 2, 7, 14 or 15 steps ends inside a group
    check(mssm, workloads.custom(2, L, 96, 16, dtype, seed=L + 500), h0=True)


@pytest.mark.parametrize("use", [(), ("z",), ("Dskip",), ("dt_bias",), ("Dskip", "dt_bias")])
def test_optional_inputs(mssm, use):
    check(mssm, workloads.custom(2, 109, 80, 16, "f32", seed=11), h0=False, use=use)


def test_softplus_off(mssm):
    # flag off: Delta = delta + dt_bias is used as is.  Keep it positive (as a
    # step size is) so the recurrence stays contractive and float32 finite.
    w = workloads.custom(2, 104, 70, 16, "f32", seed=12)
    inp = workloads.make_inputs(w)
    inp["delta"] = (0.05 * np.abs(inp["delta"])).astype(np.float32)
    inp["dt_bias"] = np.full(w.D, 0.01, np.float32)
    t = gpu_inputs(inp)
    h0n = np.random.default_rng(1).standard_normal((w.B, w.D, w.N)).astype(np.float32)
    y, hf = run_gpu_fwd(mssm, t, torch.from_numpy(h0n).cuda(), softplus=False)
    yr, hr = run_oracle_fwd(oracle, inp, h0n, softplus=False)
    assert fwd_err(to_np(y), yr) <= 1e-4 and fwd_err(to_np(hf), hr) <= 1e-4


@pytest.mark.parametrize("N", [1, 2, 4, 8, 32, 64])
def test_state_sizes(mssm, N):
    check(mssm, workloads.custom(2, 114, 90, N, "f32", seed=N), h0=True)


@pytest.mark.parametrize("N", [1, 2, 4, 8, 32, 64])
def test_state_sizes_bf16(mssm, N):
    # bf16 rows of Bm/Cm per lane (one value for N = 1), readout groups of
    # 4 steps (2 with 8 states per wave), a last tile of 3 steps
    check(mssm, workloads.custom(2, 115, 90, N, "bf16", seed=N + 7), h0=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_carry_schedule(mssm, dtype):
    # B * ceil(D/64) = 1 channel block, L = 5000: the time axis is cut into chunks
    # (aggregate + carry + rescan), the last chunk ragged
    B, L, D = 1, 5000, 40
    assert mssm.fwd_workspace_bytes(B, L, D, 16) > 0
    check(mssm, workloads.custom(B, L, D, 16, dtype, seed=21), h0=True)


@pytest.mark.parametrize("shape,dtype", [((1, 511, 200), "f32"), ((1, 512, 200), "bf16"), ((1, 700, 1536), "bf16"),
                                         ((2, 1024, 130), "f32"), ((1, 2047, 64), "f32"), ((3, 600, 1000), "bf16")])
def test_time_split_short_sequences(mssm, shape, dtype):
    # few channel blocks and 512 <= L < 2048: time cut into chunks of >= 128 steps (K = 4 at L = 512,
    # up to 16 at L = 2047), ragged last chunks and channel blocks; L = 511 stays one pass
    B, L, D = shape
    assert (mssm.fwd_workspace_bytes(B, L, D, 16) > 0) == (L >= 512)
    check(mssm, workloads.custom(B, L, D, 16, dtype, seed=L + D + 3), h0=True)


@pytest.mark.parametrize("shape,dtype", [((5, 100, 3840), "f32"), ((3, 333, 5760), "bf16"), ((4, 101, 4160), "f32")])
def test_balanced_schedule(mssm, shape, dtype):
    # more channel blocks than CUs but not a multiple of them: the persistent
    # balanced schedule splits blocks between workgroups mid-sequence and hands
    # the state over through the workspace (on a 256-CU MI355X: 300, 270 and
    # 260 blocks)
    B, L, D = shape
    assert mssm.fwd_workspace_bytes(B, L, D, 16) > 0
    check(mssm, workloads.custom(B, L, D, 16, dtype, seed=B * L), h0=True)
    # the published states are reset per call: a second call gives the same bits
    w = workloads.custom(B, L, D, 16, dtype, seed=B * L)
    t = gpu_inputs(workloads.make_inputs(w))
    y1, h1 = run_gpu_fwd(mssm, t)
    y2, h2 = run_gpu_fwd(mssm, t)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


@pytest.mark.parametrize("N", [1, 8, 64])
def test_schedules_other_state_sizes(mssm, N):
    # the chunked (1 block, L >= 2048) and the balanced (270 blocks) schedules
    # with one state per wave (N = 1, a single wave), 2 and 16 states per wave
    check(mssm, workloads.custom(1, 2100, 40, N, "f32", seed=N + 90), h0=True)
    check(mssm, workloads.custom(3, 104, 5760, N, "bf16", seed=N + 91), h0=True)


def test_130m_layer_full(mssm):
    ey, eh = check(mssm, workloads.WORKLOADS["130m"])
    print(f"130M: y err {ey:.2e}, h_final err {eh:.2e}")


def test_2p8b_layer_full(mssm):
    """The Mamba-2.8B layer workload (B=4, L=4096, D=5120, bf16) in the launch
    configuration of the benchmark (balanced persistent schedule), every
    element of y and h_final against the oracle."""
    w = workloads.WORKLOADS["2.8b"]
    print(f"[fwd full] {w}", flush=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    y, hf = run_gpu_fwd(mssm, t)
    torch.cuda.synchronize()
    yg, hg = to_np(y), to_np(hf)
    del y, hf, t
    torch.cuda.empty_cache()
    yr, hr = run_oracle_fwd(oracle, inp)
    ey, eh = fwd_err(yg, yr), fwd_err(hg, hr)
    print(f"2.8b: y err {ey:.2e}, h_final err {eh:.2e}", flush=True)
    assert ey <= FWD_TOL["bf16"] and eh <= STATE_TOL


def test_long_sequence_all_channels(mssm):
    """The 1M-step workload (B=1, L=1,048,576, D=1536, bf16; time-chunked
    schedule with the cross-chunk carry): every channel of y and h_final, the
    oracle taking 64 channels at a time (one channel block of the GPU path
    each, so all 24 blocks are covered)."""
    w = workloads.WORKLOADS["long"]
    print(f"[fwd full] {w}", flush=True)
    inp = workloads.make_inputs(w)
    t = gpu_inputs(inp)
    y, hf = run_gpu_fwd(mssm, t)
    torch.cuda.synchronize()
    del t
    hg = to_np(hf)
    ey = eh = 0.0
    for c0 in range(0, w.D, 64):
        ch = np.arange(c0, min(c0 + 64, w.D))
        yg = y[:, :, c0:c0 + len(ch)].float().cpu().numpy()
        yr, hr = run_oracle_fwd(oracle, workloads.select_channels(inp, ch))
        ey = max(ey, fwd_err(yg, yr))
        eh = max(eh, fwd_err(hg[:, ch], hr))
        print(f"  channels {c0}..{c0 + len(ch) - 1}: y err {ey:.2e}, h_final err {eh:.2e}", flush=True)
    del y, hf
    torch.cuda.empty_cache()
    assert ey <= FWD_TOL["bf16"] and eh <= STATE_TOL


def test_bitwise_deterministic(mssm):
    w = workloads.custom(4, 300, 200, 16, "f32", seed=5)
    t = gpu_inputs(workloads.make_inputs(w))
    y1, h1 = run_gpu_fwd(mssm, t)
    y2, h2 = run_gpu_fwd(mssm, t)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_split_scan_equals_one_scan(mssm):
    # both parts longer than the short-sequence path (64 steps), so all three calls run the tiled kernel
    w = workloads.custom(2, 320, 96, 16, "f32", seed=6)
    t = gpu_inputs(workloads.make_inputs(w))
    y, hf = run_gpu_fwd(mssm, t)
    L1 = 128  # a tile boundary: the two halves see exactly the same arithmetic
    t1 = {k: (v[:, :L1].contiguous() if k in ("u", "delta", "z", "Bm", "Cm") else v) for k, v in t.items()}
    t2 = {k: (v[:, L1:].contiguous() if k in ("u", "delta", "z", "Bm", "Cm") else v) for k, v in t.items()}
    y1, h1 = run_gpu_fwd(mssm, t1)
    y2, h2 = run_gpu_fwd(mssm, t2, h0=h1)
    assert torch.equal(torch.cat([y1, y2], 1), y)
    assert torch.equal(h2, hf)
