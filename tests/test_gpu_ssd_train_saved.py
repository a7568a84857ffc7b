"""GPU parity of the Mamba-2 (SSD) training pair: mssm_ssd_fwd_train (the
forward that keeps the state entering every 64-step chunk and the final
state) and mssm_ssd_bwd_saved (the backward that starts from them, with no
first pass over the chunks).

* y and h_final equal mssm_ssd_fwd's bit for bit (the same kernels, which
  also store the states), with and without time segments (few (batch, head)
  pairs) and on the balanced schedule;
* the stored states equal the oracle's state entering every chunk (with time
  segments: after the pass that adds each segment's entering state);
* the gradients dx, ddt, dA, dB, dC, dD, ddt_bias, dh0 match the float64
  oracle's adjoint element by element (helpers.grad_err: 1e-3, 2e-2 for
  bfloat16) and mssm_ssd_bwd's to 1e-5;
* shapes: ragged last chunks, both state sizes, every optional input or none,
  bfloat16, a 128-channel head, few pairs (the forward and the adjoint chain
  in time segments, up to 8 of them) and the balanced forward schedule (more
  pairs than CUs, not a multiple)."""
import numpy as np
import pytest

import oracle
from helpers import GRAD_TOL, STATE_TOL, fwd_err, grad_err, to_np
from test_gpu_ssd_bwd import GRADS, case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import selective_state_space_mssm_amd as m
    return m


def check_states(ctx, inp, h0, use, B, L, H, N):
    """The stored state entering chunk c is the oracle's final state after the first 64 c steps (checked at
    the first chunks, one in the middle and the last, and the final slot, which is h_final)."""
    nch = (L + 63) // 64
    st = to_np(ctx[:B * H * (nch + 1) * 64 * N * 4].view(torch.float32)).reshape(B, H, nch + 1, 64, N)
    for c in sorted({0, 1, nch // 2, nch - 1, nch} & set(range(nch + 1))):
        t = min(64 * c, L)
        if t == 0:
            ref = h0 if h0 is not None else np.zeros((B, H, 64, N))
        else:
            ref = oracle.ssd_fwd(inp["x"][:, :t], inp["dt"][:, :t], inp["A"], inp["Bm"][:, :t], inp["Cm"][:, :t],
                                 Dskip=inp["Dskip"] if use else None, dt_bias=inp["dt_bias"] if use else None,
                                 h0=h0)[1]
        e = fwd_err(st[:, :, c], ref)
        assert e <= STATE_TOL, f"state entering chunk {c}: {e:.2e}"


def run_pair(lib, B, L, H, N, seed, dtype="f32", opts="all"):
    print(f"[ssd train pair] B={B} L={L} H={H} N={N} {dtype} {opts}", flush=True)
    inp, t = case(B, L, H, N, seed, dtype)
    use = opts == "all"
    rng = np.random.default_rng(seed + 2)
    h0 = rng.standard_normal((B, H, 64, N)).astype(np.float32) if use else None
    dhf = rng.standard_normal((B, H, 64, N)).astype(np.float32) if use else None
    cu = lambda a: None if a is None else torch.from_numpy(a).cuda()  # noqa: E731
    D, bias = (t["Dskip"], t["dt_bias"]) if use else (None, None)
    y, hf, ctx = lib.ssd_fwd_train(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], D, bias, cu(h0))
    y0, hf0 = lib.ssd_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], D, bias, cu(h0))
    assert torch.equal(y, y0) and torch.equal(hf, hf0), "training forward differs from mssm_ssd_fwd"
    check_states(ctx, inp, h0, use, B, L, H, N)
    g = lib.ssd_bwd_saved(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx, D, bias, cu(dhf))
    ref = lib.ssd_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], D, bias, cu(h0), cu(dhf))
    torch.cuda.synchronize()
    for k in GRADS:
        e = grad_err(to_np(g[k]), to_np(ref[k]))
        assert e <= 1e-5, f"{k}: {e:.2e} from mssm_ssd_bwd"
    r = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["dy"],
                       Dskip=inp["Dskip"] if use else None, dt_bias=inp["dt_bias"] if use else None,
                       h0=h0, dh_final=dhf)
    errs = {k: grad_err(to_np(g[k]), r[k]) for k in GRADS}
    print("grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= GRAD_TOL[dtype]}
    assert not bad, f"gradients over tolerance: {bad}"


@pytest.mark.parametrize("L,N", [(1, 64), (130, 64), (257, 128), (200, 128)])
def test_shapes(lib, L, N):
    # 8 pairs: four chunks or more are cut into time segments
    run_pair(lib, 2, L, 4, N, seed=L + N)


@pytest.mark.parametrize("B,L,H,N,dtype", [(1, 900, 2, 64, "f32"), (1, 1000, 2, 128, "bf16"), (2, 700, 1, 64, "f32")])
def test_many_segments(lib, B, L, H, N, dtype):
    # few pairs, long sequences: up to 8 time segments, the last one short and ragged; bfloat16 completes the
    # outputs in a float32 copy
    run_pair(lib, B, L, H, N, seed=L + H, dtype=dtype)


def test_no_optional_inputs(lib):
    run_pair(lib, 1, 150, 3, 64, seed=21, opts="none")


def test_bf16(lib):
    run_pair(lib, 2, 190, 3, 128, seed=22, dtype="bf16")


def test_many_pairs_balanced_forward(lib):
    # 270 pairs on a 256-CU MI355X: the balanced forward schedule stores the states of a pair split between
    # two workers; one head group per (batch, chunk) in the backward
    run_pair(lib, 3, 200, 90, 64, seed=23)


def test_head_dim_128(lib):
    # a 128-channel head is two 64-channel sub-heads sharing its parameters
    print("[ssd train pair] head dim 128", flush=True)
    rng = np.random.default_rng(24)
    B, L, H, P, N = 2, 150, 3, 128, 64
    import workloads
    inp = workloads.ssd_inputs(B, L, H, P, N, seed=24)
    inp["dy"] = rng.standard_normal((B, L, H, P)).astype(np.float32)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    y, hf, ctx = lib.ssd_fwd_train(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["Dskip"], t["dt_bias"])
    g = lib.ssd_bwd_saved(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], ctx, t["Dskip"], t["dt_bias"])
    torch.cuda.synchronize()
    r = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["dy"], Dskip=inp["Dskip"],
                       dt_bias=inp["dt_bias"])
    for k in GRADS:
        assert grad_err(to_np(g[k]), r[k]) <= GRAD_TOL["f32"], k
