"""GPU parity of the Mamba-2 (SSD) backward, mssm_ssd_bwd, against the float64
oracle's adjoint (oracle.ssd_bwd, the scan adjoint over channels (head, p)
with the tied gradients summed): dx, ddt, dA, dB, dC, dD, ddt_bias, dh0,
element by element with helpers.grad_err at 1e-3 (float32) or 2e-2
(bfloat16 inputs and gradients).

Shapes span several 64-step chunks with a ragged last chunk, one step, both
built state sizes, every optional input or none, softplus off, bfloat16, the
head-group partials (few (batch, chunk) pairs) and one group per (batch,
chunk), the chains in time segments (few (batch, head) pairs), many pairs, and
the 80-head d_state-128 layer at batch 8 on sampled heads; dB, dC there by
linearity in dy."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import GRAD_TOL, grad_err, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GRADS = ["dx", "ddt", "dA", "dB", "dC", "dD", "ddt_bias", "dh0"]


@pytest.fixture(scope="module")
def lib():
    import selective_state_space_mssm_amd as m
    return m


def case(B, L, H, N, seed, dtype="f32", softplus=True):
    inp = workloads.ssd_inputs(B, L, H, 64, N, seed=seed)
    rng = np.random.default_rng(seed + 1)
    inp["dy"] = rng.standard_normal((B, L, H, 64)).astype(np.float32)
    if not softplus:  # raw steps and bias >= 0 (the softplus-inverse bias would make Delta negative)
        inp["dt"] = (np.abs(inp["dt"]) * np.float32(0.05)).astype(np.float32)
        inp["dt_bias"] = np.full(H, 0.01, np.float32)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    if dtype == "bf16":
        for k in ("x", "dt", "Bm", "Cm", "dy"):
            t[k] = t[k].to(torch.bfloat16)
        for k in ("x", "dt", "Bm", "Cm", "dy"):
            inp[k] = t[k].float().cpu().numpy()  # the oracle takes the rounded values, exact in float32
    return inp, t


def run_both(lib, B, L, H, N, seed, dtype="f32", opts="all", softplus=True):
    print(f"[ssd bwd] B={B} L={L} H={H} N={N} {dtype} {opts} softplus={softplus}", flush=True)
    inp, t = case(B, L, H, N, seed, dtype, softplus)
    use = opts == "all"
    rng = np.random.default_rng(seed + 2)
    h0 = rng.standard_normal((B, H, 64, N)).astype(np.float32) if use else None
    dhf = rng.standard_normal((B, H, 64, N)).astype(np.float32) if use else None
    cu = lambda a: None if a is None else torch.from_numpy(a).cuda()  # noqa: E731
    g = lib.ssd_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"] if use else None,
                    t["dt_bias"] if use else None, cu(h0), cu(dhf), delta_softplus=softplus)
    torch.cuda.synchronize()
    r = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], inp["dy"],
                       Dskip=inp["Dskip"] if use else None, dt_bias=inp["dt_bias"] if use else None,
                       h0=h0, dh_final=dhf, softplus=softplus)
    return g, r


def assert_grads(g, r, tol, keys=GRADS):
    errs = {k: grad_err(to_np(g[k]), r[k]) for k in keys}
    print("grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"gradients over tolerance {tol}: {bad}"


@pytest.mark.parametrize("B,L,H,N", [(2, 200, 3, 64), (1, 64, 2, 128), (2, 1, 2, 64), (1, 257, 4, 128),
                                     (3, 130, 2, 64)])
@pytest.mark.parametrize("opts", ["all", "none"])
def test_ssd_bwd_parity(lib, B, L, H, N, opts):
    g, r = run_both(lib, B, L, H, N, seed=B * 100 + L + N, opts=opts)
    if L == 1 and opts == "none":
        # one step from a zero state: the decay multiplies zero, so dA is exactly 0, which the kernel reaches
        # as the difference of two equal sums of O(1) terms (C . dC and Delta r); judged absolutely
        assert np.all(r["dA"] == 0.0) and float(to_np(g["dA"]).__abs__().max()) <= 1e-4
        assert_grads(g, r, GRAD_TOL["f32"], keys=[k for k in GRADS if k != "dA"])
        return
    assert_grads(g, r, GRAD_TOL["f32"])


@pytest.mark.parametrize("N", [64, 128])
def test_ssd_bwd_no_softplus(lib, N):
    g, r = run_both(lib, 2, 150, 3, N, seed=N + 7, softplus=False)
    assert_grads(g, r, GRAD_TOL["f32"])


@pytest.mark.parametrize("B,L,H,N", [(2, 200, 3, 64), (1, 257, 4, 128)])
def test_ssd_bwd_bf16(lib, B, L, H, N):
    g, r = run_both(lib, B, L, H, N, seed=L + 3, dtype="bf16")
    assert g["dx"].dtype == torch.bfloat16 and g["dB"].dtype == torch.bfloat16
    assert_grads(g, r, GRAD_TOL["bf16"])


def test_ssd_bwd_one_group(lib):
    # (batch, chunk) pairs >= two per CU: one head group, dB and dC written by the chunk pass directly
    g, r = run_both(lib, 4, 8192, 2, 64, seed=31)
    assert_grads(g, r, GRAD_TOL["f32"])


@pytest.mark.parametrize("B,L,H,N", [(1, 1000, 3, 64), (1, 2048, 24, 128), (2, 1100, 5, 128)])
def test_ssd_bwd_time_segments(lib, B, L, H, N):
    # few (batch, head) pairs: both chains run in time segments from zero, joined and corrected afterwards
    # (1000 steps, 3 pairs: 8 segments of 2 chunks, the last ragged; the 24-head batch-1 layer: 16 segments;
    # 10 pairs over 18 chunks: 9 segments), with h0 and dh_final entering the outer segments
    g, r = run_both(lib, B, L, H, N, seed=L + H)
    assert_grads(g, r, GRAD_TOL["f32"])


def test_ssd_bwd_many_pairs(lib):
    # 270 (batch, head) pairs: one walk per pair, more chains than CUs
    g, r = run_both(lib, 3, 130, 90, 64, seed=41)
    assert_grads(g, r, GRAD_TOL["f32"])


def test_ssd_bwd_mamba2_layer_sampled(lib):
    # the 80-head d_state-128 layer at B = 8, L = 2048: per-head gradients on heads {0, 37, 79} against the
    # oracle run on those heads alone (dx, ddt, dh0 and the head's dA, dD, ddt_bias depend on its own inputs
    # only); dB and dC, sums over all heads, by linearity: the gradient for dy is the sum of the gradients
    # for dy restricted to the sampled heads and to the others, and the first equals the oracle's
    B, L, H, N = 8, 2048, 80, 128
    print(f"[ssd bwd 2.7B layer] B={B} L={L} H={H} N={N}", flush=True)
    inp, t = case(B, L, H, N, seed=2049)
    heads = [0, 37, 79]
    g = lib.ssd_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["dt_bias"])
    mask = torch.zeros(H, device="cuda")
    mask[heads] = 1.0
    g1 = lib.ssd_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], (t["dy"] * mask[:, None]).contiguous(),
                     t["Dskip"], t["dt_bias"])
    g2 = lib.ssd_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], (t["dy"] * (1 - mask)[:, None]).contiguous(),
                     t["Dskip"], t["dt_bias"])
    torch.cuda.synchronize()
    sub = lambda k: inp[k][:, :, heads]  # noqa: E731
    r = oracle.ssd_bwd(sub("x"), sub("dt"), inp["A"][heads], inp["Bm"], inp["Cm"], sub("dy"),
                       Dskip=inp["Dskip"][heads], dt_bias=inp["dt_bias"][heads])
    tol = GRAD_TOL["f32"]
    got = {"dx": to_np(g["dx"][:, :, heads]), "ddt": to_np(g["ddt"][:, :, heads]), "dh0": to_np(g["dh0"][:, heads]),
           "dA": to_np(g["dA"][heads]), "dD": to_np(g["dD"][heads]), "ddt_bias": to_np(g["ddt_bias"][heads]),
           "dB": to_np(g1["dB"]), "dC": to_np(g1["dC"])}
    errs = {k: grad_err(v, r[k]) for k, v in got.items()}
    print("grad errs: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= tol for v in errs.values()), errs
    for k in ("dB", "dC"):
        whole, parts = to_np(g[k]), to_np(g1[k]) + to_np(g2[k])
        assert grad_err(parts, whole) <= tol, k


def test_ssd_bwd_bitwise_reproducible(lib):
    inp, t = case(2, 300, 5, 128, seed=77)
    args = (t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["dy"], t["Dskip"], t["dt_bias"])
    g1 = lib.ssd_bwd(*args)
    g2 = lib.ssd_bwd(*args)
    for k in GRADS:
        assert torch.equal(g1[k], g2[k]), k
