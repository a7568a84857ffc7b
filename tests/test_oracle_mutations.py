"""The oracle's pins must bite: plant plausible mistakes in a copy of the
oracle's C source (compiled on the CPU into a temporary library) and check
that at least one pin fails for each.  The real oracle is untouched."""
import os

import pytest

import oracle
import test_oracle_bwd_pins as bp
import test_oracle_fwd_pins as fp

FWD_PINS = [lambda: fp.test_closed_form(True), lambda: fp.test_closed_form(False),
            fp.test_blelloch_scan, fp.test_A_zero_is_prefix_sum, fp.test_delta_zero_flag_off,
            fp.test_C_zero_and_z_zero, fp.test_lti_is_causal_convolution,
            fp.test_exact_rational_tiny_case, fp.test_softplus_values]
BWD_PINS = [bp.test_torch_autograd, bp.test_reduction_invariants,
            bp.test_no_gate_A_zero_closed_form]

MUTATIONS = {
    # forward
    "A sign flipped": ("const double a = exp(dt * A[d * N + n]);",
                       "const double a = exp(-dt * A[d * N + n]);", FWD_PINS),
    "skip term dropped": ("s += opt(Dskip, d) * u[e];", "s += 0.0 * u[e];", FWD_PINS),
    "Bm state index reversed": ("h[n] = a * h[n] + dt * Bm[r + n] * u[e];",
                                "h[n] = a * h[n] + dt * Bm[r + (N - 1 - n)] * u[e];", FWD_PINS),
    "Euler step dropped from B": ("h[n] = a * h[n] + dt * Bm[r + n] * u[e];",
                                  "h[n] = a * h[n] + Bm[r + n] * u[e];", FWD_PINS),
    "gate is sigmoid not silu": ("y[e] = z ? s * silu(z[e]) : s;",
                                 "y[e] = z ? s * sig(z[e]) : s;", FWD_PINS),
    "softplus without log1p": ("return fmax(x, 0.0) + log1p(exp(-fabs(x)));",
                               "return fmax(x, 0.0) + exp(-fabs(x));", FWD_PINS),
    "readout uses Bm": ("s += Cm[r + n] * h[n];", "s += Bm[r + n] * h[n];", FWD_PINS),
    # backward
    "adjoint decay index": ("lam[n] *= Aa[(t + 1) * N + n];", "lam[n] *= Aa[t * N + n];", BWD_PINS),
    "silu derivative": ("(1.0 + zz * (1.0 - sg))", "(1.0 + zz * sg)", BWD_PINS),
    "softplus chain rule dropped": ("dDelta * sig(xs[t]) : dDelta", "dDelta : dDelta", BWD_PINS),
    "dh0 without decay": ("dh0[(b * D + d) * N + n] = Aa[n] * lam[n];",
                          "dh0[(b * D + d) * N + n] = lam[n];", BWD_PINS),
    "dB missing Delta": ("dB[r + n] += lam[n] * dts[t] * u[e];", "dB[r + n] += lam[n] * u[e];", BWD_PINS),
    "dA uses h_t": ("const double hp = H[t * N + n];", "const double hp = H[(t + 1) * N + n];", BWD_PINS),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path, monkeypatch):
    old, new, pins = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + old
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    so = oracle.build(source=str(mutated), out=str(tmp_path / "liboracle_mut.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.open_library(so))
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught the mutation '{name}'"
