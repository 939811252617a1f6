"""The pins are strong enough: every plausible mistake planted in a copy of the oracle
(read-out before the update, a sign, a dropped term, a transposed or shifted index, the
wrong gate, a broken compose rule, ...) makes at least one pin fail.

The mistakes are planted by text substitution into a temporary copy of
``oracle/sss_oracle.c``; the committed oracle is never modified.
"""
import importlib.util
import inspect
import os
import subprocess

import pytest

from tests import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sss_oracle.c")

MUTANTS = {
    "readout_before_update": (
        "      h[n] = abar * h[n] + bbar * xt;\n      v += (double)Ct[n] * h[n];",
        "      v += (double)Ct[n] * h[n];\n      h[n] = abar * h[n] + bbar * xt;"),
    "decay_sign": ("double abar = exp(dt * a);", "double abar = exp(-dt * a);"),
    "decay_without_delta": ("double abar = exp(dt * a);", "double abar = exp(a);"),
    "input_term_without_delta": ("        bbar = dt * (double)Bt[n];", "        bbar = (double)Bt[n];"),
    "dropped_skip": ("    if (Dsk) v += (double)Dsk[d] * xt;", "    (void)Dsk;"),
    "sigmoid_gate": ("      v *= zt / (1.0 + exp(-zt));\n    }\n    y_out", "      v *= 1.0 / (1.0 + exp(-zt));\n    }\n    y_out"),
    "A_transposed": ("      double a = (double)A[d * N + n];\n      double abar",
                     "      double a = (double)A[n * Dm + d];\n      double abar"),
    "B_wrong_state": ("bbar = dt * (double)Bt[n];", "bbar = dt * (double)Bt[(n + 1) % N];"),
    "C_wrong_state": ("v += (double)Ct[n] * h[n];", "v += (double)Ct[(n + 1) % N] * h[n];"),
    "B_previous_step": ("    const float* Bt = Bm + (b * L + t) * N;",
                        "    const float* Bt = Bm + (b * L + (t > 0 ? t - 1 : 0)) * N;"),
    "h0_ignored": ("for (int64_t n = 0; n < N; ++n) h[n] = h0 ? (double)h0[(b * Dm + d) * N + n] : 0.0;",
                   "for (int64_t n = 0; n < N; ++n) h[n] = 0.0;"),
    "bf16_decode": ("uint32_t w = ((uint32_t)bits) << 16;", "uint32_t w = ((uint32_t)bits) << 15;"),
    "ew_readout_before_update": (
        "    h = (double)A[e] * h + (double)Bm[e] * (double)x[e];\n    y_out[t * y_stride] = (double)Cm[e] * h;",
        "    y_out[t * y_stride] = (double)Cm[e] * h;\n    h = (double)A[e] * h + (double)Bm[e] * (double)x[e];"),
    "ew_C_for_B": ("    h = (double)A[e] * h + (double)Bm[e] * (double)x[e];",
                   "    h = (double)A[e] * h + (double)Cm[e] * (double)x[e];"),
    "ew_h0_ignored": ("  double h = h0 ? (double)h0[b * Dm + d] : 0.0;", "  double h = 0.0;"),
    "compose_wrong_order": ("  r.b = cur.a * prefix.b + cur.b;", "  r.b = prefix.a * cur.b + prefix.b;"),
    "zoh_without_A_division": ("(a != 0.0 ? expm1(dt * a) / a : dt) * (double)Bt[n]",
                               "(a != 0.0 ? expm1(dt * a) : dt) * (double)Bt[n]"),
    "zoh_zero_at_A_zero": ("(a != 0.0 ? expm1(dt * a) / a : dt) * (double)Bt[n]",
                           "(a != 0.0 ? expm1(dt * a) / a : 0.0) * (double)Bt[n]"),
    "zoh_zero_at_A_zero_chunked": ("p.b = (exact_zoh ? (a != 0.0 ? expm1(dt * a) / a : dt) : dt) * Bn * xt;",
                                   "p.b = (exact_zoh ? (a != 0.0 ? expm1(dt * a) / a : 0.0) : dt) * Bn * xt;"),
    "update_reads_old_state": ("      acc += (double)Cm[b * N + n] * h;",
                               "      acc += (double)Cm[b * N + n] * (double)state[c * N + n];"),
    "update_B_of_batch_0": ("dv * (double)Bm[b * N + n] * xv;", "dv * (double)Bm[n] * xv;"),
    "update_decay_without_delta": ("double h = exp(dv * (double)A[d * N + n])", "double h = exp((double)A[d * N + n])"),
    "update_dropped_skip": ("    if (Dsk) acc += (double)Dsk[d] * xv;", "    (void)Dsk;"),
    "conv_taps_reversed": ("if (ts >= 0) v += (double)w[d * W + k] *", "if (ts >= 0) v += (double)w[d * W + (W - 1 - k)] *"),
    "conv_shifted_one_step": ("        int64_t ts = t - (W - 1) + k;", "        int64_t ts = t - W + k;"),
    "bwd_delta_without_decay_term": ("gd += l * (Bn * xt + an * at * hp);", "gd += l * (Bn * xt);"),
    "bwd_dA_uses_new_state": ("lA[d * N + n] += l * dt * at * hp;", "lA[d * N + n] += l * dt * at * hs[(t + 1) * N + n];"),
    "bwd_dh_last_ignored": ("lam[n] = dh_last ? dh_last[c * N + n] : 0.0;", "lam[n] = 0.0;"),
    "bwd_softplus_chain_dropped": ("gd *= 1.0 / (1.0 + exp(-vr));", "gd *= 1.0;"),
    "bwd_softplus_chain_without_bias": ("double vr = load_val(delta, e, dtype) + (dbias ? (double)dbias[d] : 0.0);",
                                        "double vr = load_val(delta, e, dtype);"),
    "bwd_bias_grad_dropped": ("lDb[d] += gd;", "lDb[d] += 0.5 * gd;"),
    "bwd_front_end_ignored": ("double xt = load_val(x, e, dtype), dt = delta_value(delta, e, dtype, dbias, d, sp);\n        double g = 1.0;",
                              "double xt = load_val(x, e, dtype), dt = load_val(delta, e, dtype);\n        double g = 1.0;"),
    "bwd_adjoint_not_decayed": ("lam[n] = at * l;", "lam[n] = l;"),
    "bwd_silu_derivative": ("sg * (1.0 + zt * (1.0 - sg))", "sg"),
    "front_end_bias_ignored": ("  if (dbias) v += (double)dbias[d];", "  (void)dbias;"),
    "front_end_exp_for_softplus": ("static double softplus(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }",
                                   "static double softplus(double v) { return exp(v); }"),
}


def _pin_calls():
    """(name, callable(oracle_module)) for every pin in test_oracle_pins that uses the oracle."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or "oracle_lib" not in inspect.signature(fn).parameters:
            continue
        params = [p for p in inspect.signature(fn).parameters if p != "oracle_lib"]
        if not params:
            calls.append((name, lambda o, fn=fn: fn(o)))
        elif name == "test_M7_sequential_equals_chunked_pairs":
            calls.append((name, lambda o, fn=fn: fn(o, 7)))
        elif name == "test_M5_brute_force_unrolled":
            for io in ("f32", "bf16"):
                calls.append((name + io, lambda o, fn=fn, io=io: fn(o, io, True, True, True)))
        elif name == "test_C1_conv_is_numpy_convolve":
            calls.append((name, lambda o, fn=fn: fn(o, 4)))
        elif name == "test_U1_decode_step_is_one_step_of_the_scan":
            calls.append((name, lambda o, fn=fn: fn(o, "f32", True, True)))
        elif name == "test_L1_channel_major_running_sum":
            calls.append((name, lambda o, fn=fn: fn(o, "f32")))
    return calls


def _mutant_module(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / f"{name}.c"
    csrc.write_text(mutated)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-o", str(so),
                    str(csrc), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", os.path.join(ROOT, "oracle", "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB_PATH = str(so)
    mod._lib = None
    return mod


def test_unmutated_copy_passes_every_pin(tmp_path):
    mod = _mutant_module(tmp_path, "identity", "int oracle_max_threads(void)", "int oracle_max_threads(void)")
    for name, call in _pin_calls():
        call(mod)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # mutants may overflow; only the outcome matters
@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, mutant):
    old, new = MUTANTS[mutant]
    mod = _mutant_module(tmp_path, mutant, old, new)
    caught = []
    for name, call in _pin_calls():
        try:
            call(mod)
        except Exception:       # an assertion, or a ValueError from an impossible result
            caught.append(name)
    assert caught, f"no pin detects the planted mistake '{mutant}'"


def _reshape_not_transpose(which):
    """The channel-major adapter with one operand group reshaped instead of transposed."""
    import numpy as np

    def adapter(x, delta, z, B, C):
        tr = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a).transpose(0, 2, 1))
        rs = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a)).reshape(a.shape[0], a.shape[2], a.shape[1])
        f_io = rs if which == "io" else tr
        f_bc = rs if which == "bc" else tr
        return f_io(x), f_io(delta), f_io(z), f_bc(B), f_bc(C)
    return adapter


@pytest.mark.parametrize("which", ["io", "bc"])
def test_layout_mutant_is_caught(tmp_path, which):
    """A reshape in place of the transpose in the channel-major entry (of x/delta/z, or of
    B/C) fails a pin."""
    mod = _mutant_module(tmp_path, "layout_" + which, "int oracle_max_threads(void)", "int oracle_max_threads(void)")
    mod._to_time_major = _reshape_not_transpose(which)
    caught = []
    for name, call in _pin_calls():
        try:
            call(mod)
        except Exception:
            caught.append(name)
    assert caught, f"no pin detects a reshaped {which} operand"
