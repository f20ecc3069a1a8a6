"""Plant plausible mistakes in copies of the oracle and require that every
mutant fails at least one pin. This shows the pins constrain each term of the
definition (a dropped term, a wrong sign, a wrong index, a swapped operand)."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement, pins to run)
MUTANTS = [
    ("dt_dropped_from_decay", "exp(dt * (double)A[d * N + n])", "exp((double)A[d * N + n])", "scan"),
    ("decay_sign", "exp(dt * (double)A[d * N + n])", "exp(-dt * (double)A[d * N + n])", "scan"),
    ("A_transposed", "(double)A[d * N + n]", "(double)A[n * D + d]", "scan"),
    ("dt_dropped_from_input", "const double bx = dt * (double)Bm[r + n] * xv;",
     "const double bx = (double)Bm[r + n] * xv;", "scan"),
    ("B_and_C_swapped", "const double bx = dt * (double)Bm[r + n] * xv;",
     "const double bx = dt * (double)Cm[r + n] * xv;", "scan"),
    ("B_not_time_varying", "const double bx = dt * (double)Bm[r + n] * xv;",
     "const double bx = dt * (double)Bm[b * L * N + n] * xv;", "scan"),
    ("decay_applied_to_input", "h[n] = abar * h[n] + bx;", "h[n] = abar * (h[n] + bx);", "scan"),
    ("readout_before_update", "h[n] = abar * h[n] + bx;\n                acc += (double)Cm[r + n] * h[n];",
     "acc += (double)Cm[r + n] * h[n];\n                h[n] = abar * h[n] + bx;", "scan"),
    ("skip_dropped", "double out = acc + dsk * xv;\n            if (z) out *= silu_gate_f64((double)z[e]);\n            if (chans) y[i * L + t] = out;",
     "double out = acc;\n            if (z) out *= silu_gate_f64((double)z[e]);\n            if (chans) y[i * L + t] = out;", "scan"),
    ("gate_is_sigmoid", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));", "scan"),
    ("softplus_branch", "return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));",
     "return v > 0.0 ? log1p(exp(-v)) : log1p(exp(v));", "scan"),
    ("softplus_plain_log", "return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));",
     "return log(1.0 + exp(v));", "scan"),
    ("bias_ignored", "const double v = (double)delta[e] + bias;", "const double v = (double)delta[e];", "scan"),
    ("h0_ignored", "h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;", "scan"),
    ("h0_layout", "h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;", "h[n] = h0 ? h0[(d * batch + b) * N + n] : 0.0;",
     "scan"),
    ("bias_from_channel_0", "(double)delta_bias[d]", "(double)delta_bias[0]", "scan"),
    ("skip_from_channel_0", "const double dsk = Dskip ? (double)Dskip[d] : 0.0;",
     "const double dsk = Dskip ? (double)Dskip[0] : 0.0;", "scan"),
    ("h_final_index", "double *hf = chans ? h_final + i * N : h_final + (b * D + d) * N;",
     "double *hf = chans ? h_final + i * N : h_final + (d * batch + b) * N;", "scan"),
    ("ssd_dt_dropped_from_decay", "const double abar = exp(dtv * a);", "const double abar = exp(a);", "ssd"),
    ("ssd_head_index", "(double)dt_raw[(b * L + t) * H + hh]", "(double)dt_raw[(b * L + t) * H]", "ssd"),
    ("ssd_input_scale", "h[n] = abar * h[n] + dtv * (double)Bm[r + n] * xv;",
     "h[n] = abar * h[n] + (double)Bm[r + n] * xv;", "ssd"),
    ("ssd_x_layout", "const int64_t e = ((b * L + t) * H + hh) * P + p;",
     "const int64_t e = ((b * L + t) * P + p) * H + hh;", "ssd"),
    ("ssd_skip_from_head_0", "const double dsk = Dskip ? (double)Dskip[hh] : 0.0;",
     "const double dsk = Dskip ? (double)Dskip[0] : 0.0;", "ssd"),
    ("ssd_bias_from_head_0", "(double)dt_bias[hh]", "(double)dt_bias[0]", "ssd"),
    ("ssd_A_per_group", "const double a = (double)A[hh];", "const double a = (double)A[g];", "ssd"),
    ("ssd_h0_layout", "h[n] = h0 ? h0[c * N + n] : 0.0;",
     "h[n] = h0 ? h0[((p * H + hh) * batch + b) * N + n] : 0.0;", "ssd"),
    ("group_of_channel", "const int64_t g = d / (D / G);", "const int64_t g = d % G;", "scan"),
    ("ssd_group_of_head", "const int64_t g = hh / (H / G);", "const int64_t g = hh % G;", "ssd"),
    ("bwd_ddt_drops_decay_term", "ddt += gn * ((double)Bm[r + n] * xv + (double)A[d * N + n] * abar * hprev);",
     "ddt += gn * ((double)Bm[r + n] * xv);", "bwd"),
    ("bwd_adjoint_not_decayed", "g[n] = abar * gn;", "g[n] = gn;", "bwd"),
    ("bwd_dx_drops_skip", "dx[e] = dyc * dsk + dt * gB;", "dx[e] = dt * gB;", "bwd"),
    ("bwd_dC_previous_state", "pC[r + n] += dyc * hs[(t + 1) * N + n];", "pC[r + n] += dyc * hs[t * N + n];", "bwd"),
    ("bwd_softplus_derivative", "ddt / (1.0 + exp(-v))", "ddt / (1.0 + exp(v))", "bwd"),
    ("bwd_gate_derivative", "s * (1.0 + zv * (1.0 - s))", "s * (1.0 + zv * s)", "bwd"),
    ("bwd_dA_drops_dt", "dA[d * N + n] += gn * dt * abar * hprev;", "dA[d * N + n] += gn * abar * hprev;", "bwd"),
    ("bwd_dB_drops_x", "pB[r + n] += gn * dt * xv;", "pB[r + n] += gn * dt;", "bwd"),
    ("bwd_dDskip_ungated", "dDskip[d] += dyc * xv;", "dDskip[d] += (double)dy[e] * xv;", "bwd"),
    ("bwd_dbias_before_softplus", "dbias[d] += dd;", "dbias[d] += ddt;", "bwd"),
    ("bwd_dh0_not_decayed", "dh0[(b * D + d) * N + n] = g[n];",
     "dh0[(b * D + d) * N + n] = L > 0 ? g[n] / exp(dts[0] * (double)A[d * N + n]) : g[n];", "bwd"),
    ("bwd_dz_readout_previous_state", "yc += (double)Cm[r + n] * hs[(t + 1) * N + n];",
     "yc += (double)Cm[r + n] * hs[t * N + n];", "bwd"),
    ("conv_not_causal", "const int64_t s = t - (K - 1) + k;", "const int64_t s = t - k;", "conv"),
    ("conv_history_reversed", "x0[(b * (K - 1) + (K - 1) + s) * D + d]", "x0[(b * (K - 1) - 1 - s) * D + d]",
     "conv"),
    ("conv_state_off_by_one", "conv_input(x, x0, b, L - (K - 1) + j, L, D, K, d)",
     "conv_input(x, x0, b, L - K + j, L, D, K, d)", "conv"),
]

PINS = {"scan": oracle_pins.SCAN_PINS, "ssd": oracle_pins.SSD_PINS, "conv": oracle_pins.CONV_PINS,
        "bwd": oracle_pins.BWD_PINS}


@pytest.mark.parametrize("name,old,new,group", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, group):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found in oracle.c: %r" % old
    path_c = tmp_path / ("%s.c" % name)
    path_c.write_text(src.replace(old, new))
    path_so = str(tmp_path / ("lib%s.so" % name))
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
                           path_so, str(path_c), "-lm"])
    failed = []
    with oracle.using_library(path_so):
        for pin in PINS[group]:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name


# Mistakes in the SSD-form gradients (the composition in oracle/__init__.py over
# the scan gradients): (name, text in ssd_bwd, replacement)
SSD_BWD_MUTANTS = [
    ("ssd_bwd_group_index", "hs // (H // G)]\n    Cg", "hs // G]\n    Cg"),
    ("ssd_bwd_ddt_mean", '"ddt": o["ddelta"].reshape(batch, L, Hs, P).sum(-1)',
     '"ddt": o["ddelta"].reshape(batch, L, Hs, P).mean(-1)'),
    ("ssd_bwd_dt_tiled", "np.repeat(take(dt, 2), P, axis=2)", "np.tile(take(dt, 2), (1, 1, P))"),
    ("ssd_bwd_dA_one_state", '"dA": o["dA"].reshape(Hs, P, N).sum((1, 2))',
     '"dA": o["dA"].reshape(Hs, P, N).sum(1)[:, 0]'),
]


@pytest.mark.parametrize("name,old,new", SSD_BWD_MUTANTS, ids=[m[0] for m in SSD_BWD_MUTANTS])
def test_ssd_bwd_mutant_is_caught(monkeypatch, name, old, new):
    import inspect
    src = inspect.getsource(oracle.ssd_bwd)
    assert src.count(old) == 1, "mutation anchor not found in ssd_bwd: %r" % old
    ns = dict(oracle.__dict__)
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oracle, "ssd_bwd", ns["ssd_bwd"])
    failed = []
    for pin in oracle_pins.SSD_BWD_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
