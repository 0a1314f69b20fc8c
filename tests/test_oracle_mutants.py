"""Plants mistakes in copies of the oracle's C source (on the CPU) and checks
that the pins in test_oracle_pins.py catch every one of them."""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssm_oracle.c")

PINS = [pins.test_lti_convolution, pins.test_unrolled_sum_fp64, pins.test_delta_zero_keeps_state_exactly,
        pins.test_single_token_closed_form, pins.test_single_token_zero_state,
        pins.test_split_sequence_bit_exact, pins.test_decode_equals_scan_bit_exact,
        pins.test_reset_when_decay_underflows, pins.test_zero_A_is_prefix_sum,
        pins.test_softplus_identities_and_bias]

# (name, text in ssm_oracle.c, replacement)
MUTANTS = [
    ("decay-sign", "exp(dl * A[d * N + n]);", "exp(-dl * A[d * N + n]);"),
    ("drop-skip-term", "if (Dv) y += Dv[d] * ut;", ";"),
    ("swap-B-C", "dl * Bb[n * L + t] * ut", "dl * Cb[n * L + t] * ut"),
    ("gate-before-skip", "    if (Dv) y += Dv[d] * ut;                            /* skip term D*u         */\n"
     "    if (z) y *= oracle_silu(z[row + t]);",
     "    if (z) y *= oracle_silu(z[row + t]);\n    if (Dv) y += Dv[d] * ut;"),
    ("no-softplus", "return softplus ? oracle_softplus(x) : x;", "return x;"),
    ("no-bias", "double x = dt + (bias ? bias[d] : 0.0);", "double x = dt;"),
    ("readout-before-update", "      h[n] = abar * h[n] + bbar_u;\n      y += Cb[n * L + t] * h[n];",
     "      y += Cb[n * L + t] * h[n];\n      h[n] = abar * h[n] + bbar_u;"),
    ("ignore-h0", "h[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    ("exact-zoh-B", "const double bbar_u = dl * Bb[n * L + t] * ut;",
     "const double bbar_u = (A[d * N + n] != 0.0 ? (abar - 1.0) / A[d * N + n] : dl) * Bb[n * L + t] * ut;"),
    ("softplus-sign", "return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));",
     "return (x > 0.0 ? x : 0.0) + log1p(exp(fabs(x)));"),
    ("silu-sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("decode-drop-input", "s[n] = exp(dl * A[d * N + n]) * s[n] + dl * Bt[n] * xt;",
     "s[n] = exp(dl * A[d * N + n]) * s[n];"),
]


def _fails(fn):
    args = {"test_lti_convolution": {"with_h0": True}, "test_split_sequence_bit_exact": {"cut": 13}}
    try:
        fn(**args.get(fn.__name__, {}))
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(path), "-lm"])
    with oracle.use_library(str(lib)):
        caught = [fn.__name__ for fn in PINS if _fails(fn)]
    assert caught, f"no pin caught mutant {name}"


# Planted mistakes in the backward (scan_row_bwd), each to be caught by a pin
# in test_oracle_bwd_pins.py.
import test_oracle_bwd_pins as bpins  # noqa: E402

BWD_PINS = [
    lambda: [bpins.test_linear_inputs_exact_jvp(n, True) for n in bpins.LINEAR],
    lambda: [bpins.test_nonlinear_inputs_central_difference(n, True) for n in bpins.NONLINEAR],
    lambda: [bpins.test_nonlinear_inputs_central_difference(n, False) for n in bpins.NONLINEAR],
    bpins.test_every_element_of_du_by_unit_directions,
    bpins.test_last_state_gradient_wrt_h0_is_the_total_decay,
    bpins.test_single_token_du_closed_form,
]

BWD_MUTANTS = [
    ("bwd-carry-without-decay", "g[n] = et * adj;", "g[n] = adj;"),
    ("bwd-dz-drops-term", "dz[row + t] = dy * yt * sg * (1.0 + zt * (1.0 - sg));",
     "dz[row + t] = dy * yt * sg;"),
    ("bwd-dC-previous-state", "dCrow[n * L + t] = dy * ht;", "dCrow[n * L + t] = dy * hp;"),
    ("bwd-ddelta-drops-decay-term", "dstep += adj * (Bb[n * L + t] * ut + A[d * N + n] * et * hp);",
     "dstep += adj * Bb[n * L + t] * ut;"),
    ("bwd-no-softplus-derivative", "const double dx = softplus ? dstep * logistic(xt) : dstep;",
     "const double dx = dstep;"),
    ("bwd-dA-drops-step", "dArow[n] += adj * step * et * hp;", "dArow[n] += adj * et * hp;"),
    ("bwd-dB-readout-only", "dBrow[n * L + t] = adj * step * ut;", "dBrow[n * L + t] = dy * step * ut;"),
    ("bwd-ignores-dlast", "g[n] = dlast ? dlast[(b * dim + d) * N + n] : 0.0;", "g[n] = 0.0;"),
    ("bwd-du-drops-skip", "double dut = Dv ? dy * Dv[d] : 0.0;", "double dut = 0.0;"),
    ("bwd-du-sign", "dut += adj * step * Bb[n * L + t];", "dut -= adj * step * Bb[n * L + t];"),
]


def _fails_call(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_backward_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(path), "-lm"])
    with oracle.use_library(str(lib)):
        caught = [i for i, fn in enumerate(BWD_PINS) if _fails_call(fn)]
    assert caught, f"no pin caught mutant {name}"


# Planted mistakes in the conv branch oracle, each to be caught by a pin in
# test_oracle_conv_pins.py.
import test_oracle_conv_pins as cpins  # noqa: E402

CONV_PINS = [
    lambda: [cpins.test_zero_state_is_a_truncated_full_convolution(K) for K in (1, 2, 4)],
    cpins.test_impulse_reads_the_kernel_back,
    cpins.test_causality,
    lambda: [cpins.test_split_with_state_is_bit_exact(c) for c in (1, 3, 9)],
    cpins.test_returned_state_is_the_last_inputs,
    cpins.test_decode_steps_equal_prefill_bit_exact,
    cpins.test_width_one_is_pointwise,
]

CONV_MUTANTS = [
    ("conv-reversed-kernel", "acc += w[d * K + k] * xv;", "acc += w[d * K + (K - 1 - k)] * xv;"),
    ("conv-off-by-one", "const int64_t s = t - (K - 1) + k;           /* input index */",
     "const int64_t s = t - K + k;           /* input index */"),
    ("conv-ignores-state", "const double xv = s >= 0 ? xr[s] : (state_in ? state_in[r * K + K + s] : 0.0);",
     "const double xv = s >= 0 ? xr[s] : 0.0;"),
    ("conv-no-bias", "double acc = bias ? bias[d] : 0.0;\n        for (int64_t k = 0; k < K; ++k) {",
     "double acc = 0.0;\n        for (int64_t k = 0; k < K; ++k) {"),
    ("conv-state-out-shifted", "const int64_t s = seqlen - K + k;", "const int64_t s = seqlen - K + k - 1;"),
    ("conv-decode-no-shift", "for (int64_t k = 0; k + 1 < K; ++k) s[k] = s[k + 1];", ";"),
]


@pytest.mark.parametrize("name,old,new", CONV_MUTANTS, ids=[m[0] for m in CONV_MUTANTS])
def test_conv_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(path), "-lm"])
    with oracle.use_library(str(lib)):
        caught = [i for i, fn in enumerate(CONV_PINS) if _fails_call(fn)]
    assert caught, f"no pin caught mutant {name}"


# Planted mistakes in the group lookup and the per-group sums, each to be
# caught by a pin in test_oracle_general_pins.py.
import test_oracle_general_pins as gpins  # noqa: E402

GROUP_PINS = [
    lambda: [gpins.test_unrolled_sum_any_dstate_groups_and_sign(N, G) for N in (8, 33) for G in (2, 4)],
    gpins.test_group_decomposition_bit_exact,
    lambda: [gpins.test_decode_equals_scan_grouped(N, G) for N, G in ((8, 2), (64, 4))],
    lambda: [gpins.test_grouped_backward_exact_jvp(n, 8, 2) for n in ("B", "C", "u", "h0")],
    gpins.test_grouped_backward_decomposes_by_group,
]

GROUP_MUTANTS = [
    ("group-interleaved", "const int64_t grp = b * G + d / (dim / G);           /* this channel's B/C group */",
     "const int64_t grp = b * G + d % G;"),
    ("group-ignored", "const int64_t grp = b * G + d / (dim / G);           /* this channel's B/C group */",
     "const int64_t grp = b * G;"),
    ("decode-group-interleaved", "const double* Bt = Bm + (b * G + d / (dim / G)) * N;  /* this channel's group */",
     "const double* Bt = Bm + (b * G + d % G) * N;"),
    ("bwd-group-sum-all-channels", "for (int64_t d = gi * cpg; d < (gi + 1) * cpg; ++d) {",
     "for (int64_t d = 0; d < dim; ++d) {"),
    ("bwd-group-interleaved", "const int64_t grp = b * G + d / (dim / G);\n",
     "const int64_t grp = b * G + d % G;\n"),
]


@pytest.mark.parametrize("name,old,new", GROUP_MUTANTS, ids=[m[0] for m in GROUP_MUTANTS])
def test_group_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(path), "-lm"])
    with oracle.use_library(str(lib)):
        caught = [i for i, fn in enumerate(GROUP_PINS) if _fails_call(fn)]
    assert caught, f"no pin caught mutant {name}"


# Planted mistakes in the Mamba-2 (SSD layer) oracle, each to be caught by a
# pin in test_oracle_ssd_pins.py.
import test_oracle_ssd_pins as spins  # noqa: E402

SSD_PINS = [
    lambda: [spins.test_equals_mamba1_oracle_with_shared_head_parameters_bit_exact(*s)
             for s in ((4, 3, 2, 5), (6, 1, 3, 8))],
    lambda: [spins.test_structured_matrix_form(4, 3, 2, 5, 20, sp) for sp in (True, False)],
    spins.test_single_token_closed_form,
    spins.test_zero_input_decays_every_state_by_the_head_scalar,
]

SSD_MUTANTS = [
    ("ssd-group-interleaved", "const int64_t g = h / (H / G);                      /* the head's B/C group */",
     "const int64_t g = h % G;"),
    ("ssd-step-of-another-head", "const double step = step_size(dt[(b * L + t) * H + h], bias, h, softplus);",
     "const double step = step_size(dt[(b * L + t) * H + (h + 1) % H], bias, h, softplus);"),
    ("ssd-drop-skip", "if (Dv) y += Dv[h] * xv;", ";"),
    ("ssd-input-not-scaled-by-step", "S[p * N + n] = decay * S[p * N + n] + step * Bt[n] * xv;",
     "S[p * N + n] = decay * S[p * N + n] + Bt[n] * xv;"),
    ("ssd-ignore-h0", "S[i] = h0 ? h0[(b * H + h) * P * N + i] : 0.0;", "S[i] = 0.0;"),
    ("ssd-readout-before-update",
     "        S[p * N + n] = decay * S[p * N + n] + step * Bt[n] * xv;\n        y += Ct[n] * S[p * N + n];",
     "        y += Ct[n] * S[p * N + n];\n        S[p * N + n] = decay * S[p * N + n] + step * Bt[n] * xv;"),
    ("ssd-swap-B-C", "const double* Bt = Bm + ((b * L + t) * G + g) * N;",
     "const double* Bt = Cm + ((b * L + t) * G + g) * N;"),
]


@pytest.mark.parametrize("name,old,new", SSD_MUTANTS, ids=[m[0] for m in SSD_MUTANTS])
def test_ssd_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(path), "-lm"])
    with oracle.use_library(str(lib)):
        caught = [i for i, fn in enumerate(SSD_PINS) if _fails_call(fn)]
    assert caught, f"no pin caught mutant {name}"
