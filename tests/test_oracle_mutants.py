"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a copy of the oracle source (on the
CPU, in a temporary directory), builds it, and runs the pin suite against it:
at least one pin must fail.  This shows the pins constrain every term of the
recurrence, the epilogue, the layouts and the conv prologue.
"""
import os
import re
import subprocess

import pytest

from oracle import oracle as orc
import tests.test_oracle_pins as pins

MUTANTS = {
    "drop_delta_bias": ("if (a->delta_bias) dt += (double)a->delta_bias[d];", ""),
    "softplus_sign": ("return v + log1p(exp(-v));", "return v + log1p(exp(v));"),
    "decay_sign": ("exp(dt * (double)a->A[d * n + s])", "exp(-dt * (double)a->A[d * n + s])"),
    "drop_dt_in_input": ("dt * Bv * ut", "Bv * ut"),
    "C_reads_B": ("bc_at(a->C, a->C_kind", "bc_at(a->B, a->B_kind"),
    "A_state_reversed": ("(double)a->A[d * n + s]", "(double)a->A[d * n + (n - 1 - s)]"),
    "D_after_gate": ("if (a->D) y += (double)a->D[d] * ut;\n        if (a->z) y *= oracle_silu(load_io(a->z, a->io_dtype, base + t));",
                     "if (a->z) y *= oracle_silu(load_io(a->z, a->io_dtype, base + t));\n        if (a->D) y += (double)a->D[d] * ut;"),
    "group_interleaved": ("int64_t g = d / per_group;", "int64_t g = d % a->ngroups; (void)per_group;"),
    "contract_old_state": ("x[s] = dA * x[s] + dt * Bv * ut;\n            y += bc_at(a->C, a->C_kind, a->io_dtype, a, b, d, s, t) * x[s];",
                           "y += bc_at(a->C, a->C_kind, a->io_dtype, a, b, d, s, t) * x[s];\n            x[s] = dA * x[s] + dt * Bv * ut;"),
    "fixed_BC_transposed": ("if (kind == OR_BC_FIXED) return load_io(p, dtype, d * a->dstate + s);",
                            "if (kind == OR_BC_FIXED) return load_io(p, dtype, (s * a->dim + d) % (a->dim * a->dstate));"),
    "time_index_shift": ("* a->seqlen + t);", "* a->seqlen + (t + 1) % a->seqlen);"),
    "ignore_initial_state": ("a->initial_state ? a->initial_state[row * n + s] : 0.0", "0.0"),
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "conv_flipped": ("acc += (double)w[k] * load_io(x, dtype, base + src);",
                     "acc += (double)w[W - 1 - k] * load_io(x, dtype, base + src);"),
    "conv_pad_off_by_one": ("int64_t src = t - (W - 1) + k;", "int64_t src = t - W + k;"),
    "conv_drop_bias": ("double acc = bias;", "double acc = 0.0; (void)bias;"),
    "bf16_ties_away": ("double r = nearbyint(ldexp(v, -q));", "double r = round(ldexp(v, -q));"),
    "bf16_truncate": ("double r = nearbyint(ldexp(v, -q));", "double r = trunc(ldexp(v, -q));"),
    "last_state_stale": ("for (int64_t s = 0; s < n; ++s) last[s] = x[s];",
                         "for (int64_t s = 0; s < n; ++s) last[s] = 0.5 * x[s];"),
}


def _pin_calls():
    calls = []
    for name in dir(pins):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        if name == "test_brute_force_tiny":
            for fixed in (False, True):
                for sp in (True, False):
                    calls.append((f"{name}[{fixed},{sp}]", lambda f=fn, a=fixed, b=sp: f(a, b)))
        else:
            calls.append((name, fn))
    return calls


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, tmp_path):
    src = open(orc.SRC).read()
    old, new = MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    str(path), "-lm"], check=True, capture_output=True)
    orc.use_library(lib)
    caught = []
    try:
        for name, call in _pin_calls():
            try:
                call()
            except AssertionError:
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, f"no pin caught mutant {mutant}"


# --------------------------------------------------------------------------
# the decode functions against their own pins
# --------------------------------------------------------------------------

import tests.test_oracle_decode_pins as dpins  # noqa: E402

DECODE_MUTANTS = {
    "su_contract_old_state": ("y += load_io(C, io_dtype, bc) * h;",
                              "y += load_io(C, io_dtype, bc) * state_in[row * dstate + s];"),
    "su_drop_dt_in_input": ("+ step * load_io(B, io_dtype, bc) * xv;", "+ load_io(B, io_dtype, bc) * xv;"),
    "su_group_interleaved": ("const int64_t grp = d / per_group;",
                             "const int64_t grp = d % ngroups; (void)per_group;"),
    "su_bias_after_softplus": ("if (dt_bias) step += (double)dt_bias[d];\n            if (dt_softplus) step = oracle_softplus(step);",
                               "if (dt_softplus) step = oracle_softplus(step);\n            if (dt_bias) step += (double)dt_bias[d];"),
    "su_drop_D": ("if (D) y += (double)D[d] * xv;", ""),
    "cu_ring_read_off_by_one": ("int64_t slot = ((int64_t)cache_seqlens[b] + t - back) % state_len;",
                                "int64_t slot = ((int64_t)cache_seqlens[b] + t - back + 1) % state_len;"),
    "cu_ring_write_off_by_one": ("int64_t slot = ((int64_t)cache_seqlens[b] + t) % state_len;",
                                 "int64_t slot = ((int64_t)cache_seqlens[b] + t + 1) % state_len;"),
    "cu_shift_stale": ("memcpy(so, hist + es * (size_t)seqlen, es * (size_t)state_len);",
                       "memcpy(so, hist, es * (size_t)state_len);"),
    "cu_window_reversed": ("acc += (double)weight[d * width + k] * win[k];",
                           "acc += (double)weight[d * width + k] * win[width - 1 - k];"),
}


def _decode_pin_calls():
    F32, BF16 = orc.F32, orc.BF16
    return [
        ("chain_scan_f32", lambda: dpins.test_state_update_chain_equals_scan(F32, 2, True)),
        ("chain_scan_bf16_nosp", lambda: dpins.test_state_update_chain_equals_scan(BF16, 1, False)),
        ("a_zero", dpins.test_state_update_a_zero_is_accumulation),
        ("zero_step", dpins.test_state_update_zero_step_keeps_state),
        ("one_hot_c", dpins.test_state_update_one_hot_c_reads_one_state),
        ("groups", dpins.test_state_update_groups_broadcast),
        ("conv_chain", lambda: dpins.test_conv_update_chain_equals_conv(F32, orc.ACT_SILU, 4)),
        ("conv_multi_shift", lambda: dpins.test_conv_update_multi_token_equals_single_steps(False)),
        ("conv_multi_ring", lambda: dpins.test_conv_update_multi_token_equals_single_steps(True)),
        ("conv_identity", dpins.test_conv_update_identity_kernel_and_history),
        ("conv_ring_slots", dpins.test_conv_update_ring_reads_the_slots_before_the_position),
    ]


@pytest.mark.parametrize("mutant", sorted(DECODE_MUTANTS))
def test_decode_pins_catch_mutant(mutant, tmp_path):
    src = open(orc.SRC).read()
    old, new = DECODE_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    str(path), "-lm"], check=True, capture_output=True)
    orc.use_library(lib)
    caught = []
    try:
        for name, call in _decode_pin_calls():
            try:
                call()
            except AssertionError:
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, f"no pin caught mutant {mutant}"


# --------------------------------------------------------------------------
# the Mamba-2 scan against its own pins
# --------------------------------------------------------------------------

import tests.test_oracle_ssd_pins as spins  # noqa: E402

SSD_MUTANTS = {
    "ssd_group_interleaved": ("h = bh % nheads, g = h / hpg;", "h = bh % nheads, g = h % ngroups;"),
    "ssd_decay_sign": ("const double dA = exp(step * (double)A[h]);",
                       "const double dA = exp(-step * (double)A[h]);"),
    "ssd_contract_old_state": (
        "*hs = dA * *hs + step * load_io(B, io_dtype, bcb + s) * xv;\n"
        "                            y += load_io(C, io_dtype, bcb + s) * *hs;",
        "y += load_io(C, io_dtype, bcb + s) * *hs;\n"
        "                            *hs = dA * *hs + step * load_io(B, io_dtype, bcb + s) * xv;"),
    "ssd_drop_dt_in_input": ("*hs = dA * *hs + step * load_io(B, io_dtype, bcb + s) * xv;",
                             "*hs = dA * *hs + load_io(B, io_dtype, bcb + s) * xv;"),
    "ssd_D_channel_index": ("y += (double)(D_per_channel ? D[h * headdim + pp]",
                            "y += (double)(D_per_channel ? D[pp % nheads * headdim + h % headdim]"),
    "ssd_ignore_initial": ("H[i] = initial_states ? initial_states[sbase + i] : 0.0;", "H[i] = 0.0;"),
    "ssd_limit_swapped": ("step = step < dt_min ? dt_min : (step > dt_max ? dt_max : step);",
                          "step = step < dt_max ? dt_max : (step > dt_min ? dt_min : step);"),
    "ssd_limit_before_softplus": (
        "if (dt_softplus) step = oracle_softplus(step);\n"
        "                    if (dt_limit) step = step < dt_min ? dt_min : (step > dt_max ? dt_max : step);",
        "if (dt_limit) step = step < dt_min ? dt_min : (step > dt_max ? dt_max : step);\n"
        "                    if (dt_softplus) step = oracle_softplus(step);"),
    "ssd_no_reset": ("if (seq_idx && t > 0 && seq_idx[b * seqlen + t] != seq_idx[b * seqlen + t - 1])",
                     "if (0)"),
    "ssd_reset_after_update": (
        "if (seq_idx && t > 0 && seq_idx[b * seqlen + t] != seq_idx[b * seqlen + t - 1])",
        "if (seq_idx && t > 1 && seq_idx[b * seqlen + t - 1] != seq_idx[b * seqlen + t - 2])"),
}


def _ssd_pin_calls():
    F32, BF16 = orc.F32, orc.BF16
    return [
        ("flattened_f32", lambda: spins.test_ssd_equals_selective_scan_flattened(F32, 2, True)),
        ("flattened_bf16", lambda: spins.test_ssd_equals_selective_scan_flattened(BF16, 1, False)),
        ("dual", lambda: spins.test_ssd_dual_quadratic_form(True)),
        ("split", spins.test_ssd_split_continuation),
        ("D_forms", spins.test_ssd_D_per_head_equals_per_channel),
        ("dual_limit_seq", lambda: spins.test_ssd_dual_form_with_dt_limit_and_seq_idx(True)),
        ("separate_runs", spins.test_ssd_seq_idx_equals_separate_runs),
    ]


@pytest.mark.parametrize("mutant", sorted(SSD_MUTANTS))
def test_ssd_pins_catch_mutant(mutant, tmp_path):
    src = open(orc.SRC).read()
    old, new = SSD_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    str(path), "-lm"], check=True, capture_output=True)
    orc.use_library(lib)
    caught = []
    try:
        for name, call in _ssd_pin_calls():
            try:
                call()
            except AssertionError:
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, f"no pin caught mutant {mutant}"


# --------------------------------------------------------------------------
# the selective-scan backward against its own pins
# --------------------------------------------------------------------------

import tests.test_oracle_bwd_pins as bpins  # noqa: E402

BWD_MUTANTS = {
    "bwd_softplus_derivative_sign": ("const double dsp = delta_softplus ? 1.0 / (1.0 + exp(-raw)) : 1.0;",
                                     "const double dsp = delta_softplus ? 1.0 / (1.0 + exp(raw)) : 1.0;"),
    "bwd_dA_drops_step": ("dA[d * n + s] += da * dt * aa;", "dA[d * n + s] += da * aa;"),
    "bwd_silu_derivative": ("dz[base + t] = dy * pre * sg * (1.0 + zt * (1.0 - sg));",
                            "dz[base + t] = dy * pre * sg * (1.0 + zt * sg);"),
    "bwd_dC_old_state": ("const double dCv = dy * xs[(t + 1) * n + s];",
                         "const double dCv = dy * xs[t * n + s];"),
    "bwd_adjoint_not_decayed": ("h[s] *= aa;                               /* carried to t-1 */", ""),
    "bwd_bias_grad_skips_softplus": ("if (ddelta_bias) ddelta_bias[d] += ddt * dsp;",
                                     "if (ddelta_bias) ddelta_bias[d] += ddt;"),
    "bwd_dB_group_zero": ("else dB[((b * ngroups + g) * n + s) * l + t] += dBv;",
                          "else dB[((b * ngroups + 0 * g) * n + s) * l + t] += dBv;"),
    "bwd_du_misses_input_path": ("dut += h[s] * dt * Bv;", ""),
    "bwd_dD_ungated": ("if (D) dD[d] += dy * ut;\n", "if (D) dD[d] += dout[base + t] * ut;\n"),
}


def _bwd_pin_calls():
    calls = [(f"fd_{c}_{sp}", lambda c=c, sp=sp: bpins.test_backward_matches_finite_differences(c, sp))
             for c in sorted(bpins.CASES) for sp in (True, False)]
    calls += [("euler", lambda: bpins.test_backward_euler_identities(True)),
              ("init_closed_form", bpins.test_backward_initial_state_gradient_closed_form)]
    return calls


@pytest.mark.parametrize("mutant", sorted(BWD_MUTANTS))
def test_bwd_pins_catch_mutant(mutant, tmp_path):
    src = open(orc.SRC).read()
    old, new = BWD_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    str(path), "-lm"], check=True, capture_output=True)
    orc.use_library(lib)
    caught = []
    try:
        for name, call in _bwd_pin_calls():
            try:
                call()
            except AssertionError:
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, f"no pin caught mutant {mutant}"


# --------------------------------------------------------------------------
# the conv's optional inputs against their own pins
# --------------------------------------------------------------------------

import tests.test_oracle_conv_ex_pins as cpins  # noqa: E402

CONV_EX_MUTANTS = {
    "cx_seq_mask_ignored": ("if (src < 0 || seq_idx[b * seqlen + src] != seq_idx[b * seqlen + t]) continue;",
                            "if (src < 0) continue;"),
    "cx_initial_shifted": ("load_io(initial_states, io_dtype, row * H + H + (src))",
                           "load_io(initial_states, io_dtype, row * H + H - 1 + (src) + ((src) == -H))"),
    "cx_final_off_by_one": ("final_states[row * H + j] = XE(seqlen - H + j);",
                            "final_states[row * H + j] = XE(seqlen - H + j - 1);"),
    "cx_seq_compare_previous": ("seq_idx[b * seqlen + src] != seq_idx[b * seqlen + t]",
                                "seq_idx[b * seqlen + src] != seq_idx[b * seqlen + (t > 0 ? t - 1 : 0)]"),
}


def _conv_ex_pin_calls():
    F32, BF16 = orc.F32, orc.BF16
    return [
        ("plain", lambda: cpins.test_no_options_is_the_plain_conv(F32, 4)),
        ("states_9", lambda: cpins.test_initial_and_final_states(F32, 9)),
        ("states_2", lambda: cpins.test_initial_and_final_states(BF16, 2)),
        ("split", cpins.test_split_continuation_through_states),
        ("seq", lambda: cpins.test_seq_idx_packed_sequences(F32)),
    ]


@pytest.mark.parametrize("mutant", sorted(CONV_EX_MUTANTS))
def test_conv_ex_pins_catch_mutant(mutant, tmp_path):
    src = open(orc.SRC).read()
    old, new = CONV_EX_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    str(path), "-lm"], check=True, capture_output=True)
    orc.use_library(lib)
    caught = []
    try:
        for name, call in _conv_ex_pin_calls():
            try:
                call()
            except AssertionError:
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, f"no pin caught mutant {mutant}"


# --------------------------------------------------------------------------
# fp16 io against its own pins
# --------------------------------------------------------------------------

import tests.test_oracle_f16_pins as fpins  # noqa: E402

F16_MUTANTS = {
    "f16_ties_away": ("double out = ldexp(nearbyint(ldexp(v, -q)), q);", "double out = ldexp(round(ldexp(v, -q)), q);"),
    "f16_exponent_bias": ("else v = ldexp((double)(1024 + fr), ex - 25);", "else v = ldexp((double)(1024 + fr), ex - 24);"),
    "f16_min_normal": ("if (e < -14) e = -14;", "if (e < -15) e = -15;"),
    "f16_read_as_bf16": ("if (dtype == OR_F16) return oracle_f16_bits_to_double(((const uint16_t *)p)[i]);",
                         "if (dtype == OR_F16) return bf16_bits_to_double(((const uint16_t *)p)[i]);"),
}


@pytest.mark.parametrize("mutant", sorted(F16_MUTANTS))
def test_f16_pins_catch_mutant(mutant, tmp_path):
    src = open(orc.SRC).read()
    old, new = F16_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    str(path), "-lm"], check=True, capture_output=True)
    orc.use_library(lib)
    caught = []
    try:
        for name, call in (("decode", fpins.test_decode_every_bit_pattern),
                           ("round", fpins.test_rounding_matches_numpy),
                           ("scan", fpins.test_scan_f16_io_equals_f32_io_of_the_same_values)):
            try:
                call()
            except AssertionError:
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, f"no pin caught mutant {mutant}"


# --------------------------------------------------------------------------
# the complex-A scan against its own pins
# --------------------------------------------------------------------------

import tests.test_oracle_complex_pins as xpins  # noqa: E402

COMPLEX_MUTANTS = {
    "cplx_conj_rotation": ("const double complex dA = cexp(dt * Av);", "const double complex dA = cexp(dt * conj(Av));"),
    "cplx_conj_C": ("y += creal(bc_at_c(a->C, a->C_kind, a->io_dtype, a, b, d, s, t) * x[s]);",
                  "y += creal(conj(bc_at_c(a->C, a->C_kind, a->io_dtype, a, b, d, s, t)) * x[s]);"),
    "cplx_imag_output": ("y += creal(bc_at_c(", "y += cimag(bc_at_c("),
    "cplx_drop_imag_of_BC": ("return load_io(p, dtype, 2 * i) + I * load_io(p, dtype, 2 * i + 1);",
                           "return load_io(p, dtype, 2 * i) + 0.0 * load_io(p, dtype, 2 * i + 1);"),
    "cplx_pair_order": ("return load_io(p, dtype, 2 * i) + I * load_io(p, dtype, 2 * i + 1);",
                      "return load_io(p, dtype, 2 * i + 1) + I * load_io(p, dtype, 2 * i);"),
    "cplx_init_imag_dropped": ("+ I * a->initial_state[2 * (row * n + s) + 1]", "+ 0.0 * a->initial_state[2 * (row * n + s) + 1]"),
    "cplx_last_imag": ("last[2 * s + 1] = cimag(x[s]);", "last[2 * s + 1] = -cimag(x[s]);"),
    "cplx_group_interleaved": ("const int64_t g = d / (a->dim / a->ngroups);", "const int64_t g = d % a->ngroups;"),
    "cplx_drop_dt_in_input": ("x[s] = dA * x[s] + dt * bc_at_c(", "x[s] = dA * x[s] + bc_at_c("),
}


def _complex_pin_calls():
    F32, BF16 = orc.F32, orc.BF16
    return [
        ("real_case_f32_g2", lambda: xpins.test_complex_real_case_equals_real_scan(F32, False, 2)),
        ("real_case_bf16_fixed", lambda: xpins.test_complex_real_case_equals_real_scan(BF16, True, 1)),
        ("brute_varying", lambda: xpins.test_complex_brute_force_tiny(False, True)),
        ("brute_fixed", lambda: xpins.test_complex_brute_force_tiny(True, False)),
        ("rotation", xpins.test_complex_rotation_closed_form),
        ("conjugate", xpins.test_complex_conjugate_symmetry),
    ]


@pytest.mark.parametrize("mutant", sorted(COMPLEX_MUTANTS))
def test_complex_pins_catch_mutant(mutant, tmp_path):
    src = open(orc.SRC).read()
    old, new = COMPLEX_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    str(path), "-lm"], check=True, capture_output=True)
    orc.use_library(lib)
    caught = []
    try:
        for name, call in _complex_pin_calls():
            try:
                call()
            except AssertionError:
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, f"no pin caught mutant {mutant}"


# --------------------------------------------------------------------------
# the complex-A backward against its own pins
# --------------------------------------------------------------------------

import tests.test_oracle_complex_bwd_pins as xbpins  # noqa: E402

COMPLEX_BWD_MUTANTS = {
    "cbwd_h_from_C_unconjugated": ("h[s] += dy * conj(Cv);                              /* h_t */",
                                   "h[s] += dy * Cv;"),
    "cbwd_carry_unconjugated": ("h[s] = conj(aa) * h[s];", "h[s] = aa * h[s];"),
    "cbwd_dC_unconjugated": ("const double complex gC = dy * conj(xs[(t + 1) * n + s]);",
                             "const double complex gC = dy * xs[(t + 1) * n + s];"),
    "cbwd_dA_unconjugated": ("const double complex gA = conj(dt * aa) * ga;",
                             "const double complex gA = dt * aa * ga;"),
    "cbwd_ga_old_state_unconjugated": ("const double complex ga = h[s] * conj(xs[t * n + s]);",
                                       "const double complex ga = h[s] * xs[t * n + s];"),
    "cbwd_dB_imag_sign": ("dB[2 * ib + 1] += cimag(gB);", "dB[2 * ib + 1] -= cimag(gB);"),
    "cbwd_dt_term_drops_rotation": ("ddt += creal(ga * conj(Av * aa))", "ddt += creal(ga * creal(Av) * conj(aa))"),
    "cbwd_dinit_imag": ("dinit[2 * (row * n + s) + 1] = cimag(h[s]);", "dinit[2 * (row * n + s) + 1] = 0.0;"),
}


def _complex_bwd_pin_calls():
    return [
        ("fd_varying", lambda: xbpins.test_complex_backward_matches_finite_differences("varying", True)),
        ("fd_fixed_BC", lambda: xbpins.test_complex_backward_matches_finite_differences("fixed_BC", False)),
        ("conjugation", xbpins.test_conjugation_conjugates_the_complex_gradients),
        ("euler", xbpins.test_euler_identity_in_u_and_the_initial_state),
    ]


@pytest.mark.parametrize("mutant", sorted(COMPLEX_BWD_MUTANTS))
def test_complex_bwd_pins_catch_mutant(mutant, tmp_path):
    src = open(orc.SRC).read()
    old, new = COMPLEX_BWD_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    str(path), "-lm"], check=True, capture_output=True)
    orc.use_library(lib)
    caught = []
    try:
        for name, call in _complex_bwd_pin_calls():
            try:
                call()
            except AssertionError:
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, f"no pin caught mutant {mutant}"


# --------------------------------------------------------------------------
# the split chunk-scan operators against their own pins
# --------------------------------------------------------------------------

import tests.test_oracle_ssd_split_pins as sspins  # noqa: E402

SSD_SPLIT_MUTANTS = {
    "split_restart_not_zeroing_factor": ("            reach = 0.0;\n", ""),
    "split_factor_skips_last_token": ("        reach *= decay;\n",
                                      "        if (t + 1 < t1) reach *= decay;\n"),
    "split_restart_ignores_first_token": ("if (ssd_part_restarts(seq_idx, b, t, seqlen)) {",
                                          "if (t > t0 && ssd_part_restarts(seq_idx, b, t, seqlen)) {"),
    "split_passing_state_after_update": (
        "                carried[(c * nbh + bh) * ps + i] = S;\n"
        "                S = decays[c * nbh + bh] * S + states[(c * nbh + bh) * ps + i];",
        "                S = decays[c * nbh + bh] * S + states[(c * nbh + bh) * ps + i];\n"
        "                carried[(c * nbh + bh) * ps + i] = S;"),
    "split_passing_ignores_initial": ("double S = initial_states ? initial_states[bh * ps + i] : 0.0;",
                                      "double S = 0.0;"),
    "split_scan_from_wrong_chunk": ("memcpy(St, carried + (c * batch * nheads + bh) * ps",
                                    "memcpy(St, carried + ((c > 0 ? c - 1 : 0) * batch * nheads + bh) * ps"),
    "split_scan_last_chunk_short": ("t1 = t0 + chunk_size < seqlen ? t0 + chunk_size : seqlen;\n"
                                    "            ssd_part_run(",
                                    "t1 = t0 + chunk_size < seqlen ? t0 + chunk_size : seqlen - 1;\n"
                                    "            ssd_part_run("),
}


def _ssd_split_pin_calls():
    return [
        ("compose_seq", lambda: sspins.test_composition_is_the_scan(4, "seq")),
        ("compose_init", lambda: sspins.test_composition_is_the_scan(5, "init")),
        ("compose_bf16", lambda: sspins.test_composition_is_the_scan(4, "bf16_all")),
        ("chunk_alone", sspins.test_chunk_state_is_the_chunk_alone_from_zero),
        ("factor_zero", sspins.test_chunk_state_factor_is_zero_where_a_sequence_starts),
        ("affine", sspins.test_state_passing_is_affine),
        ("true_boundaries", sspins.test_chunk_scan_from_the_true_boundary_states),
    ]


@pytest.mark.parametrize("mutant", sorted(SSD_SPLIT_MUTANTS))
def test_ssd_split_pins_catch_mutant(mutant, tmp_path):
    src = open(orc.SRC).read()
    old, new = SSD_SPLIT_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    str(path), "-lm"], check=True, capture_output=True)
    orc.use_library(lib)
    caught = []
    try:
        for name, call in _ssd_split_pin_calls():
            try:
                call()
            except AssertionError:
                caught.append(name)
    finally:
        orc.use_library(None)
    assert caught, f"no pin caught mutant {mutant}"
