"""The oracle's pins catch plausible mistakes.

Each case below plants one mistake in a copy of oracle.c (a dropped term, a
wrong sign, exponent or index, a swapped operand, a changed tie rule),
builds it with gcc, routes the oracle package to that build and runs the pins
from test_oracle_pins.py that are named as its witnesses: every witness must
fail on the mutant.  A control build of the unmodified source passes the same
pins, so a failure is the mistake's doing and not the build's.  CPU only.
"""
import os

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c (must occur once), replacement, witness pins)
MUTANTS = [
    # ---- AdamW
    ("adamw_decay_after_update",
     "        p[i] = p[i] * (1.0 - lr * wd);\n        m[i] = beta1 * m[i] + (1.0 - beta1) * g[i];\n"
     "        v[i] = beta2 * v[i] + (1.0 - beta2) * g[i] * g[i];\n"
     "        double h = sqrt(v[i]) / bc2_sqrt + eps;\n        p[i] = p[i] - step_size * m[i] / h;\n",
     "        m[i] = beta1 * m[i] + (1.0 - beta1) * g[i];\n"
     "        v[i] = beta2 * v[i] + (1.0 - beta2) * g[i] * g[i];\n"
     "        double h = sqrt(v[i]) / bc2_sqrt + eps;\n"
     "        p[i] = (p[i] - step_size * m[i] / h) * (1.0 - lr * wd);\n",
     ["test_adamw_fresh_step_closed_form", "test_adamw_matches_torch_float64",
      "test_mutant_fails_torch_referee", "test_one_step_gap_identity",
      "test_fresh_step_gap_lr01_wd01"]),
    ("adamw_decay_sign",
     "        p[i] = p[i] * (1.0 - lr * wd);\n        m[i] = beta1",
     "        p[i] = p[i] * (1.0 + lr * wd);\n        m[i] = beta1",
     ["test_adamw_fresh_step_closed_form", "test_adamw_constant_gradient_closed_form"]),
    ("adamw_decay_without_lr",
     "        p[i] = p[i] * (1.0 - lr * wd);\n        m[i] = beta1",
     "        p[i] = p[i] * (1.0 - wd);\n        m[i] = beta1",
     ["test_adamw_fresh_step_closed_form", "test_adamw_matches_torch_float64"]),
    ("adamw_second_moment_not_squared_bias_correction",
     "double h = sqrt(v[i]) / bc2_sqrt + eps;",
     "double h = sqrt(v[i]) / bc2 + eps;",
     ["test_adamw_fresh_step_closed_form", "test_adamw_matches_torch_float64",
      "test_adamw_constant_gradient_closed_form"]),
    ("adamw_eps_inside_sqrt",
     "double h = sqrt(v[i]) / bc2_sqrt + eps;",
     "double h = sqrt(v[i] / bc2 + eps);",
     ["test_adamw_fresh_step_closed_form", "test_adamw_matches_torch_float64"]),
    ("adamw_first_moment_not_bias_corrected",
     "double step_size = lr / bc1;",
     "double step_size = lr;",
     ["test_adamw_fresh_step_closed_form", "test_adamw_matches_torch_float64",
      "test_adamw_constant_gradient_closed_form"]),
    ("adamw_step_count_off_by_one",
     "    double bc1 = 1.0 - pow(beta1, (double)t);\n    double bc2 = 1.0 - pow(beta2, (double)t);\n"
     "    double step_size",
     "    double bc1 = 1.0 - pow(beta1, (double)(t + 1));\n"
     "    double bc2 = 1.0 - pow(beta2, (double)(t + 1));\n    double step_size",
     ["test_adamw_fresh_step_closed_form", "test_adamw_matches_torch_float64"]),
    ("adamw_ema_weights_swapped",
     "        p[i] = p[i] * (1.0 - lr * wd);\n        m[i] = beta1 * m[i] + (1.0 - beta1) * g[i];",
     "        p[i] = p[i] * (1.0 - lr * wd);\n        m[i] = (1.0 - beta1) * m[i] + beta1 * g[i];",
     ["test_adamw_fresh_step_closed_form", "test_adamw_matches_torch_float64"]),
    ("adamw_second_moment_of_g_not_g_squared",
     "v[i] = beta2 * v[i] + (1.0 - beta2) * g[i] * g[i];\n        double h = sqrt(v[i]) / bc2_sqrt",
     "v[i] = beta2 * v[i] + (1.0 - beta2) * fabs(g[i]);\n        double h = sqrt(v[i]) / bc2_sqrt",
     ["test_adamw_fresh_step_closed_form", "test_adamw_matches_torch_float64"]),
    # ---- AdEMAMix
    ("ademamix_slow_ema_bias_corrected",
     "p[i] = p[i] - lr * (m1[i] / bc1 + alpha * m2[i]) / h;",
     "p[i] = p[i] - lr * (m1[i] / bc1 + alpha * m2[i] / (1.0 - pow(beta3, (double)t))) / h;",
     ["test_ademamix_fresh_step_closed_form", "test_ademamix_constant_gradient_slow_ema"]),
    ("ademamix_slow_ema_uses_beta1",
     "m2[i] = beta3 * m2[i] + (1.0 - beta3) * g[i];",
     "m2[i] = beta1 * m2[i] + (1.0 - beta1) * g[i];",
     ["test_ademamix_fresh_step_closed_form", "test_ademamix_constant_gradient_slow_ema"]),
    ("ademamix_slow_term_outside_lr",
     "p[i] = p[i] - lr * (m1[i] / bc1 + alpha * m2[i]) / h;",
     "p[i] = p[i] - (lr * m1[i] / bc1 + alpha * m2[i]) / h;",
     ["test_ademamix_fresh_step_closed_form", "test_ademamix_constant_gradient_slow_ema"]),
    ("ademamix_decay_dropped",
     "        p[i] = p[i] * (1.0 - lr * wd);\n        m1[i]",
     "        m1[i]",
     ["test_ademamix_fresh_step_closed_form", "test_ademamix_alpha_zero_is_adamw"]),
    # ---- Adam-mini
    ("adam_mini_mean_over_tensor_not_block",
     "(s / (double)block)", "(s / (double)n)",
     ["test_adam_mini_fresh_step_closed_form", "test_adam_mini_constant_magnitude_rows_is_adamw"]),
    ("adam_mini_block_stride",
     "const double *gj = g + j * block;", "const double *gj = g + j;",
     ["test_adam_mini_fresh_step_closed_form", "test_adam_mini_constant_magnitude_rows_is_adamw"]),
    ("adam_mini_decay_dropped",
     "            p[i] = p[i] * (1.0 - lr * wd);\n", "",
     ["test_adam_mini_fresh_step_closed_form", "test_adam_mini_block_one_is_adamw"]),
    ("adam_mini_first_moment_not_bias_corrected",
     "p[i] = p[i] - lr * (m[i] / bc1) / h;", "p[i] = p[i] - lr * m[i] / h;",
     ["test_adam_mini_block_one_is_adamw", "test_adam_mini_constant_magnitude_rows_is_adamw"]),
    # ---- AMP skip and lr schedule
    ("nonfinite_misses_inf", "if (!isfinite(x[i]))", "if (isnan(x[i]))",
     ["test_nonfinite_detection"]),
    ("cosine_not_held_after_end", "    if (k > K)\n        k = K;\n", "",
     ["test_cosine_lr_closed_values"]),
    ("cosine_runs_backwards", "0.5 * (1.0 + cos(M_PI * x))", "0.5 * (1.0 - cos(M_PI * x))",
     ["test_cosine_lr_closed_values"]),
    ("cosine_half_period", "0.5 * (1.0 + cos(M_PI * x))", "0.5 * (1.0 + cos(0.5 * M_PI * x))",
     ["test_cosine_lr_closed_values"]),
    # ---- bf16 + remainder
    ("remainder_truncates",
     "int64_t res = ((x + 32768) % 65536) - 32768;", "int64_t res = x % 65536;",
     ["test_remainder_bf16_is_nearest_rounding"]),
    ("remainder_ties_toward_zero",
     "int64_t res = ((x + 32768) % 65536) - 32768;",
     "int64_t res = ((x + 32767) % 65536) - 32767;",
     ["test_remainder_bf16_is_nearest_rounding"]),
    ("remainder_reconstruct_drops_sign",
     "int64_t x = (int64_t)b[i] * 65536 + (int64_t)r[i];",
     "int64_t x = (int64_t)b[i] * 65536 + (int64_t)(uint16_t)r[i];",
     ["test_remainder_bf16_is_nearest_rounding"]),
    # ---- quantization map, threshold rule, packing
    ("map_fraction_offset",
     "(0.1 + 0.9 * (double)(k + 1) / (double)nk)", "(0.1 + 0.9 * (double)k / (double)nk)",
     ["test_dynamic_map_structure", "test_dynamic_map_hand_values"]),
    ("map_binary_not_decimal_exponent",
     "pow(10.0, -(double)e)", "pow(2.0, -(double)e)",
     ["test_dynamic_map_structure", "test_dynamic_map_hand_values"]),
    ("thresholds_at_lower_code",
     "T[j] = (float)(((double)M[j - 1] + (double)M[j]) / 2.0);",
     "T[j] = M[j - 1];",
     ["test_quantizer_threshold_rule_near_every_threshold"]),
    ("threshold_ties_to_smaller_code", "if (T[j] <= a)", "if (T[j] < a)",
     ["test_quantizer_threshold_rule_near_every_threshold"]),
    ("absmax_signed_max", "        if (fabsf(x[i]) > A)\n                A = fabsf(x[i]);",
     "        if (x[i] > A)\n                A = x[i];",
     ["test_absmax_element_roundtrips"]),
    ("dequantize_sign_bit_position", "(c >> b) & 1", "(c >> (b - 1)) & 1",
     ["test_absmax_element_roundtrips"]),
    ("nibble_order_swapped", "packed[i] = (uint8_t)(lo | (hi << 4));",
     "packed[i] = (uint8_t)(hi | (lo << 4));", ["test_nibble_packing_layout"]),
    # ---- blockwise AdEMAMix
    ("blockwise_ademamix_decay_after_update",
     "        p[i] = p[i] * (1.0 - lr * wd);\n        double h = sqrt(vi) / sqrt(bc2) + eps;\n"
     "        p[i] = p[i] - lr * (mi / bc1 + alpha * m2i) / h;",
     "        double h = sqrt(vi) / sqrt(bc2) + eps;\n"
     "        p[i] = (p[i] - lr * (mi / bc1 + alpha * m2i) / h) * (1.0 - lr * wd);",
     ["test_blockwise_ademamix_fresh_step"]),
    ("blockwise_ademamix_m2_with_beta1",
     "double m2i = F32(F32(b3 * (double)scratch_m2[i]) + F32(c3 * gi));",
     "double m2i = F32(F32(b1 * (double)scratch_m2[i]) + F32(c1 * gi));",
     ["test_blockwise_ademamix_fresh_step"]),
    ("blockwise_ademamix_m2_unsigned_map", "oracle_quantize(n, block, bm, 1, scratch_m2, Tm, qm2, am2);",
     "oracle_quantize(n, block, bv, 0, scratch_m2, Tv, qm2, am2);", ["test_blockwise_ademamix_fresh_step"]),
    ("blockwise_ademamix_m1_bias_uncorrected", "p[i] = p[i] - lr * (mi / bc1 + alpha * m2i) / h;",
     "p[i] = p[i] - lr * (mi + alpha * m2i) / h;",
     ["test_blockwise_ademamix_fresh_step", "test_blockwise_ademamix_alpha_zero_is_blockwise_adamw"]),
    # ---- Lion
    ("lion_decay_after_update", "        p[i] = p[i] * (1.0 - lr * wd);\n        p[i] = p[i] - lr * sg;",
     "        p[i] = p[i] - lr * sg;\n        p[i] = p[i] * (1.0 - lr * wd);",
     ["test_lion_constant_gradient_closed_form"]),
    ("lion_sign_of_gradient", "double sg = c > 0.0 ? 1.0 : (c < 0.0 ? -1.0 : 0.0);",
     "double sg = gi > 0.0 ? 1.0 : (gi < 0.0 ? -1.0 : 0.0);", ["test_lion_reversal_follows_the_interpolation"]),
    ("lion_interpolates_with_beta2", "double c = F32(F32(b1 * (double)m[i]) + F32(c1 * gi));",
     "double c = F32(F32(b2 * (double)m[i]) + F32(c2 * gi));", ["test_lion_reversal_follows_the_interpolation"]),
    ("lion_momentum_before_sign",
     "        double c = F32(F32(b1 * (double)m[i]) + F32(c1 * gi));\n",
     "        m[i] = (float)F32(F32(b2 * (double)m[i]) + F32(c2 * gi));\n"
     "        double c = F32(F32(b1 * (double)m[i]) + F32(c1 * gi));\n",
     ["test_lion_reversal_follows_the_interpolation"]),
    # ---- LAMB
    ("lamb_trust_without_sqrt", "double trust = (pn > 0.0 && un > 0.0) ? sqrt(pn) / sqrt(un) : 1.0;",
     "double trust = (pn > 0.0 && un > 0.0) ? pn / un : 1.0;", ["test_lamb_step_norm_is_lr_times_param_norm"]),
    ("lamb_trust_inverted", "double trust = (pn > 0.0 && un > 0.0) ? sqrt(pn) / sqrt(un) : 1.0;",
     "double trust = (pn > 0.0 && un > 0.0) ? sqrt(un) / sqrt(pn) : 1.0;",
     ["test_lamb_step_norm_is_lr_times_param_norm", "test_lamb_scale_equivariance"]),
    ("lamb_no_decay_term", "        u[i] = r + wd * p[i];", "        u[i] = r;",
     ["test_lamb_fresh_step_direction"]),
    ("lamb_uncorrected_moments", "double r = (m[i] / bc1) / (sqrt(v[i]) / sqrt(bc2) + eps);",
     "double r = m[i] / (sqrt(v[i]) + eps);", ["test_lamb_fresh_step_direction"]),
    # ---- low-precision model copy
    ("bf16_copy_ties_away", "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))", "if (lo >= 0x8000u)",
     ["test_model_copy_bf16_is_torch_rne"]),
    ("bf16_copy_truncates", "        hi += 1u; /* a carry into the exponent is the correct rounding */",
     "        hi += 0u;", ["test_model_copy_bf16_is_torch_rne"]),
    ("f16_copy_ties_up", "if (rem > half || (rem == half && (kept & 1u)))", "if (rem >= half)",
     ["test_model_copy_f16_is_numpy_rne"]),
    ("f16_copy_subnormal_shift", "shift = 14 - e; /* subnormal", "shift = 13 - e; /* subnormal",
     ["test_model_copy_f16_is_numpy_rne"]),
    ("f16_copy_exponent_bias", "int e = (int)ex - 127 + 15; /* fp16 biased exponent */",
     "int e = (int)ex - 127 + 14; /* fp16 biased exponent */", ["test_model_copy_f16_is_numpy_rne"]),
    # ---- scaled 16-bit moments
    ("scaled_state_not_unscaled", "double mt = F32(h16_to_double(qm[i], half) * (double)*sm);",
     "double mt = F32(h16_to_double(qm[i], half));", ["test_scaled_fp16_states_track_fp32_adamw"]),
    ("scaled_state_scale_without_range", "if (am > 0.0) nsm = (float)(am / 65504.0);",
     "if (am > 0.0) nsm = (float)am;", ["test_scaled_states_fresh_step"]),
    ("scaled_state_not_rescaled", "qm[i] = f32_to_16((float)((double)scratch_m[i] * (double)rm), half);",
     "qm[i] = f32_to_16(scratch_m[i], half);", ["test_scaled_states_fresh_step", "test_scaled_states_round_trip_precision"]),
    ("scaled_state_decay_after", "        p[i] = p[i] * (1.0 - lr * wd);\n        double h = sqrt(vi) / sqrt(bc2) + eps;\n"
     "        p[i] = p[i] - (lr / bc1) * mi / h;\n    }\n    float nsm",
     "        double h = sqrt(vi) / sqrt(bc2) + eps;\n"
     "        p[i] = (p[i] - (lr / bc1) * mi / h) * (1.0 - lr * wd);\n    }\n    float nsm",
     ["test_scaled_states_fresh_step"]),
    # ---- gradient clipping and loss scale
    ("sumsq_of_magnitudes", "        s += x[i] * x[i];\n    return s;", "        s += fabs(x[i]);\n    return s;",
     ["test_grad_norm_library_and_closed_form", "test_clip_matches_torch_clip_grad_norm"]),
    ("clip_not_clamped_to_one", "    return c < 1.0 ? c : 1.0;", "    return c;",
     ["test_clip_matches_torch_clip_grad_norm", "test_clip_coef_special_cases"]),
    ("clip_without_eps_guard", "double c = max_norm / (norm + 1e-6);", "double c = max_norm / norm;",
     ["test_clip_matches_torch_clip_grad_norm", "test_clip_coef_special_cases"]),
    ("scaler_keeps_count_on_overflow",
     "        *scale = (float)((double)*scale * backoff);\n        *tracker = 0;",
     "        *scale = (float)((double)*scale * backoff);",
     ["test_scaler_update_matches_torch", "test_scaler_update_closed_form"]),
    ("scaler_grows_one_step_late", "    if (k >= interval) {", "    if (k > interval) {",
     ["test_scaler_update_matches_torch", "test_scaler_update_closed_form"]),
    ("scaler_grows_to_infinity", "        if (isfinite(grown))\n            *scale = grown;",
     "        *scale = grown;", ["test_scaler_update_matches_torch"]),
    # ---- blockwise-quantized step
    ("blockwise_decay_after_update",
     "        p[i] = p[i] * (1.0 - lr * wd);\n        double h = sqrt(vi) / sqrt(bc2) + eps;\n"
     "        p[i] = p[i] - (lr / bc1) * mi / h;\n    }\n    oracle_quantize",
     "        double h = sqrt(vi) / sqrt(bc2) + eps;\n"
     "        p[i] = (p[i] - (lr / bc1) * mi / h) * (1.0 - lr * wd);\n    }\n    oracle_quantize",
     ["test_blockwise_fresh_step"]),
    ("blockwise_v_of_g_not_g_squared",
     "double vi = F32(F32(b2 * (double)scratch_v[i]) + F32(c2 * F32(gi * gi)));\n        scratch_m[i] = (float)mi;\n        scratch_v",
     "double vi = F32(F32(b2 * (double)scratch_v[i]) + F32(c2 * fabs(gi)));\n        scratch_m[i] = (float)mi;\n        scratch_v",
     ["test_blockwise_fresh_step"]),
    ("blockwise_m_with_unsigned_map", "oracle_quantize(n, block, bm, 1, scratch_m, Tm, qm, am);\n    oracle_quantize(n, block, bv",
     "oracle_quantize(n, block, bm, 0, scratch_m, Tm, qm, am);\n    oracle_quantize(n, block, bv",
     ["test_blockwise_fresh_step"]),
    ("blockwise_beta_weights_swapped",
     "oracle_thresholds(1 << bv, Mv, Tv);\n\n    double b1 = F32(beta1), c1 = F32(1.0 - beta1);\n    double b2 = F32(beta2), c2 = F32(1.0 - beta2);\n    double bc1",
     "oracle_thresholds(1 << bv, Mv, Tv);\n\n    double c1 = F32(beta1), b1 = F32(1.0 - beta1);\n    double b2 = F32(beta2), c2 = F32(1.0 - beta2);\n    double bc1",
     ["test_blockwise_fresh_step"]),
    # invisible on a fresh step (zero states): only the multi-step pins see them
    ("blockwise_v_dequantized_with_m_absmax",
     "    oracle_dequantize(n, block, bv, 0, qv, Mv, av, scratch_v);\n    for (int64_t i = 0; i < n; ++i) {\n"
     "        double gi = (double)g[i];\n        double mi = F32(F32(b1 * (double)scratch_m[i]) + F32(c1 * gi));\n"
     "        double vi",
     "    oracle_dequantize(n, block, bv, 0, qv, Mv, am, scratch_v);\n    for (int64_t i = 0; i < n; ++i) {\n"
     "        double gi = (double)g[i];\n        double mi = F32(F32(b1 * (double)scratch_m[i]) + F32(c1 * gi));\n"
     "        double vi",
     ["test_blockwise_constant_magnitude_blocks_track_adamw"]),
    ("blockwise_ademamix_m2_dequantized_with_m1_absmax",
     "oracle_dequantize(n, block, bm, 1, qm2, Mm, am2, scratch_m2);",
     "oracle_dequantize(n, block, bm, 1, qm2, Mm, am, scratch_m2);",
     ["test_blockwise_ademamix_constant_magnitude_blocks_track_ademamix"]),
]


def _cases(fn):
    """Expand a pin's parametrize marks into keyword dicts."""
    cases = [{}]
    for mark in getattr(fn, "pytestmark", []):
        if mark.name != "parametrize":
            continue
        names = mark.args[0]
        names = [s.strip() for s in names.split(",")] if isinstance(names, str) else list(names)
        expanded = []
        for c in cases:
            for v in mark.args[1]:
                v = tuple(v) if len(names) > 1 else (v,)
                expanded.append({**c, **dict(zip(names, v))})
        cases = expanded
    return cases


def _failing_cases(pin_name):
    """Run every parametrization of a pin against the active oracle build;
    return how many of them fail."""
    fn = getattr(pins, pin_name)
    bad = 0
    for kw in _cases(fn):
        try:
            fn(oracle, **kw)
        except Exception:  # a failed assertion, or NaN/inf tripping numpy
            bad += 1
    return bad


def _source():
    with open(SRC) as f:
        return f.read()


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def test_mutant_table_is_well_formed():
    src = _source()
    names = [m[0] for m in MUTANTS]
    assert len(set(names)) == len(names)
    for name, old, new, witnesses in MUTANTS:
        assert src.count(old) == 1, name
        assert old != new and witnesses, name
        for w in witnesses:
            assert callable(getattr(pins, w)), (name, w)


def test_control_build_passes_every_witness(builds):
    path = str(builds / "control.so")
    oracle.compile_source(_source(), path)
    witnesses = sorted({w for m in MUTANTS for w in m[3]})
    with oracle.use_build(path):
        failing = [w for w in witnesses if _failing_cases(w)]
    assert not failing


@pytest.mark.parametrize("name,old,new,witnesses", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(builds, name, old, new, witnesses):
    src = _source()
    path = str(builds / f"{name}.so")
    oracle.compile_source(src.replace(old, new), path)
    with oracle.use_build(path):
        survived = [w for w in witnesses if _failing_cases(w) == 0]
    assert not survived, f"{name} passes {survived}"
