"""Planted-mistake check of the oracle's pins (CPU only).

Each mutant below copies the oracle's C source, plants one plausible mistake
(a dropped term, a wrong sign or index, a swapped order, a different rounding
rule), compiles it to a temporary library and runs the pin battery of
test_oracle.py against it.  Every mutant must make at least one pin fail;
the unmodified source must pass them all."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import tests.test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kvq_oracle.c")

# context that tells the Hadamard rotation's input line from the SRFT's
_H = ";\n    double norm = 1.0 / sqrt((double)D);\n    for (int i = 0; i < D; i++) {"
_F = ";\n    double norm = 1.0 / sqrt((double)D);\n    for (int k = 0; k <= D / 2; k++) {"

MUTANTS = {
    "lambda_divides_on_quantize": ("(double)s[j] * (double)lam[j] * kvqo_f16_to_f64(x[j])" + _H,
                                   "(double)s[j] / (double)lam[j] * kvqo_f16_to_f64(x[j])" + _H),
    "signs_dropped": ("(double)s[j] * (double)lam[j] * kvqo_f16_to_f64(x[j])" + _H,
                      "(double)lam[j] * kvqo_f16_to_f64(x[j])" + _H),
    "srft_lambda_divides": ("(double)s[j] * (double)lam[j] * kvqo_f16_to_f64(x[j])" + _F,
                            "(double)s[j] / (double)lam[j] * kvqo_f16_to_f64(x[j])" + _F),
    "no_normalisation": ("y[i] = acc * norm;", "y[i] = acc;"),
    "hadamard_sign_flipped": ("& 1) ? -1 : 1;", "& 1) ? 1 : -1;"),
    "hadamard_or_index": ("popcount((unsigned)(i & j))", "popcount((unsigned)(i | j))"),
    "unstored_scale": ("double sbar = kvqo_f16_to_f64(sc);\n            for (int i = g * G; i < (g + 1) * G; i++) q[i]",
                       "double sbar = amax / 7.0;\n            for (int i = g * G; i < (g + 1) * G; i++) q[i]"),
    "amax_over_8": ("kvqo_f64_to_f16(amax / 7.0)", "kvqo_f64_to_f16(amax / 8.0)"),
    "round_half_away": ("double r = nearbyint(y / scale);\n    if (r > 7.0)", "double r = round(y / scale);\n    if (r > 7.0)"),
    "truncate_codes": ("double r = nearbyint(y / scale);\n    if (r > 7.0)", "double r = trunc(y / scale);\n    if (r > 7.0)"),
    "nibble_order_swapped": ("bytes[k] = (uint8_t)(((unsigned)q[2 * k] & 0xfu) |\n"
                             "                             (((unsigned)q[2 * k + 1] & 0xfu) << 4));",
                             "bytes[k] = (uint8_t)(((unsigned)q[2 * k + 1] & 0xfu) |\n"
                             "                             (((unsigned)q[2 * k] & 0xfu) << 4));"),
    "group_index_interleaved": ("code_of(y[r * D + i],\n                                           kvqo_f16_to_f64(scales[r * ng + i / G]));",
                                "code_of(y[r * D + i],\n                                           kvqo_f16_to_f64(scales[r * ng + i % ng]));"),
    "dequant_group_interleaved": ("(double)q[i] * kvqo_f16_to_f64(scales[r * ng + i / G]);",
                                  "(double)q[i] * kvqo_f16_to_f64(scales[r * ng + i % ng]);"),
    "unscale_multiplies": ("* yhat[i];\n        xhat[j] = ((double)s[j] / (double)lam[j]) * (acc * norm)",
                           "* yhat[i];\n        xhat[j] = ((double)s[j] * (double)lam[j]) * (acc * norm)"),
    "isrft_unscale_multiplies": ("}\n        xhat[j] = ((double)s[j] / (double)lam[j]) * (acc * norm)",
                                 "}\n        xhat[j] = ((double)s[j] * (double)lam[j]) * (acc * norm)"),
    "vq_ties_to_highest": ("if (d < bd) { bd = d; best = k; }", "if (d <= bd) { bd = d; best = k; }"),
    "vq_abs_distance": ("d += diff * diff;", "d += fabs(diff);"),
    "f16_truncates": ("double n = nearbyint((2.0 * m - 1.0) * 1024.0);",
                      "double n = floor((2.0 * m - 1.0) * 1024.0);"),
    "f16_subnormal_truncates": ("double n = nearbyint(ldexp(a, 24));", "double n = floor(ldexp(a, 24));"),
    "int8_amax_over_128": ("kvqo_f64_to_f16(amax / 127.0)", "kvqo_f64_to_f16(amax / 128.0)"),
    "int8_clamp_128": ("if (r > 127.0) r = 127.0;", "if (r > 128.0) r = 128.0;"),
    "int8_truncates": ("double r = nearbyint(y / scale);\n    if (r > 127.0)", "double r = trunc(y / scale);\n    if (r > 127.0)"),
    "mx_ties_to_odd": ("(a - lo == hi - a && (mag & 1))", "(a - lo == hi - a && !(mag & 1))"),
    "mx_exponent_off_by_one": ("int e = (E - 1) - 2;", "int e = (E - 1) - 1;"),
    "mx_subnormal_quarter": ("double mag = e == 0 ? 0.5 * m", "double mag = e == 0 ? 0.25 * m"),
    "mx_scale_multiplies": ("q[i] = (int8_t)e2m1_code(ldexp(y[i], -e));", "q[i] = (int8_t)e2m1_code(ldexp(y[i], e));"),
    "kmeans_divides_by_count_plus_one": ("mean64[e] /= (double)counts[k];", "mean64[e] /= (double)(counts[k] + 1);"),
    "kmeans_empty_cluster_to_zero": ("mean64[e] = kvqo_f16_to_f64(cb_old[e]);\n                cb_new[e] = cb_old[e];",
                                     "mean64[e] = 0.0;\n                cb_new[e] = 0;"),
    "kmeans_drops_first_sample": ("for (int64_t i = 0; i < n; i++) {\n        int k = idx[i];",
                                  "for (int64_t i = 1; i < n; i++) {\n        int k = idx[i];"),
    "kmeans_coordinate_shifted": ("mean64[(int64_t)k * sub + t] += ysub[i * sub + t];",
                                  "mean64[(int64_t)k * sub + t] += ysub[i * sub + (t + 1) % sub];"),
    "srft_imag_sign_flipped": ("            im -= v[j] * sn[t];", "            im += v[j] * sn[t];"),
    "srft_sqrt2_dropped": ("else { y[2 * k] = sqrt(2.0) * re; y[2 * k + 1] = sqrt(2.0) * im; }",
                           "else { y[2 * k] = re; y[2 * k + 1] = im; }"),
    "srft_re_im_swapped": ("else { y[2 * k] = sqrt(2.0) * re; y[2 * k + 1] = sqrt(2.0) * im; }",
                           "else { y[2 * k] = sqrt(2.0) * im; y[2 * k + 1] = sqrt(2.0) * re; }"),
    "srft_nyquist_dropped": ("else if (k == D / 2) y[1] = re;", "else if (k == D / 2) y[1] = 0.0;"),
    "isrft_alternating_sign": ("double acc = yhat[0] + ((j & 1) ? -yhat[1] : yhat[1]);",
                               "double acc = yhat[0] + yhat[1];"),
    "isrft_sine_sign": ("acc += sqrt(2.0) * (yhat[2 * k] * c[t] - yhat[2 * k + 1] * sn[t]);",
                        "acc += sqrt(2.0) * (yhat[2 * k] * c[t] + yhat[2 * k + 1] * sn[t]);"),
    "attend_no_max_shift": ("double w = exp(a[t] - amax);", "double w = exp(a[t]);"),
    "attend_scale_dropped": ("a[t] = scale * dot;", "a[t] = dot;"),
    "attend_values_from_keys": ("o[c] += w * vh[(int64_t)t * D + c];", "o[c] += w * kh[(int64_t)t * D + c];"),
    "attend_query_head_interleaved": ("int j = h * R + r;", "int j = r * H + h;"),
    "attend_one_token_short": ("for (int t = 0; t < n; t++) {\n                    double w",
                               "for (int t = 0; t + 1 < n; t++) {\n                    double w"),
}

# every pin of test_oracle.py that takes no fixture other than golden_dir
BATTERY = [
    ("test_f16_encode_matches_numpy_rne", {}),
    ("test_f16_encode_midpoints_go_to_even", {}),
    ("test_hadamard_matches_scipy_sylvester", {"D": 16}),
    ("test_rotate_matches_dense_scipy_product", {"D": 128}),
    ("test_lambda_multiplies_before_rotation", {}),
    ("test_signs_apply_before_rotation", {}),
    ("test_parseval_and_roundtrip", {"D": 128}),
    ("test_unrotate_closed_form", {}),
    ("test_nibbles_golden", {"golden_dir": None}),
    ("test_worked_examples", {"golden_dir": None}),
    ("test_case_single_spike", {"D": 128}),
    ("test_case_all_ones_energy_in_group0", {}),
    ("test_ties_round_half_to_even", {}),
    ("test_codes_given_scales_matches_quantizer", {"D": 128, "G": 32}),
    ("test_quantizer_invariants", {"D": 128, "G": 32}),
    ("test_dequant_single_code_closed_form", {}),
    ("test_roundtrip_error_bound", {"D": 128, "G": 32}),
    ("test_vq_encode_bruteforce", {"sub": 4, "K": 16}),
    ("test_vq_duplicate_centroids_lowest_index_and_exact_hits", {}),
    ("test_vq_decode_closed_form_and_roundtrip", {}),
    ("test_int8_single_spike", {"D": 128}),
    ("test_int8_ties_round_half_to_even_and_clamp", {}),
    ("test_int8_quantizer_invariants", {"D": 128, "G": 32}),
    ("test_int8_dequant_single_code_closed_form", {}),
    ("test_e2m1_table_golden", {"golden_dir": None}),
    ("test_e2m1_rounding_ties_even_and_saturation", {"golden_dir": None}),
    ("test_mxfp4_block_scale_rule_and_invariants", {"D": 128, "golden_dir": None}),
    ("test_mxfp4_zero_block_and_single_spike", {"golden_dir": None}),
    ("test_srft_matches_numpy_fft", {"D": 96}),
    ("test_srft_orthonormal_parseval_and_roundtrip", {"D": 96}),
    ("test_srft_closed_forms", {}),
    ("test_srft_quantizer_invariants_and_roundtrip", {"D": 128, "G": 32}),
    ("test_srft_dequant_single_code_closed_form", {}),
    ("test_kmeans_step_matches_scipy_lloyd_iteration", {}),
    ("test_kmeans_update_closed_form_clusters", {}),
    ("test_kmeans_update_is_the_sse_minimiser_and_lloyd_descends", {}),
    ("test_attend_single_token_returns_its_value", {}),
    ("test_attend_zero_query_is_mean_of_values", {}),
    ("test_attend_matches_torch_sdpa", {"R": 4, "D": 128, "G": 32}),
    ("test_attend_large_scores_stay_finite", {}),
    ("test_attend_empty_context_gives_zeros", {}),
]


def run_battery(lib, golden_dir):
    """Run the battery with `lib` bound into the oracle module; return the
    names of the pins that failed."""
    failed = []
    saved = oracle._lib
    oracle._lib = lib
    try:
        for name, kw in BATTERY:
            kw = {k: (golden_dir if k == "golden_dir" else v) for k, v in kw.items()}
            try:
                getattr(pins, name)(**kw)
            except (AssertionError, ValueError):
                failed.append(name)
    finally:
        oracle._lib = saved
    return failed


def compile_variant(src_text, tmpdir, tag):
    c = os.path.join(tmpdir, tag + ".c")
    so = os.path.join(tmpdir, tag + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", so, c, "-lm"], check=True)
    return oracle.bind(so)


@pytest.fixture(scope="module")
def src():
    with open(SRC) as f:
        return f.read()


def test_unmodified_source_passes_battery(src, golden_dir, tmp_path):
    lib = compile_variant(src, str(tmp_path), "orig")
    assert run_battery(lib, golden_dir) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src, golden_dir, tmp_path):
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation site not found uniquely: %s" % name
    lib = compile_variant(src.replace(old, new), str(tmp_path), name)
    np.random.seed(0)
    failed = run_battery(lib, golden_dir)
    assert failed, "planted mistake %r passed every pin" % name
