"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU, in a
temporary directory), builds it, swaps it in, and runs the pin tests: at least one
pin must fail.  The committed oracle itself is never modified.
"""
import os

import pytest

import oracle
import tests.test_oracle_cache as tc
import tests.test_oracle_codec as tq
import tests.test_oracle_keys as tk
import tests.test_oracle_logquant as tl
import tests.test_oracle_outliers as to

SRC = os.path.join(os.path.dirname(oracle.__file__), "kvq_oracle.c")

MUTANTS = {
    # rounding half away from zero instead of half to even
    "half_away": ("float r = rintf(xi / s);", "float r = roundf(xi / s);"),
    # the zero point added before rounding (the other operation order)
    "add_before_round": ("float r = rintf(xi / s);\n        float t = r + z;",
                         "float t = rintf(xi / s + z);"),
    # missing upper clamp
    "no_upper_clamp": ("if (t > qmax) t = qmax;", ""),
    # signed code range [-2^(n-1), 2^(n-1)-1]
    "signed_clamp": ("if (t > qmax) t = qmax;",
                     "if (t > (float)((1 << (bits - 1)) - 1)) t = (float)((1 << (bits - 1)) - 1);"),
    # 2^n levels in the scale instead of 2^n - 1
    "scale_2n": ("float s = range / qmax;", "float s = range / (qmax + 1.0f);"),
    # no degenerate-group rule (division by a zero scale)
    "no_degenerate_rule": ("if (mx == mn || s == 0.0f) {", "if (0) {"),
    # a zero point of -0 kept as is
    "keep_negative_zero": ("if (z == 0.0f) z = 0.0f;", ""),
    # dequantization in the expanded order q*s - z*s
    "dequant_expanded": ("float d = (float)q - z;\n    return d * s;",
                         "return (float)q * s - z * s;"),
    # flush before storing the token (residual may hold R tokens between calls)
    "flush_before_append": (
        "    memcpy(c->res_k + c->r * D, k, sizeof(float) * D);\n"
        "    memcpy(c->res_v + c->r * D, v, sizeof(float) * D);\n"
        "    c->r += 1;\n"
        "    if (c->r == c->R) {\n"
        "        if (c->W > 0) flush_log(c);\n"
        "        else flush_residual(c);\n"
        "    }",
        "    if (c->r == c->R) {\n"
        "        if (c->W > 0) flush_log(c);\n"
        "        else flush_residual(c);\n"
        "    }\n"
        "    memcpy(c->res_k + c->r * D, k, sizeof(float) * D);\n"
        "    memcpy(c->res_v + c->r * D, v, sizeof(float) * D);\n"
        "    c->r += 1;"),
    # keys grouped along channels of a token instead of along tokens of a channel
    "key_groups_transposed": ("orc_quant_group_skip(col, G, D, c->bits,",
                              "orc_quant_group_skip(col, G, 1, c->bits,"),
    # softmax scale dropped
    "no_softmax_scale": ("sc[j] = dot * scale;", "sc[j] = dot;"),
    # the last token of the cache is left out of the softmax denominator
    "drop_last_token": ("    for (int64_t j = 0; j < T; ++j) {\n        double w = exp(sc[j] - M);",
                        "    for (int64_t j = 0; j < T - 1; ++j) {\n        double w = exp(sc[j] - M);"),
    # symmetric scale without the factor 2 (max|x| / (2^n - 1))
    "sym_no_factor_2": ("const float twice = 2.0f * amax;", "const float twice = amax;"),
    # symmetric zero point one level low
    "sym_zero_off_by_one": ("const float zz = (float)(1 << (bits - 1));",
                            "const float zz = (float)((1 << (bits - 1)) - 1);"),
    # symmetric upper clamp at 2^(n-1) (one code too many)
    "sym_upper_clamp": ("if (r > zz - 1.0f) r = zz - 1.0f;", "if (r > zz) r = zz;"),
    # symmetric rounding half away from zero
    "sym_half_away": ("float r = rintf(x[i * stride] / ss);", "float r = roundf(x[i * stride] / ss);"),
    # log-sparse retention: the later token of each pair quantized, the earlier kept
    "log_keep_earlier": (
        "        memcpy(bk + (size_t)i * D, c->res_k + (size_t)(2 * i) * D, sizeof(float) * D);\n"
        "        memcpy(bv + (size_t)i * D, c->res_v + (size_t)(2 * i) * D, sizeof(float) * D);\n"
        "        memcpy(keep_k + (size_t)i * D, c->res_k + (size_t)(2 * i + 1) * D, sizeof(float) * D);\n"
        "        memcpy(keep_v + (size_t)i * D, c->res_v + (size_t)(2 * i + 1) * D, sizeof(float) * D);",
        "        memcpy(bk + (size_t)i * D, c->res_k + (size_t)(2 * i + 1) * D, sizeof(float) * D);\n"
        "        memcpy(bv + (size_t)i * D, c->res_v + (size_t)(2 * i + 1) * D, sizeof(float) * D);\n"
        "        memcpy(keep_k + (size_t)i * D, c->res_k + (size_t)(2 * i) * D, sizeof(float) * D);\n"
        "        memcpy(keep_v + (size_t)i * D, c->res_v + (size_t)(2 * i) * D, sizeof(float) * D);"),
    # log-sparse retention: the newest keys taken from the wrong window
    "log_newest_from_middle": (
        "memcpy(keep_k + (size_t)W * D, c->res_k + (size_t)2 * W * D, sizeof(float) * (size_t)W * D);",
        "memcpy(keep_k + (size_t)W * D, c->res_k + (size_t)W * D, sizeof(float) * (size_t)W * D);"),
    # log-sparse retention: only W tokens kept after a flush
    "log_keep_w": ("    c->r = 2 * W;", "    c->r = W;"),
    # log-sparse retention: the oldest W quantized as one run (a sliding window, no thinning)
    "log_no_thinning": (
        "        memcpy(bk + (size_t)i * D, c->res_k + (size_t)(2 * i) * D, sizeof(float) * D);\n"
        "        memcpy(bv + (size_t)i * D, c->res_v + (size_t)(2 * i) * D, sizeof(float) * D);\n"
        "        memcpy(keep_k + (size_t)i * D, c->res_k + (size_t)(2 * i + 1) * D, sizeof(float) * D);\n"
        "        memcpy(keep_v + (size_t)i * D, c->res_v + (size_t)(2 * i + 1) * D, sizeof(float) * D);",
        "        memcpy(bk + (size_t)i * D, c->res_k + (size_t)i * D, sizeof(float) * D);\n"
        "        memcpy(bv + (size_t)i * D, c->res_v + (size_t)i * D, sizeof(float) * D);\n"
        "        memcpy(keep_k + (size_t)i * D, c->res_k + (size_t)(W + i) * D, sizeof(float) * D);\n"
        "        memcpy(keep_v + (size_t)i * D, c->res_v + (size_t)(W + i) * D, sizeof(float) * D);"),
    # dense-and-sparse: the outlier chosen by value instead of magnitude
    "outlier_by_value": ("if (fabsf(x[i * stride]) > fabsf(x[best * stride])) best = i;",
                         "if (x[i * stride] > x[best * stride]) best = i;"),
    # dense-and-sparse: the last of equal magnitudes
    "outlier_tie_last": ("if (fabsf(x[i * stride]) > fabsf(x[best * stride])) best = i;",
                         "if (fabsf(x[i * stride]) >= fabsf(x[best * stride])) best = i;"),
    # dense-and-sparse: the outlier kept in the range
    "outlier_in_range": ("        if (i == skip) continue;\n", ""),
    # dense-and-sparse: key outliers dequantized from their codes
    "outlier_key_dequant_dense": (
        "if (outliers && ko_idx[grp * D + ch] == t % G) k_out[(nS + t) * D + ch] = ko_val[grp * D + ch];", ""),
    # dense-and-sparse: value outlier channel taken from the vector's start
    "outlier_value_channel": ("vo_idx[t * nvg + h] == ch - h * GV", "vo_idx[t * nvg + h] == ch"),
    # head-granular keys: the token block read column by column (a transposed row)
    "key_token_transposed": ("orc_quant_group(bk + (int64_t)t * D, D, 1, c->bits, c->codec,",
                             "orc_quant_group(bk + (int64_t)t, D, m, c->bits, c->codec,"),
    # head-granular keys: every token dequantized with the first token of its key group's scale
    "key_token_scale_of_group": ("key_axis == ORC_KEY_PER_TOKEN ? t : grp * D + ch",
                                 "key_axis == ORC_KEY_PER_TOKEN ? grp * G : grp * D + ch"),
    # residual tokens left out of the dequantized token sequence
    "drop_residual": ("memcpy(k_out + (nS + Lq) * D, res_k, sizeof(float) * r * D);",
                      "memset(k_out + (nS + Lq) * D, 0, sizeof(float) * r * D);"),
}


def _pins():
    """Every pin test, bound to its parameters."""
    pins = []
    for case in tq._cases():
        pins.append(lambda c=case: tq.test_golden_example(c))
    for bits in (2, 4, 8):
        pins.append(lambda b=bits: tq.test_invariants_random_groups(b))
        pins.append(lambda b=bits: tq.test_symmetric_invariants_random_groups(b))
        pins.append(lambda b=bits: tq.test_exact_grid_reconstruction(b))
    pins.append(tq.test_signed_zero_inputs)
    pins.append(tq.test_underflowing_scale_uses_degenerate_rule)
    for args in [(0, 8, 4, 29), (3, 8, 2, 40), (5, 16, 4, 100)]:
        pins.append(lambda a=args: tc.test_counts_closed_form(*a))
    pins += [tc.test_flush_exactly_at_R, tc.test_grouping_axes_by_direct_regrouping,
             tc.test_workload_schedules_flush_where_expected,
             tc.test_attention_closed_form_equal_keys_and_zero_query,
             tc.test_attention_single_token, tc.test_attention_matches_torch_sdpa_float64,
             tc.test_unquantized_cache_is_plain_attention]
    for case in tl._cases():
        pins.append(lambda c=case: tl.test_golden_worked_example(c))
    for args in [(2, 4, 2, 13), (3, 8, 4, 100)]:
        pins.append(lambda a=args: tl.test_counts_closed_form(*a))
    for W in (2, 3):
        pins.append(lambda w=W: tl.test_every_token_once_newest_kept_and_log_sparse_gaps(w))
    pins.append(lambda: tl.test_matches_brute(2, 0, 0, 4, 2, 8, 37))
    pins.append(tl.test_before_first_flush_is_plain_attention)
    for case in to._cases():
        pins.append(lambda c=case: to.test_golden_example(c))
    for bits in (2, 4):
        pins.append(lambda b=bits: to.test_invariants_random_groups(b, 0))
    pins.append(lambda: to.test_slice_outliers_exact_and_matches_brute(4, 0, 0, 4, 8, 8, 37, 0))
    pins.append(lambda: to.test_slice_outliers_exact_and_matches_brute(2, 1, 2, 8, 4, 16, 50, 0))
    for case in tk._cases():
        pins.append(lambda c=case: tk.test_golden_cache(c))
    pins.append(lambda: tk.test_invariants_random_slices(4, 0))
    pins.append(lambda: tk.test_matches_brute(2, 0, 2, 0, 8, 4, 45, 1))
    return pins


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, "mutation anchor not found: " + name
    mutated = src.replace(old, new, 1)
    assert mutated != src
    p = tmp_path / ("mut_%s.c" % name)
    p.write_text(mutated)
    so = oracle.compile_source(str(p), str(tmp_path / ("mut_%s.so" % name)))
    saved = oracle._lib
    oracle._lib = oracle.load(so)
    failed = 0
    try:
        for pin in _pins():
            try:
                pin()
            except Exception:
                failed += 1
    finally:
        oracle._lib = saved
    assert failed > 0, "no pin caught mutant " + name
