"""The pins catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle.c (on the CPU), builds it with the
oracle's flags, points the oracle module at it, and runs the pin tests: at least one pin
must fail.  The planted copies live in a temporary directory and are never used elsewhere.
"""
import pytest

import oracle
from tests import test_oracle_ef as T_ef
from tests import test_oracle_quant as T_q
from tests import test_oracle_ratio as T_r
from tests import test_oracle_select as T_s
from tests import test_oracle_sign as T_g
from tests import test_oracle_qsgd as T_q8
from tests import test_oracle_threshold as T_t
from tests import test_oracle_randk as T_rk
from tests import test_oracle_gathered as T_ga
from tests import test_oracle_clip as T_cl

MUTANTS = {
    "tie_rule_higher_index_wins": ("return a->pos < b->pos ? -1 : 1;",
                                   "return a->pos > b->pos ? -1 : 1;"),
    "signed_key_order": ("return bits_of(x) & 0x7FFFFFFFu;", "return bits_of(x) ^ 0x80000000u;"),
    "fused_momentum": ("float mu = m * u[i];\n            u[i] = mu + x;",
                       "u[i] = fmaf(m, u[i], x);"),
    "dropped_residual_term": ("e[i] = e[i] + x;\n    }\n\n    /* step 3",
                              "e[i] = x;\n    }\n\n    /* step 3"),
    "sign_dropped_residual_term": ("e[i] = e[i] + x;\n    }\n    double s",
                                   "e[i] = x;\n    }\n    double s"),
    "negative_zero_residual": ("e[sel[j]] = 0.0f;", "e[sel[j]] = -0.0f;"),
    "output_in_rank_order": ("qsort(sel, (size_t)k, sizeof *sel, by_pos);", ""),
    "off_by_one_selection": ("for (int64_t j = 0; j < k; ++j) sel[j] = rec[j].pos;",
                             "for (int64_t j = 0; j < k; ++j) sel[j] = rec[j + (j + 1 < n)].pos;"),
    "philox_no_key_bump": ("k0 += weyl0;", ""),
    "philox_swapped_words": ("uint32_t n1 = lo1;", "uint32_t n1 = lo0;"),
    "sr_round_to_nearest": ("q = (int)f + (((float)u24 < frac * 16777216.0f) ? 1 : 0);",
                            "q = (int)f + (frac >= 0.5f ? 1 : 0);"),
    "scale_over_128": ("float scale = absmax / 127.0f;", "float scale = absmax / 128.0f;"),
    "quant_error_not_fed_back": ("e_seg[idx[j]] = v - deq;", "e_seg[idx[j]] = v;"),
    "k_floor_not_ceil": ("__int128 num = (__int128)n * ppb + 999999999;",
                         "__int128 num = (__int128)n * ppb;"),
    "decompress_ignores_scale": ("(float)codes[out + j] * scales[s]", "(float)codes[out + j]"),
    "sign_scale_not_mean": ("float scale = n > 0 ? (float)(s / (double)n) : 0.0f;",
                            "float scale = n > 0 ? (float)s : 0.0f;"),
    "sign_negative_zero_sends_minus": ("int neg = e[i] < 0.0f;", "int neg = signbit(e[i]) != 0;"),
    "sign_residual_added": ("e[i] = e[i] - q;", "e[i] = e[i] + q;"),
    "sign_bits_msb_first": ("if (neg) bits[i / 32] |= 1u << (i % 32);",
                            "if (neg) bits[i / 32] |= 1u << (31 - i % 32);"),
    "qsgd_step_without_levels": ("float qstep = norm / (float)s;\n    *norm_out",
                                 "float qstep = norm;\n    *norm_out"),
    "qsgd_norm_without_sqrt": ("float norm = (float)sqrt(sq);", "float norm = (float)sq;"),
    "qsgd_round_to_nearest": ("q = (int)l + (((float)qsgd_draw24(seed, step, seg_base + i) < frac * 16777216.0f) ? 1 : 0);",
                              "q = (int)l + (frac >= 0.5f ? 1 : 0);"),
    "qsgd_residual_not_fed_back": ("            e[i] = v - deq;\n        }\n    }\n    free(acc);",
                                   "            e[i] = v;\n        }\n    }\n    free(acc);"),
    "threshold_strict": ("if (magnitude_key(acc_copy[i]) >= magnitude_key(tau)) ++c;",
                         "if (magnitude_key(acc_copy[i]) > magnitude_key(tau)) ++c;"),
    "threshold_ignored": ("int64_t k = c < k_cap ? c : k_cap;", "int64_t k = k_cap;"),
    "randk_word0_only": ("return r[(uint64_t)gidx & 3u] >> 1;", "return r[0] >> 1;"),
    "randk_scale_k_over_n": ("(float)((double)n / (double)k)", "(float)((double)k / (double)n)"),
    "randk_smallest_keys": ("sel[j] = rec[j].pos;\n    free(rec);\n    qsort(sel, (size_t)k, sizeof *sel, by_pos);\n    float scale",
                            "sel[j] = rec[n - 1 - j].pos;\n    free(rec);\n    qsort(sel, (size_t)k, sizeof *sel, by_pos);\n    float scale"),
    "randk_residual_not_kept": ("for (int64_t i = 0; i < n; ++i) e[i] = acc[i];", ""),
    "randk_same_mask_every_step": ("(uint32_t)step, 0x53u", "0u, 0x53u"),
    "clip_without_sqrt": ("float norm = (float)sqrt(sq);\n    *norm_out = norm;\n    if (norm > c)",
                          "float norm = (float)sq;\n    *norm_out = norm;\n    if (norm > c)"),
    "clip_inverted_factor": ("float f = c / norm;", "float f = norm / c;"),
    "gathered_reverse_worker_order": ("for (int32_t w = 0; w < n_workers; ++w)",
                                      "for (int32_t w = n_workers - 1; w >= 0; --w)"),
    "gathered_overwrite": ("scales ? scales + (int64_t)w * n_seg : NULL, idx + (int64_t)w * kk,\n                       dense, 1);",
                           "scales ? scales + (int64_t)w * n_seg : NULL, idx + (int64_t)w * kk,\n                       dense, 0);"),
}


def _pins(orc):
    yield lambda: T_s.test_hand_examples(orc)
    yield lambda: [T_s.test_brute_force_tiny(orc, s) for s in range(12)]
    yield lambda: T_s.test_numpy_lexsort(orc, 1, 5000, 37)
    yield lambda: T_s.test_signed_zero_and_inf_order(orc)
    yield lambda: T_ef.test_ef_add_is_ieee_fp32(orc)
    yield lambda: T_ef.test_momentum_is_two_roundings(orc)
    yield lambda: T_ef.test_split_is_exact(orc, 57)
    yield lambda: T_q.test_philox_known_answers(orc)
    yield lambda: T_q.test_sr_toy_from_pages(orc)
    yield lambda: T_q.test_int8_closed_forms(orc)
    yield lambda: T_q.test_int8_zero_segment_and_error_feedback(orc)
    yield lambda: T_q.test_decompress_reconstructs(orc, False)
    yield lambda: T_r.test_k_from_ratio(orc)
    yield lambda: T_g.test_hand_cases(orc)
    yield lambda: T_g.test_scale_bits_residual(orc, 1000)
    yield lambda: T_g.test_conservation_and_ratio(orc)
    yield lambda: T_q8.test_hand_integer_levels(orc)
    yield lambda: T_q8.test_unbiased_and_toy(orc)
    yield lambda: T_q8.test_norm_codes_and_error_feedback(orc)
    yield lambda: [T_t.test_brute_force(orc, s) for s in range(4)]
    yield lambda: T_t.test_edges(orc)
    yield lambda: T_rk.test_exact_k_and_conservation(orc, 1000, 37)
    yield lambda: T_rk.test_marginal_and_pairwise_uniform(orc)
    yield lambda: T_rk.test_unbiased_without_error_feedback(orc)
    yield lambda: T_rk.test_mask_depends_on_step_and_segment_not_values(orc)
    yield lambda: T_rk.test_counter_mapping(orc, 3)
    yield lambda: T_ga.test_worker_order_is_the_summation_order(orc)
    yield lambda: T_ga.test_numpy_worker_by_worker(orc)
    yield lambda: T_cl.test_three_four_five(orc)
    yield lambda: T_cl.test_norm_direction_and_bound(orc, 1)


def _failures():
    n = 0
    for pin in _pins(oracle):
        try:
            pin()
        except Exception:          # noqa: BLE001 - any failing pin counts
            n += 1
    return n


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.source()
    assert src.count(old) >= 1, f"mutation site for {name} not found"   # planted everywhere
    path = oracle.compile_variant(src.replace(old, new), str(tmp_path / f"{name}.so"))
    saved = oracle._lib
    try:
        oracle._lib = oracle.load(path)
        assert _failures() >= 1, f"no pin caught the planted mistake {name}"
    finally:
        oracle._lib = saved


def test_unplanted_oracle_passes_every_pin():
    oracle.lib()
    assert _failures() == 0
