"""Plant plausible mistakes in copies of the oracle (on the CPU) and check a pin catches each.

Every mutant is a textual edit of ``oracle/msa_oracle.c`` compiled into a
temporary library; the pins of ``test_oracle_pins`` are run against it and at
least one must fail.  The committed oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "msa_oracle.c")

MUTANTS = [
    ("causal_off_by_one", "for (int64_t j = 0; j <= i; ++j) {\n    double s = 0.0;\n    for (int d = 0; d < d_idx",
     "for (int64_t j = 0; j < i; ++j) {\n    double s = 0.0;\n    for (int d = 0; d < d_idx"),
    ("index_scale_dropped", "  s *= scale;\n    int64_t b = block_of", "  int64_t b = block_of"),
    ("maxpool_is_sum", "if (s > Mrow[b]) Mrow[b] = s;", "Mrow[b] = (Mrow[b] == -INFINITY ? 0.0 : Mrow[b]) + s;"),
    ("block_of_wrong", "return j / B_k;", "return (j + 1) / B_k;"),
    ("tie_to_higher_index", "Mrow[b] > Mrow[best]", "Mrow[b] >= Mrow[best]"),
    ("topk_ascending", "Mrow[b] > Mrow[best]", "Mrow[b] < Mrow[best]"),
    ("local_not_forced", "  chosen[bl] = 1;\n  int count = 1;", "  int count = 0;"),
    ("fill_stops_early", "if (best < 0) break;", "if (best < 0 || count + 1 == k) break;"),
    ("attn_wrong_group", "int r = h / G;", "int r = h % H_kv;"),
    ("attn_causal_off", "int64_t jmax = i < N - 1 ? i : N - 1;", "int64_t jmax = N - 1;"),
    ("attn_no_max_shift", "double p = exp(s_buf[j] - m);", "double p = exp(s_buf[j]);"),
    ("attn_not_normalised", "orow[d] /= l;", "orow[d] /= 1.0;"),
    ("lse_missing_max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("attn_key_head_index", "s += bf16(qv[d]) * bf16(kbase[j * stride + d]);",
     "s += bf16(qv[d]) * bf16(kbase[j * stride + (d_h - 1 - d)]);"),
    ("attn_value_from_key", "orow[d] += p * bf16(vbase[j * stride + d]);",
     "orow[d] += p * bf16(kbase[j * stride + d]);"),
    ("decode_query_position", "int64_t i = L - 1; /* the new token", "int64_t i = L - 2; /* the new token"),
    ("kl_no_head_mean", "P[t] += exp(s_buf[t] - m) / l / G;", "P[t] += exp(s_buf[t] - m) / l;"),
    ("kl_mean_of_log_probs", "P[t] += exp(s_buf[t] - m) / l / G;", "P[t] *= pow(exp(s_buf[t] - m) / l, 1.0 / G);"),
    ("kl_reversed", "if (P[t] > 0.0) kl += P[t] * (log(P[t]) - (sidx[t] - lse_idx));",
     "kl += exp(sidx[t] - lse_idx) * ((sidx[t] - lse_idx) - log(P[t]));"),
    ("kl_index_scale_dropped", "sidx[t] = sv / sqrt((double)d_idx);", "sidx[t] = sv;"),
    ("kl_not_causal", "for (int64_t j = 0; j <= jmax; ++j)\n    if (inset", "for (int64_t j = 0; j < N; ++j)\n    if (inset"),
    ("kl_index_query_group", "q_idx + (i * H_kv + r) * d_idx", "q_idx + (i * H_kv) * d_idx"),
    ("kl_lse_idx_missing_max", "double lse_idx = mi + log(li);", "double lse_idx = log(li);"),
    ("fp8_exponent_bias", "v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("fp8_subnormal_scale", "v = ldexp(m / 8.0, -6);", "v = ldexp(m / 8.0, -7);"),
    ("paged_wrong_row", "(((int64_t)pages[j / B_k] * B_k + j % B_k) * H_kv + r) * d_h;\n          double sv",
     "(((int64_t)pages[j / B_k] * B_k + (j + 1) % B_k) * H_kv + r) * d_h;\n          double sv"),
    ("paged_scales_swapped", "sv += bf16(qv[d]) * (k_scale * msa_oracle_fp8_e4m3(kr[d]));",
     "sv += bf16(qv[d]) * (v_scale * msa_oracle_fp8_e4m3(kr[d]));"),
    ("bwd_no_scale_dq", "dqr[d] += scale * ds * bf16(kr[d]);", "dqr[d] += ds * bf16(kr[d]);"),
    ("bwd_no_D", "double ds = P[j] * (dp - D);", "double ds = P[j] * dp;"),
    ("bwd_dv_from_ds", "dvr[d] += P[j] * bf16(dov[d]);", "dvr[d] += ds * bf16(dov[d]);"),
    ("bwd_dk_wrong_operand", "dkr[d] += scale * ds * bf16(qv[d]);", "dkr[d] += scale * ds * bf16(dov[d]);"),
    ("bwdpart_diagonal_block", "for (int64_t i = jlo; i < N; ++i)", "for (int64_t i = jhi; i < N; ++i)"),
    ("bwdpart_block_range", "const int in_blk = j >= jlo && j < jhi;", "const int in_blk = j > jlo && j < jhi;"),
    ("bwdpart_dq_row_head", "dq_rows + (a * H_q + r * G + g) * d_h", "dq_rows + (a * H_q + g * H_kv + r) * d_h"),
    ("bwdpart_dv_operand", "bf16(qv[d]);\n        dvr[d] += P[j] * bf16(dov[d]);", "bf16(qv[d]);\n        dvr[d] += P[j] * bf16(qv[d]);"),
    ("paged_index_page", "kidx_pages + ((int64_t)pages[j / B_k] * B_k + j % B_k) * d_idx",
     "kidx_pages + ((int64_t)(j / B_k) * B_k + j % B_k) * d_idx"),
]


def _all_pins():
    """Every pin, called with fixed arguments; yields (name, thunk)."""
    cases = pins._golden_topk_cases()
    yield "partition", pins.test_partition_counts_match_workloads
    yield "one_hot", pins.test_block_scores_one_hot_closed_form
    yield "scale", pins.test_block_scores_scale_does_not_change_ranking
    for c in cases:
        yield f"golden_{c[0]}", (lambda c=c: pins.test_topk_golden(c))
    yield "full_sort", lambda: pins.test_topk_matches_full_sort(0)
    yield "local", pins.test_local_block_always_selected_and_exp_free
    yield "padding", pins.test_fewer_than_k_blocks_padding
    yield "dense", lambda: pins.test_k_covering_all_blocks_is_dense_gqa(37, 4, 2, 8, 16)
    yield "sum_to_one", pins.test_softmax_rows_sum_to_one
    yield "uniform", pins.test_uniform_scores_closed_form
    yield "lse_merge", pins.test_lse_merge_of_disjoint_partials
    yield "order", pins.test_block_order_and_empty_sets
    yield "decode", pins.test_decode_equals_last_prefill_row
    yield "kl_zero", pins.test_kl_zero_when_index_scores_equal_main_scores
    yield "kl_closed_form", pins.test_kl_closed_form_mean_of_two_heads
    yield "kl_token_set", pins.test_kl_token_set_is_causal_and_selected
    yield "kl_groups", pins.test_kl_is_nonnegative_and_groups_are_separate
    yield "bwd_autograd", lambda: pins.test_attention_backward_matches_autograd(300, 4, 2, 2, 64)
    yield "bwd_fd", pins.test_attention_backward_finite_differences
    yield "bwd_part", lambda: pins.test_restricted_backward_matches_autograd(300, 4, 2, 2, 64)
    yield "bwd_part_full", pins.test_restricted_backward_equals_full_oracle
    yield "fp8", pins.test_fp8_e4m3_decoding
    yield "paged", pins.test_paged_fp8_decode_equals_contiguous_decode
    yield "paged_scales", pins.test_paged_fp8_scales_multiply_keys_and_values


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m[0])
def test_a_pin_catches_the_mutant(mutant, tmp_path):
    name, old, new = mutant
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mut_src = tmp_path / "mut.c"
    mut_src.write_text(src.replace(old, new, 1))
    so = tmp_path / f"libmut_{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-I",
                    os.path.dirname(SRC), "-o", str(so), str(mut_src), "-lm"], check=True)
    caught = []
    oracle.use_library(str(so))
    try:
        for pin_name, fn in _all_pins():
            try:
                fn()
            except (AssertionError, ValueError, IndexError):
                caught.append(pin_name)
    finally:
        oracle.use_library(None)
    assert caught, f"no pin caught mutant {name}"
