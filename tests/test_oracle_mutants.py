"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of oracle/sv_oracle.c with one plausible mistake
planted (a dropped term, a wrong sign, index, operand or comparison).  The
copy is compiled into a temporary directory, the oracle module is pointed at
it, and the pin battery is run: every mutant must make at least one pin
fail.  The real oracle is restored afterwards.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as P
import test_oracle_stats as S
import test_oracle_tree_kv as TK
import test_oracle_tree_build as TB
import test_oracle_tree_mask as TM
import test_oracle_draft as TD

SRC = os.path.join(os.path.dirname(oracle.__file__), "sv_oracle.c")

MUTANTS = {
    "residual_sign": ("double d = qt - pt;", "double d = pt - qt;"),
    "accept_not_strict": ("return u < threshold;", "return u <= threshold;"),
    "accept_ratio_inverted": ("double r = exp(lq - lp);", "double r = exp(lp - lq);"),
    "p_zero_rejects": ("        *ratio = INFINITY;\n        return 1;", "        *ratio = INFINITY;\n        return 0;"),
    "temperature_dropped_on_p": ("logit_at(pr, dtype, tok) / T, lse_p[i]", "logit_at(pr, dtype, tok), lse_p[i]"),
    "residual_fallback_dropped": ("    if (s == 0.0) {\n        row_probs", "    if (s < 0.0) {\n        row_probs"),
    "cdf_not_strict": ("if (cum > target) {", "if (cum >= target) {"),
    "residual_wrong_q_row": ("const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, k);",
                             "const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, k + 1);"),
    "bonus_wrong_row": ("const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, N);",
                        "const void* qr = row_ptr(zq, dtype, q_seq_stride, q_row_stride, b, N - 1);"),
    "sample_slot_off_by_one": ("orc_uniforms(seed, round, (uint32_t)b, (uint32_t)(k + 1), NULL, &us);",
                               "orc_uniforms(seed, round, (uint32_t)b, (uint32_t)(k + 2), NULL, &us);"),
    "lse_missing_max": ("    if (lse_out) *lse_out = m + log(s);", "    if (lse_out) *lse_out = log(s);"),
    "philox_key_bump": ("k0 += 0x9E3779B9u;", "k0 += 0x9E3779B1u;"),
    "u53_shift": ("double lo = (double)(b >> 6);", "double lo = (double)(b >> 5);"),
    "tree_child_own_rows": ("            int pa = par[n];", "            int pa = n;"),
    "tree_highest_child": ("            for (int n = cur + 1; n < nn; ++n) {\n                if (par[n] != cur) continue;",
                           "            for (int n = nn - 1; n > cur; --n) {\n                if (par[n] != cur) continue;"),
    "tree_best_child_tries_siblings": ("                    if (acc[n]) next = n;\n                    break;",
                                       "                    if (acc[n]) {\n                        next = n;\n                        break;\n                    }"),
    "tree_best_child_ignored": ("                if (walk == 1) {        /* R5b", "                if (walk == 2) {        /* R5b"),
    "tree_bonus_after_reject": ("            if (next < 0) {\n                residual = 1;",
                                "            if (next < 0) {\n                residual = 0;"),
    "kv_len_off_by_one": ("out_kv_len[b] = L0 + k + 1;", "out_kv_len[b] = L0 + k;"),
    "kv_gather_wrong_dst": ("memcpy(seqbase + (int64_t)(L0 + i) * row_stride,", "memcpy(seqbase + (int64_t)(L0 + k - i) * row_stride,"),
    "mask_misses_self": ("            for (int j = n;; j = par[j]) {", "            for (int j = n ? par[n] : 0;; j = par[j]) {"),
    "mask_one_word": ("row[j / 64] |= (uint64_t)1 << (j % 64);", "row[0] |= (uint64_t)1 << (j % 64);"),
    "mask_depth_counts_self": ("positions[(int64_t)b * nn + n] = L0 + depth;", "positions[(int64_t)b * nn + n] = L0 + depth + 1;"),
    "mask_root_unchecked": ("int ok = par[0] == -1;", "int ok = 1;"),
    "tree_ties_to_later_token": ("while (pos > 0 && top_val[pos - 1] < v) {", "while (pos > 0 && top_val[pos - 1] <= v) {"),
    "tree_score_without_lse": ("c_score[n] = f_score[f] + (top_val[r] / T - lse);", "c_score[n] = f_score[f] + top_val[r] / T;"),
    "tree_frontier_worst": ("                    f_ids[r] = order[r].id;\n                    f_score[r] = order[r].score;",
                            "                    f_ids[r] = order[cnt - 1 - r].id;\n                    f_score[r] = order[cnt - 1 - r].score;"),
    "draft_verify_stream": ("orc_philox_block(seed, round, (uint32_t)b, (uint32_t)(pos0 + r), 1u, w4);",
                            "orc_philox_block(seed, round, (uint32_t)b, (uint32_t)(pos0 + r), 0u, w4);"),
    "draft_logprob_without_T": ("logit_at(row, dtype, tok) / T - lse : NAN;", "logit_at(row, dtype, tok) - lse : NAN;"),
    "draft_wrong_row": ("const void* row = row_ptr(zp, dtype, seq_stride, row_stride, b, r);",
                        "const void* row = row_ptr(zp, dtype, seq_stride, row_stride, b, 0);"),
    "cdf_edges_off_by_one": ("for (int t = 0; t < V && t < g; ++t) cum += w[t];",
                             "for (int t = 0; t < V && t <= g; ++t) cum += w[t];"),
    "cdf_edges_hi_without_token": ("*hi = (g >= 0 && g < V) ? cum + w[g] : cum;", "*hi = cum;"),
    "tree_parent_score_dropped": ("c_score[n] = f_score[f] + (top_val[r] / T - lse);", "c_score[n] = top_val[r] / T - lse;"),
}


def _battery():
    """Pins that run in seconds and together cover every function."""
    yield lambda: P.test_philox_known_answers(oracle)
    yield lambda: P.test_u53_is_exact_dyadic(oracle)
    for dt in ("f32", "bf16"):
        yield lambda dt=dt: P.test_row_lse_matches_logsumexp(oracle, dt, 0.7)
    yield lambda: P.test_n0_is_plain_categorical_sampling(oracle)
    yield lambda: P.test_theorem_on_oracle_primitives(oracle, 5, 2)
    yield lambda: P.test_accept_rule_edges(oracle)
    for V, N, T in [(5, 2, 1.0), (5, 2, 0.75)]:
        yield lambda V=V, N=N, T=T: P.test_chain_structure_under_forced_uniforms(oracle, V, N, T)
    yield lambda: P.test_chain_uses_documented_uniforms(oracle)
    yield lambda: P.test_residual_of_equal_rows_falls_back_to_q(oracle)
    yield lambda: P.test_inverse_cdf_edges_are_strict(oracle)
    yield lambda: P.test_cdf_edges_of_queried_tokens(oracle)
    yield lambda: P.test_exercise4_batched_kv_length(oracle)
    yield lambda: S.test_stratified_sampling_sweep(oracle, 4)
    yield lambda: S.test_chain_b1_every_slot_is_distributed_as_q(oracle)
    yield lambda: TK.test_tree_walk_under_forced_flags(oracle, 4)
    yield lambda: TK.test_tree_walk_under_forced_flags(oracle, 7)
    yield lambda: TK.test_best_child_walk_ignores_an_accepted_sibling(oracle)
    yield lambda: TK.test_best_child_walk_under_forced_flags(oracle, 5)
    yield lambda: TK.test_kv_gather_matches_fancy_indexing(oracle, False)
    yield lambda: TM.test_chain_is_the_causal_mask(130)
    yield lambda: TM.test_every_small_tree_by_matrix_powers(5)
    yield lambda: TM.test_bad_parents_mark_only_their_sequence()
    yield lambda: TB.test_ties_go_to_the_lower_token()
    yield lambda: TB.test_depth1_is_the_roots_topk(1.0)
    yield lambda: TB.test_matches_the_generators_construction(512, 3)
    yield lambda: TB.test_level2_scores_are_path_sums()
    yield lambda: TD.test_uniform_source_and_token_by_searchsorted()
    yield lambda: TD.test_logprob_is_log_softmax()


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site of {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", str(src), "-o",
                    str(lib), "-lm"], check=True)
    prev = oracle._swap_library(str(lib))
    killed = None
    try:
        for check in _battery():
            try:
                check()
            except (AssertionError, ValueError, IndexError, KeyError) as e:
                killed = repr(e)[:120]
                break
    finally:
        oracle._swap_library(prev)
    assert killed is not None, f"mutant {name} survived every pin"
