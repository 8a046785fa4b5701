"""Each plausible mistake planted in the oracle must fail at least one pin.

The mutants are built from a patched copy of the oracle's C source in a
temporary directory (the committed oracle is never modified) and loaded as
separate shared libraries.  Every mutant keeps memory accesses in bounds.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = [
    ("no_max_shift",  # logsumexp without subtracting the maximum
     "S += exp(oracle_widen(row, dtype, i) - M);\n  return (float)(M + log(S));",
     "S += exp(oracle_widen(row, dtype, i));\n  return (float)(log(S));"),
    ("log2_instead_of_ln", "return (float)(M + log(S));", "return (float)(M + log2(S));"),
    ("float_accumulation", "double S = 0.0;", "float S = 0.0f;"),
    ("ties_by_larger_id", "return (p->id < q->id) ? -1 : (p->id > q->id) ? 1 : 0;",
     "return (p->id > q->id) ? -1 : (p->id < q->id) ? 1 : 0;"),
    ("ascending_values", "if (p->lp > q->lp) return -1;\n  if (p->lp < q->lp) return 1;",
     "if (p->lp < q->lp) return -1;\n  if (p->lp > q->lp) return 1;"),
    ("no_signed_zero_canon", "if (lp == 0.0f) lp = 0.0f;", ""),
    ("wrong_sign", "float lp = x - L;", "float lp = L - x;"),
    ("rank_raw_logits", "all[i].lp = oracle_reported(row, dtype, i, L);",
     "all[i].lp = (float)oracle_widen(row, dtype, i);"),
    ("normalize_with_max", "return (float)(M + log(S));", "return (float)M;"),
    ("padded_lanes_included", "int rc = oracle_row(row, dtype, V, tokens[r], n,",
     "int rc = oracle_row(row, dtype, V_pad, tokens[r], n,"),
    ("ignore_request_flag", "if (requested[s] == 0) continue;", ""),
    ("rows_transposed", "int64_t r = (int64_t)s * T + t;",
     "int64_t r = (int64_t)t * capacity + s;"),
    ("chosen_from_slot", "oracle_row(row, dtype, V, tokens[r], n,",
     "oracle_row(row, dtype, V, tokens[s], n,"),
    ("selected_reversed", "oracle_pair(row, dtype, V, sel[j], L, words + 2 + 2 * j);",
     "oracle_pair(row, dtype, V, sel[n_sel - 1 - j], L, words + 2 + 2 * j);"),
    ("pad_id_zero", "      w[0] = -1;\n", "      w[0] = 0;\n"),
    ("one_alternative_short", "for (int32_t j = 0; j < K; ++j) {\n    int32_t* w",
     "for (int32_t j = 0; j + 1 < K; ++j) {\n    int32_t* w"),
    ("bf16_low_half", "uint32_t w = ((uint32_t)h) << 16;", "uint32_t w = ((uint32_t)h) << 15;"),
    ("no_count_clamp_to_zero", "if (n < 0) n = 0;\n    if (n > ORACLE_MAX_IDS)",
     "if (n < 0) n = 1;\n    if (n > ORACLE_MAX_IDS)"),
    ("invalid_id_zero_bits", "else\n    w[1] = (int32_t)ORACLE_NAN_BITS;", "else\n    w[1] = 0;"),
    ("prompt_rank_counts_ties", "if (oracle_reported(row, dtype, i, L) > rt) ++greater;",
     "if (oracle_reported(row, dtype, i, L) >= rt) ++greater;"),
    ("prompt_rank_on_raw_logits", "if (oracle_reported(row, dtype, i, L) > rt) ++greater;",
     "if (oracle_widen(row, dtype, i) > oracle_widen(row, dtype, target)) ++greater;"),
    ("prompt_rank_zero_based", "words[2] = 1 + greater;", "words[2] = greater;"),
    ("prompt_invalid_rank_one", "words[2] = 0;", "words[2] = 1;"),
    ("prompt_invalid_alt_id_zero", "words[3 + 2 * j] = -1;", "words[3 + 2 * j] = 0;"),
    ("prompt_padded_lanes_ranked", "if (oracle_prompt_row(row, dtype, V, targets[r],",
     "if (oracle_prompt_row(row, dtype, V_pad, targets[r],"),
    ("prompt_targets_reversed", "if (oracle_prompt_row(row, dtype, V, targets[r],",
     "if (oracle_prompt_row(row, dtype, V, targets[rows - 1 - r],"),
    ("packed_rows_read_rectangular",
     "(const char*)logits + (size_t)(first + t) * (size_t)V_pad * esize;",
     "(const char*)logits + (size_t)pos * (size_t)V_pad * esize;"),
    ("packed_range_unchecked", "if (e > 0 && (first < 0 || first + e > P)) continue;", ""),
    ("records_token_field_off_by_one", "int64_t tok64 = record[16 + t];",
     "int64_t tok64 = record[15 + t];"),
    ("records_stride_short", "records + (size_t)s * (16 + (size_t)T);",
     "records + (size_t)s * (15 + (size_t)T);"),
    ("records_count_unchecked", "int32_t e = (count < 0 || count > 2147483647LL) ? 0 : (int32_t)count;",
     "int32_t e = (int32_t)count;"),
    ("records_compact_stride", "memcpy(out + (size_t)at * (size_t)row_words,",
     "memcpy(out + (size_t)at * (size_t)(row_words - 2),"),
    ("prompt_last_alternative_dropped", "sizeof(int32_t) * 2 * ORACLE_PROMPT_ALTS);",
     "sizeof(int32_t) * 2 * (ORACLE_PROMPT_ALTS - 1));"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutated = src.replace(old, new)
    path = os.path.join(tmp_path, "oracle_mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = os.path.join(tmp_path, "liboracle_mutant.so")
    oracle.build(src=path, out=lib, extra=["-Wno-unused-variable", "-Wno-unused-but-set-variable"])
    o = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, OverflowError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
