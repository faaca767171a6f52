"""Plant plausible mistakes in copies of the oracle and check that the pins catch
each one.  CPU only: every mutant is built from a patched copy of oracle.c in
a temporary directory, loaded beside the real oracle, and run through the same
pin checks."""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("centre_lower_middle", "int64_t t = (lo + hi) / 2;", "int64_t t = (lo + hi - 1) / 2;"),
    ("centre_ignores_partial_block",
     "int64_t hi = e * s->block_k < Tp ? e * s->block_k : Tp;",
     "int64_t hi = e * s->block_k;"),
    ("split_ceil_midpoint", "int64_t m = ca[i] + (ce[i] - ca[i]) / 2;",
     "int64_t m = ca[i] + (ce[i] - ca[i] + 1) / 2;"),
    ("tie_prefers_higher_start", "return x->a < y->a;", "return x->a > y->a;"),
    ("keeps_lowest_scores", "if (x->score != y->score) return x->score > y->score;",
     "if (x->score != y->score) return x->score < y->score;"),
    ("no_causal_vote", "if (s->causal && position(s, i) < t) continue;", "if (0) continue;"),
    ("causal_vote_off_by_one", "if (s->causal && position(s, i) < t) continue;",
     "if (s->causal && position(s, i) <= t) continue;"),
    ("strided_head_group", "for (int64_t h = g * G; h < (g + 1) * G; h++)",
     "for (int64_t h = g; h < s->Hq; h += s->Hkv)"),
    ("first_row_only", "for (int64_t i = r0; i < r1; i++) {", "for (int64_t i = r0; i < r0 + 1; i++) {"),
    ("ceil_initial_partition", "ca[i] = first + i * M / Kb;\n    ce[i] = first + (i + 1) * M / Kb;",
     "ca[i] = first + (i * M + Kb - 1) / Kb;\n    ce[i] = first + ((i + 1) * M + Kb - 1) / Kb;"),
    ("attn_no_scale", "const double scale = 1.0 / sqrt((double)s->d);", "const double scale = 1.0;"),
    ("attn_no_causal_mask", "if (t > limit) continue;\n      double w", "double w"),
    ("attn_value_head_of_query", "int64_t vo = ((b * s->Hkv + g) * s->T_cap + t) * s->d;",
     "int64_t vo = ((b * s->Hkv + h % s->Hkv) * s->T_cap + t) * s->d;"),
    ("margin_not_relative", "return den == 0.0 ? 0.0 : (hiS - loS) / den;", "return hiS - loS;"),
    ("dense_case_skipped", "if (M <= Kb) {", "if (M < 0) {"),
    ("score_sum_over_group", "if (v > best) best = v;",
     "best = (best == -INFINITY) ? v : best + v;"),
    ("e5m2_bias_16", "mag = ldexp(1.0 + m / 4.0, e - 15);", "mag = ldexp(1.0 + m / 4.0, e - 16);"),
    ("e5m2_three_mantissa_bits", "mag = ldexp(1.0 + m / 4.0, e - 15);",
     "mag = ldexp(1.0 + m / 8.0, e - 15);"),
    ("e5m2_subnormal_as_normal", "else if (e == 0) mag = ldexp(m / 4.0, -14);",
     "else if (e == 0) mag = ldexp(1.0 + m / 4.0, -15);"),
    ("e5m2_sign_dropped", "return sign ? -mag : mag;", "return mag;"),
    ("e5m2_infinity_as_nan", "if (e == 31) mag = m == 0 ? INFINITY : NAN;", "if (e == 31) mag = NAN;"),
    ("key_type_of_query", "elem(K, s->kv_dtype, ko + x)", "elem(K, s->dtype, ko + x)"),
    ("value_type_of_query", "elem(V, s->kv_dtype, vo + x)", "elem(V, s->dtype, vo + x)"),
    ("window_searched", "const int64_t lo = sb, M = Np - sb - wb;", "const int64_t lo = sb, M = Np - sb;"),
    ("sink_searched", "const int64_t lo = sb, M = Np - sb - wb;", "const int64_t lo = 0, M = Np - wb;"),
    ("sink_not_attended", "((n) < sb ? (n)", "((n) < sb ? -1"),
    ("window_off_by_one", "Np - wb + ((n) - sb)", "Np - wb - 1 + ((n) - sb)"),
    ("dense_listed_twice", "list[(n) - nd] < sb ||", "0 ||"),
    # near-tie-tolerant search
    ("reach_band_not_halved", "double dl = isfinite(sc) ? 0.5 * c->tol * fabs(sc) : 0.0;",
     "double dl = isfinite(sc) ? c->tol * fabs(sc) : 0.0;"),
    ("reach_tolerance_ignored", "double dl = isfinite(sc) ? 0.5 * c->tol * fabs(sc) : 0.0;",
     "double dl = 0.0;"),
    ("reach_band_inverted", "lo[j] = sc - dl;\n    hi[j] = sc + dl;", "lo[j] = sc + dl;\n    hi[j] = sc - dl;"),
    ("reach_one_threshold_only", "for (int64_t k = 0; k < 2 * n && !c->status; k++) {",
     "for (int64_t k = 0; k < 1 && !c->status; k++) {"),
    # multi-stage search
    ("stage0_partial_chunk_dropped", "const int64_t n = (M + c0 - 1) / c0;", "const int64_t n = M / c0;"),
    ("stage0_chunks_overlap", "ce[j] = first + (j + 1) * c0 < first + M ? first + (j + 1) * c0 : first + M;",
     "ce[j] = first + (j + 2) * c0 < first + M ? first + (j + 2) * c0 : first + M;"),
    ("stage_keeps_one_less", "const int64_t kept = n < keep ? n : keep;",
     "const int64_t kept = n < keep ? n : (keep > 1 ? keep - 1 : keep);"),
    ("stage_ends_a_round_early", "        if (ce[i] - ca[i] > tb) wide = 1;",
     "        if (ce[i] - ca[i] > 2 * tb) wide = 1;"),
    ("stage0_ignores_sink_offset", "    ca[j] = first + j * c0;", "    ca[j] = j * c0;"),
    ("stage_without_first_round", "      if (!wide && !fresh) break; /* the stage is done */",
     "      if (!wide) break; /* the stage is done */"),
    ("stage_halving_to_one_block", "const int64_t n = halve_all(ca, ce, nk, tb, ha, he);",
     "const int64_t n = halve_all(ca, ce, nk, 1, ha, he);"),
    ("reach_required_dropped", "req[j] = c->target ? (char)contains_target(c, a[j], e[j]) : 0;",
     "req[j] = c->target ? (char)!contains_target(c, a[j], e[j]) : 0;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique in oracle.c"
    mpath = tmp_path / f"{name}.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(mpath), str(tmp_path / f"lib{name}.so")))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
