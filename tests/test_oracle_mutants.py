"""Plant a plausible mistake in a copy of the oracle's C source, compile the
copy with gcc, and check that at least one pin rejects it.  This shows that
the pins would catch a dropped term, a wrong sign or index, a transposed
operand or a broken tie rule in the oracle itself.  CPU only."""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

# (name, original snippet, mutated snippet); every original must occur in
# oracle.c, so a refactor of the oracle makes this test fail loudly rather
# than silently testing nothing.
MUTANTS = [
    ("sigmoid_sign", "exp(-L[e])", "exp(L[e])"),
    ("bias_dropped", "v[e] = s[e] + (bias ? (double)bias[e] : 0.0);", "v[e] = s[e];"),
    ("bias_doubled", "v[e] = s[e] + (bias ? (double)bias[e] : 0.0);",
     "v[e] = s[e] + (bias ? 2.0 * (double)bias[e] : 0.0);"),
    ("gather_biased_scores", "out_w[k] = s[sel[k]] / denom * route_scale;",
     "out_w[k] = v[sel[k]] / denom * route_scale;"),
    ("denominator_biased", "denom += s[sel[k]];", "denom += v[sel[k]];"),
    ("no_renormalise", "out_w[k] = s[sel[k]] / denom * route_scale;",
     "out_w[k] = s[sel[k]] * route_scale;"),
    ("no_route_scale", "out_w[k] = s[sel[k]] / denom * route_scale;",
     "out_w[k] = s[sel[k]] / denom;"),
    ("group_top1_only", "gs[g] = top1 + top2;", "gs[g] = top1 + top1;"),
    ("group_top2_no_multiplicity", "} else if (v[e] > top2) {",
     "} else if (v[e] > top2 && v[e] < top1) {"),
    ("tie_higher_index_wins", "return a < b;", "return a > b;"),
    ("group_index_modulo", "keep[e / S]", "keep[e % G]"),
    ("keep_one_group_too_many", "keep[g] = ahead < KG;", "keep[g] = ahead <= KG;"),
    ("mask_with_zero", "const double fill = opt->mask_zero ? 0.0 : -INFINITY;",
     "const double fill = 0.0;"),
    ("mask_zero_ignored", "const double fill = opt->mask_zero ? 0.0 : -INFINITY;",
     "const double fill = -INFINITY;"),
    ("transposed_W", "acc += bf16_to_double(x_row[j]) * (double)w[j];",
     "acc += bf16_to_double(x_row[j]) * (double)W[j * E + e];"),
    ("bf16_shift", "((uint32_t)h) << 16", "((uint32_t)h) << 15"),
    ("first_logit_term_dropped", "for (int64_t j = 0; j < d; ++j)\n            acc +=",
     "for (int64_t j = 1; j < d; ++j)\n            acc +="),
    ("canonical_order_descending", "while (b >= 0 && sel[b] > key) {",
     "while (b >= 0 && sel[b] < key) {"),
    ("margin_uses_first_winner", "margin[0] = any ? mv[sel[K - 1]] - best_loser : INFINITY;",
     "margin[0] = any ? mv[sel[0]] - best_loser : INFINITY;"),
    ("softmax_unshifted_sum", "sum += exp(L[e] - mx);", "sum += exp(L[e]);"),
    ("softmax_as_sigmoid", "s[e] = exp(L[e] - mx) / sum;", "s[e] = 1.0 / (1.0 + exp(-L[e]));"),
    ("group_max_uses_top2", "gs[g] = top1;   /* no bias: the group maximum */",
     "gs[g] = top1 + top2;"),
    ("renorm_rule_flipped",
     "const int renorm = opt->renorm == 0 ? opt->score_func == 0 : opt->renorm == 1;",
     "const int renorm = opt->renorm == 0 ? opt->score_func == 1 : opt->renorm == 1;"),
    ("epsilon_ignored", "denom += opt->denom_eps;", ""),
    ("combine_not_unpermuted", "acc += w[t * K + k] * bf16_to_double(out[pos * d + j]);",
     "acc += w[t * K + k] * bf16_to_double(out[(t * K + k) * d + j]);"),
    ("combine_first_weight", "acc += w[t * K + k] * bf16_to_double(out[pos * d + j]);",
     "acc += w[t * K] * bf16_to_double(out[pos * d + j]);"),
    ("group_margin_wrong_rank", "if (ahead == KG) next = gs[g];",
     "if (ahead == KG + 1) next = gs[g];"),
    ("dispatch_unstable",
     "for (int64_t p = 0; p < n; ++p) {\n        int32_t e = indices[p];",
     "for (int64_t p = n - 1; p >= 0; --p) {\n        int32_t e = indices[p];"),
    ("offsets_not_cumulative", "offsets[e + 1] = offsets[e] + counts[e];",
     "offsets[e + 1] = counts[e];"),
    ("ep_splits_skip_last_expert", "for (int64_t j = 0; j < per; ++j) c += tokens_per_expert[r * per + j];",
     "for (int64_t j = 0; j + 1 < per; ++j) c += tokens_per_expert[r * per + j];"),
    ("ep_regroup_unstable", "for (int64_t i = 0; i < n; ++i) regroup[fill[label[i]]++] = (int32_t)i;",
     "for (int64_t i = n - 1; i >= 0; --i) regroup[fill[label[i]]++] = (int32_t)i;"),
    ("ep_dedup_keeps_duplicates", "if (indices[t * K + k2] / per == r) { first = k2; break; }",
     "if (0) { first = k2; break; }"),
    ("gather_wrong_row", "memcpy(out + pos * d, x + (p / K) * d,",
     "memcpy(out + pos * d, x + (p % T) * d,"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, orig, mut):
    assert orig in source, f"mutant {name}: snippet not found in oracle.c"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(orig, mut))
    lib = oracle.compile_oracle(str(src), str(tmp_path / f"lib{name}.so"), strict=False)
    o = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except Exception:  # any failure of a pin is a detection
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


def test_unmutated_copy_passes(tmp_path, source):
    """Control: the same compile path without a mutation passes every pin."""
    src = tmp_path / "clean.c"
    src.write_text(source)
    o = oracle.Oracle(oracle.compile_oracle(str(src), str(tmp_path / "libclean.so")))
    for pin in ALL_PINS:
        pin(o)
    assert os.path.exists(o.path)
