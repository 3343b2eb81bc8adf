"""The oracle pins reject plausible mistakes.

Each case below plants one mistake into a copy of the oracle's C source (on
the CPU, in a temporary directory), builds that copy, and runs the pins of
test_oracle_pins.py against it: at least one pin must fail.  The committed
oracle is untouched; this only shows that the pins would catch a dropped
term, a wrong weight, a wrong sign, a wrong divisor or a wrong index.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild

from . import test_oracle_pins as P

INF = float("inf")

PINS = {
    "pool-const-ragged": lambda: P.test_pool_constant_blocks_closed_form(100, 64),
    "pool-const": lambda: P.test_pool_constant_blocks_closed_form(10, 4),
    "eq11": lambda: P.test_eq11_column_mean_of_token_tile_is_proxy(300, 64),
    "eq5": P.test_eq5_moment_form_matches_direct_statistics,
    "gauss": lambda: P.test_gaussian_row_density_is_upper_tail(1.0),
    "gauss-pages": P.test_pages_gaussian_density_example,
    "strict": P.test_threshold_is_strict_and_infinite_betas,
    "dense": lambda: P.test_beta_minus_inf_is_dense_attention(100, 16, 8),
    "B1": lambda: P.test_block_size_one_is_dense_for_every_beta(0.0),
    "blockconst": lambda: P.test_block_constant_keys_give_dense_for_every_beta(0.0, 90, 16),
    "mean-value": lambda: P.test_single_approximate_block_gives_its_mean_value(0.0, 40, 64),
    "wsum": lambda: P.test_weights_sum_to_one(0.0),
    "brute": lambda: P.test_merge_equals_brute_force_token_logits(130, 16, 8, 0.3),
    "brute2": lambda: P.test_merge_equals_brute_force_token_logits(200, 32, 16, -0.2),
    "pooled-attn": P.test_beta_plus_inf_is_attention_over_pooled_keys,
    "perm": P.test_permuting_keys_inside_unselected_block_changes_nothing,
    "topk-count": lambda: P.test_topk_keeps_k_blocks_and_none_scored_below_a_dropped_one(5),
    "topk-ties": P.test_topk_ties_go_to_the_lower_block_index,
    "topk-vs-threshold": P.test_topk_at_a_rows_own_count_is_the_threshold_selection,
    "drop-dense": P.test_drop_with_every_block_selected_is_dense_attention,
    "drop-brute": lambda: P.test_drop_is_softmax_over_the_selected_tokens_only(100, 16),
    "drop-empty": P.test_drop_with_nothing_selected_is_zero,
}

# name -> (text in sol_oracle.c, replacement, replace every occurrence)
MUTANTS = {
    "value-pooled-as-mean": ("vs[c] = sv;", "vs[c] = sv / (double)n;", False),
    "query-mean-over-B": ("qb[c] = sq / (double)n;", "qb[c] = sq / (double)B;", False),
    "key-mean-over-B": ("kb[c] = sk / (double)n;", "kb[c] = sk / (double)B;", False),
    "proxy-unscaled": ("row[j] = c * s;", "row[j] = s;", False),
    "proxy-drops-a-dim": ("for (int x = 0; x < d; ++x) s += qi[x] * kj[x];",
                          "for (int x = 0; x < d - 1; ++x) s += qi[x] * kj[x];", True),
    "sample-variance": ("var /= (double)N;", "var /= (double)(N > 1 ? N - 1 : 1);", False),
    "non-strict-threshold": ("const int s_in = row[j] > t;", "const int s_in = row[j] >= t;",
                             False),
    "threshold-sign": ("else t = m + beta * sg;", "else t = m - beta * sg;", False),
    "threshold-uses-variance": ("else t = m + beta * sg;", "else t = m + beta * var;", False),
    "approx-denominator-B": ("D += (double)n * w;", "D += (double)B * w;", False),
    "approx-denominator-unweighted": ("D += (double)n * w;", "D += w;", False),
    "approx-numerator-dropped": ("for (int e = 0; e < d; ++e) num[e] += w * vs[e];", ";", False),
    "approx-numerator-times-n": ("num[e] += w * vs[e];", "num[e] += (double)n * w * vs[e];",
                                 False),
    "exact-logits-unscaled": ("a_tok[tok] = c * s;", "a_tok[tok] = s;", False),
    "approx-logits-unscaled": ("g_blk[j] = c * s;", "g_blk[j] = s;", False),
    "exact-denominator-dropped": ("D += w;\n                        for (int e = 0; e < d; ++e) "
                                  "num[e] += w * (double)vt[e];",
                                  "for (int e = 0; e < d; ++e) num[e] += w * (double)vt[e];",
                                  False),
    "selection-transposed": ("if (srow[j])", "if (sel[((int64_t)h * N + j) * N + i])", True),
    "query-block-off-by-one": ("const int64_t i = r / B;", "const int64_t i = (r + 1) / B;",
                               False),
    "dense-unscaled": ("s[t] = c * acc;", "s[t] = acc;", False),
    "topk-ties-to-higher-index": ("return (x->j > y->j) - (x->j < y->j);",
                                  "return (x->j < y->j) - (x->j > y->j);", False),
    "topk-keeps-one-fewer": ("for (int x = 0; x < k; ++x) sel[base + row[x].j] = 1;",
                             "for (int x = 0; x + 1 < k; ++x) sel[base + row[x].j] = 1;", False),
    "topk-keeps-smallest": ("if (x->s > y->s) return -1;", "if (x->s < y->s) return -1;", False),
    "drop-keeps-approx-terms": ("} else if (!drop_approx) {\n                    /* approximate",
                                "} else {\n                    /* approximate", False),
    "drop-empty-row-nan": ("o[e] = D > 0.0 ? num[e] / D : 0.0;", "o[e] = num[e] / D;", False),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def _build_mutant(name, mdir):
    old, new, every = MUTANTS[name]
    src = open(obuild.SRC).read()
    n = src.count(old)
    assert n >= 1 and (every or n == 1), f"mutation site for {name} not unique ({n})"
    src = src.replace(old, new) if every else src.replace(old, new, 1)
    c = os.path.join(mdir, f"{name}.c")
    so = os.path.join(mdir, f"{name}.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, c, "-lm"],
                   check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, mutant_dir):
    so = _build_mutant(name, str(mutant_dir))
    caught = []
    with oracle.using_library(so):
        for pin, fn in PINS.items():
            try:
                fn()
            except (AssertionError, RuntimeError, ValueError):
                caught.append(pin)
    assert caught, f"no pin rejects the planted mistake {name!r}"


def test_unmutated_oracle_passes_every_pin():
    for pin, fn in PINS.items():
        fn()
