"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (on the CPU, in a
temporary directory), builds it with the oracle's own flags, binds the
wrapper to it and runs the pins that should notice; at least one must fail.
The committed oracle is never modified.
"""
import os
import shutil
import subprocess
import tempfile
import ctypes

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
HDR = os.path.join(os.path.dirname(oracle.__file__), "oracle.h")

# (name, text in oracle.c, replacement, pins that must notice)
MUTANTS = [
    ("residual sign flipped",
     "double diff = exp(pr[v] / T - lp) - exp(qr[v] / T - lq);",
     "double diff = exp(qr[v] / T - lq) - exp(pr[v] / T - lp);",
     [lambda: pins.test_oracle_output_distribution_equals_target(oracle, "token", 5),
      lambda: pins.test_oracle_acceptance_equals_overlap_mass(oracle)]),
    ("acceptance ratio inverted",
     "double r = exp(lp - lq);", "double r = exp(lq - lp);",
     [lambda: pins.test_printed_acceptance_ratio(oracle)]),
    ("residual not clamped at zero",
     "wv[v] = diff > 0.0 ? diff : 0.0;", "wv[v] = diff;",
     [lambda: pins.test_oracle_output_distribution_equals_target(oracle, "token", 5),
      lambda: pins.test_oracle_acceptance_equals_overlap_mass(oracle)]),
    ("walk does not stop at the first rejection",
     "if (!(u < (float)ratio)) { tau = i - 1; break; }", "if (!(u < (float)ratio)) { tau = i - 1; }",
     [lambda: pins.test_oracle_output_distribution_equals_target(oracle, "token", 5),
      lambda: pins.test_printed_expected_words(oracle)]),
    ("block running ratio not capped",
     "w[i] = prod < 1.0 ? prod : 1.0;", "w[i] = prod;",
     [lambda: pins.test_oracle_block_toy_example_forced_uniforms(oracle),
      lambda: pins.test_oracle_output_distribution_equals_target(oracle, "block", 6)]),
    ("block threshold without 1 - w",
     "h[i] = den > 0.0 ? m / den : 1.0;", "h[i] = den > 0.0 ? m / (m + 1.0) : 1.0;",
     [lambda: pins.test_oracle_block_toy_example_forced_uniforms(oracle),
      lambda: pins.test_oracle_output_distribution_equals_target(oracle, "block", 6)]),
    ("block keeps the first passing prefix",
     "if (eta < (float)h[i]) tau = i;", "if (eta < (float)h[i] && tau == 0) tau = i;",
     [lambda: pins.test_oracle_block_toy_example_monte_carlo(oracle),
      lambda: pins.test_oracle_output_distribution_equals_target(oracle, "block", 6)]),
    ("block correction ignores w_tau",
     "double diff = w[tau] * exp(pr[v] / T - lp) - exp(qr[v] / T - lq);",
     "double diff = exp(pr[v] / T - lp) - exp(qr[v] / T - lq);",
     [lambda: pins.test_oracle_output_distribution_equals_target(oracle, "block", 210)]),
    ("inverse CDF threshold halved",
     "const float tf = (float)((double)u * (double)Zf);",
     "const float tf = (float)((double)u * (double)Zf * 0.5);",
     [lambda: pins.test_icdf_equals_searchsorted(oracle)]),
    ("normaliser sum ignores temperature",
     "for (int64_t v = 0; v < V; ++v) s += exp(row[v] / T - m);",
     "for (int64_t v = 0; v < V; ++v) s += exp(row[v] - m);",
     [lambda: pins.test_row_lse_closed_forms_and_library(oracle)]),
    ("Philox Weyl constant",
     "const uint32_t W0 = 0x9E3779B9u", "const uint32_t W0 = 0x9E3779BBu",
     [lambda: pins.test_philox_matches_rocrand_engine(oracle)]),
    ("scheduler ignores the batch growth",
     "double gain = c[k].s * (sps_k + rows);", "double gain = c[k].s * sps_k;",
     [lambda: pins.test_scheduler_equals_brute_force_optimum(oracle)]),
    ("scheduler ranks ascending",
     "if (a->s > c->s) return -1;          /* survival descending */\n    if (a->s < c->s) return 1;",
     "if (a->s < c->s) return -1;\n    if (a->s > c->s) return 1;",
     [lambda: pins.test_scheduler_equals_brute_force_optimum(oracle)]),
    ("temperature multiplies the log-odds",
     "exp(-(l / temps[i]))", "exp(-(l * temps[i]))",
     [lambda: pins.test_sts_closed_forms(oracle)]),
    ("temperature of the previous position",
     "exp(-(l / temps[i]))", "exp(-(l / temps[i > 0 ? i - 1 : 0]))",
     [lambda: pins.test_sts_closed_forms(oracle), lambda: pins.test_sts_equals_library_logistic(oracle)]),
    ("logistic of the negated log-odds",
     "exp(-(l / temps[i]))", "exp(l / temps[i])",
     [lambda: pins.test_sts_closed_forms(oracle)]),
    ("RNN state ignores the recurrent matrix",
     "acc = fmaf(hb[r], (float)A[(int64_t)j * R + r], acc);", "acc = fmaf(hb[r], 0.0f, acc);",
     [lambda: pins.test_rnn_state_recurrence_against_numpy(oracle),
      lambda: pins.test_rnn_chain_distribution(oracle)]),
    ("RNN recurrent matrix transposed",
     "acc = fmaf(hb[r], (float)A[(int64_t)j * R + r], acc);", "acc = fmaf(hb[r], (float)A[(int64_t)r * R + j], acc);",
     [lambda: pins.test_rnn_state_recurrence_against_numpy(oracle),
      lambda: pins.test_rnn_chain_distribution(oracle)]),
    ("RNN state not carried to the next position",
     "for (int j = 0; j < R; ++j) hb[j] = hn[j];", "for (int j = 0; j < R; ++j) (void)hn[j];",
     [lambda: pins.test_rnn_without_recurrence_is_markov_on_tanh_embeddings(oracle)]),
    ("RNN state without tanh",
     "hn[j] = orc_bf16_round(tanhf(acc), &d);", "hn[j] = orc_bf16_round(acc, &d);",
     [lambda: pins.test_rnn_without_recurrence_is_markov_on_tanh_embeddings(oracle)]),
    ("bf16 rounding truncates",
     "if (low > 0x8000u || (low == 0x8000u && (kept & 0x10000u))) kept += 0x10000u;", "(void)low;",
     [lambda: pins.test_bf16_rounding_equals_torch(oracle)]),
    ("tree residual restarts from p at every rejection",
     "double diff = r[v] / Zr - qd[v];", "double diff = pd[v] - qd[v];",
     [lambda: pins.test_oracle_tree_output_distribution_equals_target(oracle, [0, 0, 0, 1])]),
    ("tree later children tested with the first child's ratio",
     "if (rejections == 0) {", "if (1) {",
     [lambda: pins.test_oracle_tree_output_distribution_equals_target(oracle, [0, 0, 0, 1])]),
    ("tree final draw from p instead of the residual",
     "y = orc_icdf(r, V, u2, &Z, &marg);          /* every child rejected: the residual */",
     "y = orc_icdf(pd, V, u2, &Z, &marg);",
     [lambda: pins.test_tree_chain_equals_token_verification(oracle),
      lambda: pins.test_oracle_tree_output_distribution_equals_target(oracle, [0, 0, 0, 1])]),
    ("tree first child ratio inverted",
     "const double lr = (prow[x] / T - lp) - (qr[x] / T - lq);", "const double lr = (qr[x] / T - lq) - (prow[x] / T - lp);",
     [lambda: pins.test_tree_chain_equals_token_verification(oracle)]),
    ("Markov transition from the anchor only",
     "prev = (int32_t)y;", "(void)y;",
     [lambda: pins.test_markov_chain_distribution(oracle)]),
    ("Markov transition subtracted",
     "z[v] = bk[v] + dsum;", "z[v] = bk[v] - dsum;",
     [lambda: pins.test_markov_contraction_matches_matmul(oracle)]),
]


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, checks):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as td:
        shutil.copy(HDR, td)
        c = os.path.join(td, "oracle.c")
        with open(c, "w") as f:
            f.write(mutated)
        so = os.path.join(td, "liboracle_mutant.so")
        subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                        "-o", so, c, "-lm"], check=True, capture_output=True)
        lib = oracle.declare(ctypes.CDLL(so))
        saved = oracle._load()
        oracle._lib = lib
        caught = []
        try:
            for chk in checks:
                try:
                    chk()
                except (AssertionError, ValueError) as e:
                    caught.append(type(e).__name__)
        finally:
            oracle._lib = saved
    assert caught, f"no pin noticed the planted mistake: {name}"
