"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a private copy of oracle.c (on the CPU, in a
temporary directory), builds it, and runs the pin tests that should notice it
against that copy (through the ORACLE_SO override).  A case passes when the
pin run FAILS.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
HDR = os.path.join(ROOT, "oracle", "oracle.h")

R = "tests/test_oracle_routing.py"
X = "tests/test_oracle_experts.py"
S = "tests/test_oracle_sigmoid.py"
B = "tests/test_oracle_balance.py"
D = "tests/test_oracle_backward.py"
FD = D + "::test_every_gradient_matches_central_differences"

MUTANTS = {
    "group_score_top1": ("  return m1 + m2;", "  return m1 + m1;", [R + "::test_brute_force_full_shape"]),
    "group_tie_to_higher": ("if (best < 0 || gs[g] > gs[best]) best = g;",
                            "if (best < 0 || gs[g] >= gs[best]) best = g;", [R + "::test_hand_examples"]),
    "expert_tie_to_higher": ("if (best < 0 || sb[e] > sb[best]) best = e;",
                             "if (best < 0 || sb[e] >= sb[best]) best = e;", [R + "::test_hand_examples"]),
    "weights_from_biased": ("    float q = s[idx[j]] / d;", "    float q = sb[idx[j]] / d;",
                            [R + "::test_hand_examples"]),
    "group_score_unbiased": ("gs[g] = group_top2_sum(sb, g * gsize, gsize);",
                             "gs[g] = group_top2_sum(s, g * gsize, gsize);", [R + "::test_hand_examples"]),
    "no_scale": ("    w[j] = q * scale;", "    w[j] = q;", [R + "::test_weights_sum_and_ratio"]),
    "no_epsilon": ("  float d = S + 1e-20f;", "  float d = S;",
                   [R + "::test_epsilon_matters_when_scores_underflow"]),
    "bias_ignored": ("sb[e] = s[e] + (bias ? bias[e] : 0.0f);", "sb[e] = s[e];",
                     [R + "::test_hand_examples"]),
    "no_group_mask": ("    if (!gkeep[e / gsize]) sb[e] = -INFINITY;", "    ;",
                      [R + "::test_hand_examples"]),
    "permute_unstable": ("  for (int64_t p = 0; p < P; ++p) {\n    int32_t pos",
                         "  for (int64_t p = P - 1; p >= 0; --p) {\n    int32_t pos",
                         [R + "::test_permute_matches_numpy"]),
    "logits_transposed": ("const float* wr = c->w + (size_t)e * c->H;",
                          "const float* wr = c->w + (size_t)e;",
                          [R + "::test_logits_match_numpy"]),
    "gate_up_swapped": ("    a[i] = g / (1.0 + exp(-g)) * u;", "    a[i] = u / (1.0 + exp(-u)) * g;",
                        [X + "::test_matches_numpy_matmul"]),
    "shared_weighted": ("      for (int h = 0; h < H; ++h) yr[h] = o[h];",
                        "      for (int h = 0; h < H; ++h) yr[h] = o[h] * c->w[(size_t)t * K];",
                        [X + "::test_zero_weights_leave_shared_expert_unweighted"]),
    "sigmoid_bad_coefficient": ("    taylor_c[i] = 1.0 / fact;", "    taylor_c[i] = 1.0 / (fact + (i == 5));",
                                [S + "::test_accuracy_and_monotonicity_sampled"]),
    "track_no_accumulate": ("    tracking[e] += n;", "    tracking[e] = n;",
                            [B + "::test_track_hand_example_and_accumulation"]),
    "stats_sample_variance": ("s[3] = sqrt(ss / (double)E) / mean;",
                              "s[3] = sqrt(ss / (double)(E - 1)) / mean;", [B + "::test_stats_hand_example"]),
    "stats_cold_tie_to_higher": ("if (h[e] < h[cold]) cold = e;", "if (h[e] <= h[cold]) cold = e;",
                                 [B + "::test_stats_ties_take_the_lowest_index"]),
    "bias_step_sign": ("double v = (-rate * ((double)counts[e] - cbar)) / d;",
                       "double v = (rate * ((double)counts[e] - cbar)) / d;",
                       [B + "::test_bias_update_hand_example"]),
    "bias_not_normalised": ("    if (ex > d) d = ex;", "    ;", [B + "::test_bias_update_hand_example"]),
    "aux_no_num_experts": ("  *loss = (double)E * acc;", "  *loss = acc;", [B + "::test_aux_loss_balanced_is_k"]),
    "aux_unnormalised_probs": ("    for (int e = 0; e < E; ++e) P[e] += p[e] / z;",
                               "    for (int e = 0; e < E; ++e) P[e] += p[e];",
                               [B + "::test_aux_loss_balanced_is_k"]),
    "aux_sigmoid_probs": ("      p[e] = exp((double)l[e] - m);", "      p[e] = 1.0 / (1.0 + exp(-(double)l[e]));",
                          [B + "::test_aux_loss_closed_form_one_large_logit"]),
    "sigmoid_sign": ("  double t = -(double)z;", "  double t = (double)z;", [S + "::test_textbook_values"]),
    "bwd_silu_derivative_one_term": ("    double dsilu = sg * (1.0 + g[i] * (1.0 - sg));",
                                     "    double dsilu = sg;", [FD]),
    "bwd_quotient_rule_sign": ("      double ds = c->scale / D * (gw[j] - sgs / D);",
                               "      double ds = c->scale / D * (gw[j] + sgs / D);", [FD]),
    "bwd_up_grad_uses_gate": ("    du[i] = da * silu;", "    du[i] = da * g[i];", [FD]),
    "bwd_no_sigmoid_slope": ("      double dlam = ds * s[j] * (1.0 - s[j]);",
                             "      double dlam = ds * s[j];", [FD]),
    "bwd_pairs_unweighted": ("      w = wj[c->pj[p]];", "      w = 1.0;", [FD]),
    "bwd_down_grad_from_gate": ("        rd[h] += ai * d_o[h];", "        rd[h] += gi * d_o[h];", [FD]),
    "bwd_router_grad_no_x": ("      for (int h = 0; h < H; ++h) dwr[(size_t)e * H + h] += d * elem(x, xdt, (size_t)t * H + h);",
                             "      for (int h = 0; h < H; ++h) dwr[(size_t)e * H + h] += d;", [FD]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    find, repl, nodes = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(find) >= 1, f"mutation site for {name} not found"
    # the transposed-logits mutant indexes with a stride of 1 instead of H; keep
    # it in bounds by striding over e with H (reads W as if it were [H][E])
    if name == "logits_transposed":
        src = src.replace("acc += xr[h] * (double)wr[h];", "acc += xr[h] * (double)wr[(size_t)h * c->E];")
    mutated = src.replace(find, repl)
    with tempfile.TemporaryDirectory() as d:
        shutil.copy(HDR, os.path.join(d, "oracle.h"))
        with open(os.path.join(d, "oracle.c"), "w") as f:
            f.write(mutated)
        so = os.path.join(d, "liboracle.so")
        subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
                        "-pthread", "-o", so, os.path.join(d, "oracle.c"), "-lm"], check=True)
        env = dict(os.environ, ORACLE_SO=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"]
                           + nodes, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived:\n{r.stdout[-2000:]}"
