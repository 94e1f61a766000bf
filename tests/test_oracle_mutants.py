"""The oracle pins must catch plausible mistakes: each case below plants one
mistake in a copy of oracle/pisa_oracle.c (never in the original), builds the
copy with gcc and runs tests/test_oracle_pins.py against it, which must fail."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pisa_oracle.c")

# (name, text in the original, replacement)
MUTANTS = [
    ("eligibility_strict", "if (A[k] * span <= t)", "if (A[k] * span < t)"),
    ("leaf_mean_over_C", "lev1[i * d + e] = s / (double)(hi - lo);", "lev1[i * d + e] = s / (double)C;"),
    ("node_mean_over_g", "dst[i * d + e] = s / (double)(hi - lo);", "dst[i * d + e] = s / (double)g;"),
    ("no_scale", "double scale = 1.0 / sqrt((double)P->d);\n    if (l == 1)",
     "double scale = 1.0;\n    if (l == 1)"),
    ("lse_is_max", "return m + log(s);", "return m;"),
    ("tie_higher_index", "return (x->i < y->i) ? -1 : (x->i > y->i);",
     "return (x->i > y->i) ? -1 : (x->i < y->i);"),
    ("no_previous_block", "if (c >= 1) cand[nc++] = (c - 1) / den;", ""),
    ("group_mean", "u += orc_lse_score(P, P->item_b[item], h, q, l, i);",
     "u += orc_lse_score(P, P->item_b[item], h, q, l, i) / G;"),
    ("drop_last_child", "int64_t lo = i * P->g, hi = i * P->g + P->g < P->M[l - 1] ? i * P->g + P->g : P->M[l - 1];",
     "int64_t lo = i * P->g, hi = i * P->g + P->g - 1 < P->M[l - 1] ? i * P->g + P->g - 1 : P->M[l - 1];"),
    ("forced_outside_budget", "int keep = Kt - nF;\n            nI = 0;", "int keep = Kt;\n            nI = 0;"),
    ("keep_all_strict", "if (nA <= Kt) {", "if (nA < Kt) {"),
    ("bsa_unnormalised", "S[k].u += exp(z[k] - lz);", "S[k].u += z[k];"),
    ("attn_mask_self", "if (P->causal && j > t) continue;", "if (P->causal && j >= t) continue;"),
    ("wrong_children", "int64_t lo = I[k] * P->g;", "int64_t lo = I[k] * P->g + 1;"),
    ("transposed_operand", "for (int e = 0; e < d; e++) s += (double)q[e] * k[e];",
     "for (int e = 0; e < d; e++) s += (double)q[e] * k[d - 1 - e];"),
    ("pisa1_sum_not_mean", "    return s / (double)n;\n}\n\n/* Population", "    return s;\n}\n\n/* Population"),
    ("pisa2_sample_variance", "s += (z[j] - mu) * (z[j] - mu);\n    return s / (double)n;",
     "s += (z[j] - mu) * (z[j] - mu);\n    return s / (double)(n > 1 ? n - 1 : 1);"),
    ("pisa2_whole_variance", "return mean_of(z, n) + 0.5 * var_of(z, n);", "return mean_of(z, n) + var_of(z, n);"),
    ("pisa1_normalised_lse", "if (kind == 1) return mean_of(z, n);",
     "if (kind == 1) return logsumexp(z, n) - log((double)n);"),
    ("bwd_no_centering", "double dz = p * (dp[k] - pdp);", "double dz = p * dp[k];"),
    ("bwd_dk_unscaled", "P->dK[row + e] += dz * scale * (double)q[e];", "P->dK[row + e] += dz * (double)q[e];"),
    ("bwd_dv_unnormalised", "P->dV[row + e] += p * (double)dO[e];", "P->dV[row + e] += exp(z[k]) * (double)dO[e];"),
    ("bwd_saved_output_ignored", "if (P->Osaved) pdp = dot_ff(", "if (0) pdp = dot_ff("),
    ("quality_mass_not_normalised", "Pm[B] += exp(a[B] - la) / (double)G;", "Pm[B] += exp(a[B]) / (double)G;"),
    ("quality_recall_denominator", "P->recall[o] = (double)hit / (double)Kt;",
     "P->recall[o] = (double)hit / (double)(Kt + 1);"),
    ("quality_future_key", "if (hi > i + 1) hi = i + 1;", "if (hi > i + 2) hi = i + 2;"),
    ("bwd_mask_self", "if (P->causal && t < j) continue;", "if (P->causal && t <= j) continue;"),
    ("bsa_exp_unnormalised", "S[k].u += exp(z[k] - lz);", "S[k].u += exp(z[k]);"),
    ("bsa_forced_in_softmax", "        if (contains(F, nF, i)) continue;\n        S[ns].i = i;",
     "        S[ns].i = i;"),
    ("reach_no_cost", "double cl = mx - mn > 0.0 ? mx - mn : 0.0;", "double cl = 0.0;"),
    ("reach_last_level_cost", "double nc = cl > cost ? cl : cost;", "double nc = cl;"),
    ("reach_sure_in_without_band", "if (S[k].u > hi + R->cap) st[k] = 1;", "if (S[k].u > hi) st[k] = 1;"),
    ("reach_pool_too_narrow", "else if (S[k].u < lo - R->cap) st[k] = 0;", "else if (S[k].u < lo) st[k] = 0;"),
    ("ascending_scores", "if (x->u > y->u) return -1;\n    if (x->u < y->u) return 1;",
     "if (x->u < y->u) return -1;\n    if (x->u > y->u) return 1;"),
]


def _run(m, tmp):
    name, old, new = m
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = os.path.join(tmp, name + ".c")
    lib = os.path.join(tmp, name + ".so")
    open(path, "w").write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    path, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, PISA_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _run(m, tmp), MUTANTS))
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, "mutants not caught by the pins: %s" % survivors
