"""Planted mistakes in the oracle must be caught by its pins.

Each case copies fckl_oracle.c, changes one line the way a plausible slip would
(a dropped temperature, a flipped sign, a transposed operand, a wrong index),
builds the copy with gcc into a temporary directory and runs the pin suite
against it in a child process.  The pin suite must fail for every mutant.  The
oracle's own source is never modified.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "fckl_oracle.c")

MUTANTS = {
    "teacher_temperature_dropped": ("lp[k] = tl[k] / T - log_norm;", "lp[k] = tl[k] - log_norm;"),
    "kl_sign_flipped": ("kl += p[k] * (lp[k] - log_q);", "kl += p[k] * (lp[k] + log_q);"),
    "t_squared_dropped": ("loss_out[r] = T * T * kl;", "loss_out[r] = T * kl;"),
    "head_transposed": ("acc += h_row[j] * w[j];", "acc += h_row[j] * W[j * V + v];"),
    "gather_index_reversed": ("double log_q = z[idx[i * K + k]] / T - lse;",
                              "double log_q = z[idx[i * K + (K - 1 - k)]] / T - lse;"),
    "lse_temperature_dropped": ("s += exp(z[v] / T - m);", "s += exp(z[v] - m);"),
    "scatter_sign_flipped": ("gr[idx[i * K + k]] -= scale * p[k];", "gr[idx[i * K + k]] += scale * p[k];"),
    "grad_temperature_dropped": ("scale[r] = grad_scale * T / (double)n_norm;",
                                 "scale[r] = grad_scale / (double)n_norm;"),
    "dW_vocab_index_wrong": ("double gv = g[r * V + v];\n                const double *hr",
                             "double gv = g[r * V + (V - 1 - v)];\n                const double *hr"),
    "dH_uses_softmax_only": ("gr[v] = scale * psum * exp(z[v] / T - lse);",
                             "gr[v] = scale * psum * exp(z[v] - lse);"),
    "weighted_mean_over_count": ("s += w[i] * loss[i];\n        *mean_out = wsum > 0.0 ? s / wsum : 0.0;",
                                 "s += w[i] * loss[i];\n        *mean_out = wsum > 0.0 ? s / (double)N : 0.0;"),
    "full_gradient_sign_flipped": ("g[i * V + v] = scale * (exp(log_q) - p);",
                                   "g[i * V + v] = scale * (p - exp(log_q));"),
    "full_reverse_kl": ("kl += p * (log_p - log_q);", "kl += exp(log_q) * (log_q - log_p);"),
    "topk_ties_to_larger_index": ("return a->z > b->z || (a->z == b->z && a->v < b->v);",
                                  "return a->z > b->z || (a->z == b->z && a->v > b->v);"),
    "topk_ascending": ("return a->z > b->z || (a->z == b->z && a->v < b->v);",
                       "return a->z < b->z || (a->z == b->z && a->v < b->v);"),
    "topk_drops_last_slot": ("if (n == K && !rank_before(&c, &best[K - 1]))",
                             "if (n == K && !rank_before(&c, &best[K > 1 ? K - 2 : 0]))"),
    "weighted_grad_row_weight_dropped": ("scale[r] = wsum > 0.0 ? grad_scale * T * w[i] / wsum : 0.0;",
                                         "scale[r] = wsum > 0.0 ? grad_scale * T / wsum : 0.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    mut_src = tmp_path / "mutant.c"
    mut_src.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(mut_src), "-lm"], check=True)
    env = dict(os.environ, FCKL_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "planted mistake %s was not caught:\n%s" % (name, r.stdout[-2000:])
