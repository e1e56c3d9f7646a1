"""Mutation check of the oracle's pins.

Each case copies oracle/oracle.c, plants one plausible mistake (a dropped term,
a wrong sign, a wrong index or mask, an operand swapped), builds the copy with
gcc and runs every pin of tests/oracle_pins.py against it in a subprocess.  The
pins must reject every mutant: at least one pin fails.  The real oracle is
never modified; the mutants live in a temporary directory.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "oracle_pins.py")

MUTANTS = [
    ("favor_drops_norm_term", "exp(s - 0.5 * xx)", "exp(s)"),
    ("favor_drops_inv_sqrt_M", "/ sqrt((double)M)", ""),
    ("favor_W_index_swapped", "W[(size_t)m * d + e] * x[e]", "W[(size_t)(e % M) * d + (m % d)] * x[e]"),
    ("elu_drops_plus_one", "x[j] + 1.0 : exp(x[j])", "x[j] : exp(x[j])"),
    ("elu_vjp_branches_swapped", "(x[j] > 0.0 ? 1.0 : exp(x[j]))", "(x[j] > 0.0 ? exp(x[j]) : 1.0)"),
    ("favor_vjp_sign", "(W[(size_t)m * d + e] - x[e])", "(W[(size_t)m * d + e] + x[e])"),
    ("quadratic_mask_excludes_diagonal",
     "for (long i = 0; i <= l; ++i) {\n            double a = dot(fq, Fk",
     "for (long i = 0; i < l; ++i) {\n            double a = dot(fq, Fk"),
    ("quadratic_ignores_R0", "num[e] += dot(R0 + (size_t)e * M, fq, M);", "num[e] += 0.0;"),
    ("prefix_state_uses_query_features", "R[(size_t)e * M + m] += v * fk[m];", "R[(size_t)e * M + m] += v * fq[m];"),
    ("bwd_drops_denominator_term", "double c = dot(g, V + (size_t)i * d, d) + E[l];",
     "double c = dot(g, V + (size_t)i * d, d);"),
    ("bwd_denominator_term_sign", "E[l] = -dot(", "E[l] = dot("),
    ("bwd_dV_wrong_row", "dV[(size_t)i * d + e] += a * g[e];", "dV[(size_t)l * d + e] += a * g[e];"),
    ("bwd_dR0_drops_dRout", "double s = dRout ? dRout[(size_t)e * M + m] : 0.0;", "double s = 0.0;"),
    ("prefix_bwd_grad_state_uses_key", "GR[(size_t)e * M + m] += g[e] * fq[m];",
     "GR[(size_t)e * M + m] += g[e] * fk[m];"),
    ("prefix_bwd_no_state_reversal", "R[(size_t)e * M + m] -= v[e] * fk[m];", "R[(size_t)e * M + m] -= 0.0;"),
    ("prefix_bwd_drops_dS", "double s = GS[m];", "double s = 0.0;"),
    ("wgrad_wrong_input_index", "dW[(size_t)m * d + e] += gm * x[e];",
     "dW[(size_t)m * d + e] += gm * x[(e + 1) % d];"),
    ("wgrad_drops_feature_factor", "const double gm = dphi[m] * phi[m];", "const double gm = dphi[m];"),
    ("quadratic_wgrad_keys_take_query_grad", "oracle_featmap_wgrad(L, d, M, K, W, dFk, dW);",
     "oracle_featmap_wgrad(L, d, M, K, W, dFq, dW);"),
    ("prefix_wgrad_skips_keys", "feat_wgrad_row(d, M, k, fk, dfk, dW);", "(void)0;"),
    ("softmax_half_temperature", "double p = exp(s[i] - mx);", "double p = exp(0.5 * (s[i] - mx));"),
    ("rows_mask_excludes_diagonal",
     "for (long i = 0; i <= l; ++i) {\n            feat_row(kind, d, M, K",
     "for (long i = 0; i < l; ++i) {\n            feat_row(kind, d, M, K"),
]


def _run_mutant(tmp, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mut = src.replace(old, new, 1)
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    open(c, "w").write(mut)
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-o", so, c, "-lm"])
    r = subprocess.run([sys.executable, PINS, so], capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-400:]


def test_every_mutant_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
            res = list(ex.map(lambda m: (m[0],) + _run_mutant(tmp, *m), MUTANTS))
    survivors = [(n, out) for n, rc, out in res if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"


def test_unmutated_copy_passes():
    with tempfile.TemporaryDirectory() as tmp:
        rc, out = _run_mutant(tmp, "identity", "#include <math.h>", "#include <math.h>")
    assert rc == 0, out
