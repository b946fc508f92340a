"""Plant plausible mistakes in a copy of the oracle and check that the pins catch
each one: a dropped term, a wrong sign, a wrong index or operand, a misplaced gate.
The mistakes are planted in the oracle, on the CPU, in a temporary copy; the real
oracle is untouched."""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))

MUTANTS = {
    "decay_dropped": ("            double g = exp(lg[t]);\n", "            double g = 1.0;\n"),
    "decay_gate_off_by_one": ("            double g = exp(lg[t]);\n",
                              "            double g = exp(lg[t > 0 ? t - 1 : 0]);\n"),
    "gdn_sign": ("a * (S[i * dv + j] - b * kt[i] * r[j])", "a * (S[i * dv + j] + b * kt[i] * r[j])"),
    "gdn_beta_dropped_on_write": ("+ b * kt[i] * vt[j];", "+ kt[i] * vt[j];"),
    "gdn_alpha_on_write": ("a * (S[i * dv + j] - b * kt[i] * r[j]) + b * kt[i] * vt[j];",
                           "a * (S[i * dv + j] - b * kt[i] * r[j] + b * kt[i] * vt[j]);"),
    "gdn_retrieve_with_query": ("for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * kt[i];",
                                "for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i];"),
    "normalizer_wrong_operand": ("for (long i = 0; i < dk; ++i) z[i] += kt[i];",
                                 "for (long i = 0; i < dk; ++i) z[i] += qt[i];"),
    "normalizer_dropped": ("for (long j = 0; j < dv; ++j) ot[j] /= den;", "(void)den;"),
    "state_in_ignored": ("for (long i = 0; i < dk * dv; ++i) S[i] = s_in ? s_in[i] : 0.0;",
                         "for (long i = 0; i < dk * dv; ++i) S[i] = 0.0;"),
    "plain_transposed_write": ("S[i * dv + j] += kt[i] * vt[j];", "S[i * dv + j] += kt[j % dk] * vt[i % dv];"),
    "readout_uses_key": ("acc += S[i * dv + j] * qt[i];\n            ot[j] = acc;",
                         "acc += S[i * dv + j] * kt[i];\n            ot[j] = acc;"),
    "vector_gate_channel_reversed": ("double g = exp(lg[t * dk + i]);",
                                     "double g = exp(lg[t * dk + (dk - 1 - i)]);"),
    "vector_gate_one_token_late": ("double g = exp(lg[t * dk + i]);",
                                   "double g = exp(lg[(t > 0 ? t - 1 : 0) * dk + i]);"),
    "kda_gate_dropped": ("for (long j = 0; j < dv; ++j) S[i * dv + j] *= ai;", "(void)ai;"),
    "kda_gate_of_channel_zero": ("const double ai = exp(lg[t * dk + i]);", "const double ai = exp(lg[t * dk]);"),
    "kda_write_sign": ("S[i * dv + j] += bk * kt[i] * (vt[j] - r[j]);", "S[i * dv + j] += bk * kt[i] * (vt[j] + r[j]);"),
    "kda_retrieve_before_decay": ("for (long i = 0; i < dk; ++i) rj += kt[i] * S[i * dv + j];",
                                  "for (long i = 0; i < dk; ++i) rj += kt[i] * S[i * dv + j] / exp(lg[t * dk + i]);"),
    "bwd_dq_reads_old_state": ("for (long j = 0; j < dv_; ++j) acc += Sa[i * dv_ + j] * dot[j];",
                               "for (long j = 0; j < dv_; ++j) acc += Sb[i * dv_ + j] * dot[j];"),
    "bwd_state_grad_not_decayed": ("for (long i = 0; i < D; ++i) dS[i] *= g;", "(void)g;"),
    "bwd_gate_grad_without_gate": ("if (dlg) dlg[t] = g * acc;", "if (dlg) dlg[t] = acc;"),
    "bwd_dv_transposed": ("for (long i = 0; i < dk_; ++i) acc += dS[i * dv_ + j] * kt[i];",
                          "for (long i = 0; i < dk_; ++i) acc += dS[(i % dv_) * dv_ + (j % dk_)] * kt[i];"),
    "bwd_gdn_dk_missing_state_term": ("dk[t * dk_ + i] = b * gv - a * b * (gr + sgk);",
                                      "dk[t * dk_ + i] = b * gv - a * b * gr;"),
    "bwd_gdn_dbeta_without_retrieval": ("db += Gk[j] * (vt[j] - a * r[j]);", "db += Gk[j] * vt[j];"),
    "bwd_gdn_state_grad_no_projection": ("G[i * dv_ + j] = a * (G[i * dv_ + j] - b * kt[i] * Gk[j]);",
                                         "G[i * dv_ + j] = a * G[i * dv_ + j];"),
    "bwd_gdn_gate_grad_sign": ("if (dlg) dlg[t] = a * (gs - b * gkr);", "if (dlg) dlg[t] = a * (gs + b * gkr);"),
    "bwd_gdn_dv_without_beta": ("dv[t * dv_ + j] = b * gk;", "dv[t * dv_ + j] = gk;"),
    "conv_taps_reversed": ("acc += w[(h * d + c) * K + tau] * hist[(W + t - tau) * d + c];",
                           "acc += w[(h * d + c) * K + (K - 1 - tau)] * hist[(W + t - tau) * d + c];"),
    "conv_head_weights_shared": ("acc += w[(h * d + c) * K + tau]", "acc += w[c * K + tau]"),
    "conv_window_ignored": ("hist[j * d + c] = state_in ? state_in[(bh * W + j) * d + c] : 0.0;",
                            "hist[j * d + c] = 0.0;"),
    "conv_window_out_stale": ("state_out[(bh * W + j) * d + c] = hist[(L + j) * d + c];",
                              "state_out[(bh * W + j) * d + c] = hist[(L + j - (L > 0)) * d + c];"),
    "exclusive_mask": ("double *ot = o + t * dv;\n",
                       "double *ot = o + t * dv;\n        if (t > 0) { for (long j = 0; j < dv; ++j) { double acc = 0.0; for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i]; ot[j] = acc; } }\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {name}"
    if name == "exclusive_mask":
        # The output is read before the update (strict mask j < t); the read-out
        # below the update is disabled.
        src = src.replace("for (long j = 0; j < dv; ++j) {\n            double acc = 0.0;\n"
                          "            for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i];",
                          "for (long j = 0; j < 0; ++j) {\n            double acc = 0.0;\n"
                          "            for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i];")
    n_before = src.count(old)
    src = src.replace(old, new)
    assert n_before == 1 and src.count(new) >= 1
    msrc = tmp_path / "oracle_mutant.c"
    msrc.write_text(src)
    lib = obuild.build(src=str(msrc), out=str(tmp_path / "liboracle_mutant.so"))
    res = subprocess.run([sys.executable, os.path.join(HERE, "pin_runner.py"), lib],
                         capture_output=True, text=True, timeout=300)
    fails = [l for l in res.stdout.splitlines() if l.startswith("FAIL")]
    crashed = res.returncode != 0
    assert fails or crashed, f"mutant {name} passed every pin:\n{res.stdout}"
