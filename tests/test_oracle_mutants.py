"""Mutation test for the oracle's pins: each case plants one plausible mistake (a wrong
sign, a dropped term, an off-by-one mask, a swapped operand) into a copy of oracle.cpp,
builds it on the CPU, and requires the pin suite to fail against that build."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = {
    "rescale_sign": ("const double alpha = std::exp(m[r] - mn);",
                     "const double alpha = std::exp(mn - m[r]);"),
    "normalised_update_drops_l_ratio": ("sr[c] = sr[c] * (l[r] / ln) * alpha + pv / ln;",
                                        "sr[c] = sr[c] * alpha + pv / ln;"),
    "causal_off_by_one": ("return causal ? std::min(i + 1, L) : L;",
                          "return causal ? std::min(i, L) : L;"),
    "dot_drops_last_term": ("for (long c = 0; c < d; ++c) s += a[c] * b[c];",
                            "for (long c = 0; c + 1 < d; ++c) s += a[c] * b[c];"),
    "scale_dropped": ("sc[j] = scale * dot(qi, s.k + j * s.rs, d);",
                      "sc[j] = dot(qi, s.k + j * s.rs, d);"),
    "lse_drops_max": ("s.lse[i * s.ls] = m + std::log(l);", "s.lse[i * s.ls] = std::log(l);"),
    "ds_sign_dq": ("const double dS = P * (dP - Di);\n      const double* kj",
                   "const double dS = P * (dP + Di);\n      const double* kj"),
    "dq_uses_q": ("for (long c = 0; c < d; ++c) dqi[c] += dS * kj[c];",
                  "for (long c = 0; c < d; ++c) dqi[c] += dS * qi[c];"),
    "dk_scale_dropped": ("for (long c = 0; c < d; ++c) dkj[c] *= scale;", ""),
    "dv_uses_q": ("dvj[c] += P * doi[c];", "dvj[c] += P * qi[c];"),
    "dk_causal_range": ("for (long i = causal ? j : 0; i < s.L; ++i) {",
                        "for (long i = causal ? j + 1 : 0; i < s.L; ++i) {"),
    "varlen_lse_offset": ("lse + h * T + cu[s], H * d, 1, L};\n    fwd_rows",
                          "lse + h * T, H * d, 1, L};\n    fwd_rows"),
    "decode_causal_off_by_one": ("const long e = Nk - Nq + i + 1;", "const long e = Nk - Nq + i;"),
    "decode_top_left_mask": ("const long e = Nk - Nq + i + 1;", "const long e = i + 1;"),
    "merge_weight_sign": ("const double w = ls[t] * std::exp(ms[t] - m);",
                          "const double w = ls[t] * std::exp(m - ms[t]);"),
    "merge_drops_l": ("const double w = ls[t] * std::exp(ms[t] - m);",
                      "const double w = std::exp(ms[t] - m);"),
    "merge_lse_drops_max": ("lse = m + std::log(l);", "lse = std::log(l);"),
    "rows_dq_scale_dropped": ("for (long c = 0; c < d; ++c) dqr[c] *= scale;", ""),
    "tail_keys_skip_diagonal": ("for (long r = c; r < R; ++r) {",
                                "for (long r = c + 1; r < R; ++r) {"),
}


def _run_mutant(name, tmpdir):
    old, new = MUTANTS[name]
    with open(os.path.join(ROOT, "oracle", "oracle.cpp"), encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    lib = obuild.build_from_text(src.replace(old, new), os.path.join(tmpdir, f"lib_{name}.so"))
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda n: _run_mutant(n, str(tmp_path)), MUTANTS))
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"
