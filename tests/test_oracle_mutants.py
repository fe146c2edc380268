"""The oracle's pins must catch plausible mistakes in the oracle itself.

Each case copies ``oracle/kda_oracle.c``, plants one mistake (a dropped term,
a wrong sign, a wrong operand, a wrong order), compiles the copy on the CPU and
runs the pin suite against it in a subprocess; the suite has to fail.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

MUTANTS = {
    "no_decay": ("S[i * dv + j] *= a[i];", "S[i * dv + j] *= 1.0;"),
    "decay_sign": ("a[i] = exp(rd(g, in_type, qo + i));", "a[i] = exp(-rd(g, in_type, qo + i));"),
    "correction_sign": ("u[j] = b * (rd(v, in_type, vo + j) - p[j]);",
                        "u[j] = b * (rd(v, in_type, vo + j) + p[j]);"),
    "no_beta": ("u[j] = b * (rd(v, in_type, vo + j) - p[j]);",
                "u[j] = (rd(v, in_type, vo + j) - p[j]);"),
    "no_write": ("S[i * dv + j] += ki * u[j];", "S[i * dv + j] += 0.0 * ki * u[j];"),
    "predict_with_query": ("p[j] += S[i * dv + j] * ki;\n    }\n    /* delta-rule",
                           "p[j] += S[i * dv + j] * rd(q, in_type, qo + i);\n    }\n    /* delta-rule"),
    "no_gate": ("y[j] = sigmoid(rd(z, in_type, vo + j)) * (scale * p[j]);",
                "y[j] = (scale * p[j]);"),
    "no_scale": ("y[j] = sigmoid(rd(z, in_type, vo + j)) * (scale * p[j]);",
                 "y[j] = sigmoid(rd(z, in_type, vo + j)) * (p[j]);"),
    "read_with_key": ("double qi = rd(q, in_type, qo + i);", "double qi = rd(k, in_type, qo + i);"),
}


# planted mistakes in the backward; the backward pins have to catch them
BACKWARD_MUTANTS = {
    "bwd_no_prediction_term": ("const double dsd = dS[r * dv + j] + kr * dp[j];",
                               "const double dsd = dS[r * dv + j];"),
    "bwd_read_term_sign": ("dS[r * dv + j] += scale * qr * dov[j];",
                           "dS[r * dv + j] -= scale * qr * dov[j];"),
    "bwd_dg_without_decay": ("dg[qo + r] = a[r] * da;", "dg[qo + r] = da;"),
    "bwd_dbeta_without_prediction": ("db += du[j] * (vj - p[j]);", "db += du[j] * vj;"),
    "bwd_dk_without_prediction": ("dk_out[qo + r] += acc;", "dk_out[qo + r] += 0.0 * acc;"),
    "bwd_dz_gate_derivative": ("dz[vo + j] = dout[vo + j] * o * sg * (1.0 - sg);",
                               "dz[vo + j] = dout[vo + j] * o * sg;"),
}


def _run_pins_against(name, old, new, pin_file, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", str(mutant_c),
                    "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, KDA_ORACLE_LIB=str(lib))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", pin_file)],
                          env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    old, new = BACKWARD_MUTANTS[name]
    r = _run_pins_against(name, old, new, "test_oracle_backward.py", tmp_path)
    assert r.returncode != 0, f"backward pins did not catch mutant {name}:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", str(mutant_c),
                    "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, KDA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
