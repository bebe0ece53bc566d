"""The pins must be strong enough to catch plausible mistakes in the oracle.

Each case compiles a copy of the oracle with one planted mistake (a dropped
term, a wrong sign, a transposed index, a wrong gradient point, ...) into a
temporary directory, runs the pin tests against it in a subprocess, and
requires that at least one pin fails.  Everything runs on the CPU; the real
oracle source is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ttt_oracle.c")

MUTANTS = {
    "update_sign": ("S[i] -= eta * G[i];", "S[i] += eta * G[i];"),
    "output_before_update": (
        "ttt_oracle_linear_apply(d, c->use_ln, c->use_residual, c->ln_eps, S,",
        "ttt_oracle_linear_apply(d, c->use_ln, c->use_residual, c->ln_eps, Sb,"),
    "loss_factor_2_dropped": ("gy[j] = 2.0 * r;", "gy[j] = r;"),
    "ln_bwd_xhat_term_dropped": ("gh[j] = (a - ma - xhat[j] * max) / st.sigma;",
                                 "gh[j] = (a - ma) / st.sigma;"),
    "grad_transposed": ("gW[(size_t)i * d + j] = k[i] * gh[j];",
                        "gW[(size_t)j * d + i] = k[i] * gh[j];"),
    "grad_at_running_state": ("Sb, kk, vv, gam, bet, G);", "S, kk, vv, gam, bet, G);"),
    "unbiased_variance": ("var /= d;", "var /= (d - 1);"),
    "gelu_grad_sign": ("+ x * inv_sqrt_2pi", "- x * inv_sqrt_2pi"),
    "mlp_w2_grad_pre_ln": ("gW2[(size_t)n * d + j] = a[n] * go[j];",
                           "gW2[(size_t)n * d + j] = a[n] * gy[j];"),
    "mlp_bias1_not_state": ("for (int n = 0; n < m; ++n) gb1[n] = gp[n];",
                            "for (int n = 0; n < m; ++n) gb1[n] = 0.0;"),
    "minibatch_boundary_off_by_one": ("int t1 = t0 + bsz < T ? t0 + bsz : T;",
                                      "int t1 = t0 + bsz + 1 < T ? t0 + bsz + 1 : T;"),
    "residual_uses_v": ("double r = (use_residual ? k[j] : 0.0) + y[j] - v[j];",
                        "double r = (use_residual ? v[j] : 0.0) + y[j] - v[j];"),
}

PIN_FILES = ["tests/test_oracle_linear.py", "tests/test_oracle_mlp.py"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor vanished: " + name
    mutated = src.replace(old, new)
    shutil.copy(os.path.join(ROOT, "oracle", "ttt_oracle.h"), tmp_path / "ttt_oracle.h")
    (tmp_path / "ttt_oracle.c").write_text(mutated)
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(lib),
                           str(tmp_path / "ttt_oracle.c"), "-lm", "-lpthread"])
    env = dict(os.environ, TTT_ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"]
                       + PIN_FILES, cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, "no pin caught mutant %s:\n%s" % (name, r.stdout[-2000:])
