"""Plant plausible mistakes in a copy of the C oracle and check that the pin
suite catches every one.  The oracle file itself is never modified: each
mutant is a text substitution compiled into a temporary library."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

# (name, original text, replacement).  Each original must occur exactly once.
MUTANTS = [
    ("readback_undecayed",  # read back before the decay (the loose paraphrase's order)
     "    /* forget: row i of S (key channel i) is scaled by alpha_t[i] */\n"
     "    for (int i = 0; i < dk; ++i) {\n"
     "      const double a = exp(lat[i]);\n"
     "      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;\n"
     "    }\n"
     "    /* read back the decayed state along k_t */\n"
     "    for (int j = 0; j < dv; ++j) r[j] = 0.0;\n"
     "    for (int i = 0; i < dk; ++i)\n"
     "      for (int j = 0; j < dv; ++j) r[j] += S[(size_t)i * dv + j] * kt[i];\n",
     "    for (int j = 0; j < dv; ++j) r[j] = 0.0;\n"
     "    for (int i = 0; i < dk; ++i)\n"
     "      for (int j = 0; j < dv; ++j) r[j] += S[(size_t)i * dv + j] * kt[i];\n"
     "    for (int i = 0; i < dk; ++i) {\n"
     "      const double a = exp(lat[i]);\n"
     "      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;\n"
     "    }\n"),
    ("delta_sign", "bt * kt[i] * (vt[j] - r[j])", "bt * kt[i] * (vt[j] + r[j])"),
    ("drop_beta", "bt * kt[i] * (vt[j] - r[j])", "kt[i] * (vt[j] - r[j])"),
    ("beta_only_on_write", "bt * kt[i] * (vt[j] - r[j])", "kt[i] * (bt * vt[j] - r[j])"),
    ("gate_not_exponentiated", "const double a = exp(lat[i]);", "const double a = 1.0 + lat[i];"),
    ("gate_squared", "const double a = exp(lat[i]);", "const double a = exp(2.0 * lat[i]);"),
    ("readback_with_q", "r[j] += S[(size_t)i * dv + j] * kt[i];", "r[j] += S[(size_t)i * dv + j] * qt[i];"),
    ("output_with_k", "ot[j] += S[(size_t)i * dv + j] * qt[i];", "ot[j] += S[(size_t)i * dv + j] * kt[i];"),
    ("ignore_S0", "  if (J->S0) {\n", "  if (0) {\n"),
    ("output_before_write",
     "    /* erase-then-write: add beta k (v - r)^T */\n"
     "    for (int i = 0; i < dk; ++i)\n"
     "      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bt * kt[i] * (vt[j] - r[j]);\n"
     "    /* output from the updated state */\n"
     "    for (int j = 0; j < dv; ++j) ot[j] = 0.0;\n"
     "    for (int i = 0; i < dk; ++i)\n"
     "      for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)i * dv + j] * qt[i];\n",
     "    for (int j = 0; j < dv; ++j) ot[j] = 0.0;\n"
     "    for (int i = 0; i < dk; ++i)\n"
     "      for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)i * dv + j] * qt[i];\n"
     "    for (int i = 0; i < dk; ++i)\n"
     "      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bt * kt[i] * (vt[j] - r[j]);\n"),
    ("gate_one_token_late", "const double *lat = J->la + ((size_t)t * H + h) * dk;",
     "const double *lat = J->la + ((size_t)(t > 0 ? t - 1 : 0) * H + h) * dk;"),
    ("decay_skips_last_channel", "    for (int i = 0; i < dk; ++i) {\n      const double a",
     "    for (int i = 0; i < dk - 1; ++i) {\n      const double a"),
]


def _build_mutant(tmp_path, name, old, new):
    # the mutants target the forward recurrence; the backward section that
    # follows it in the same file (with its own copy of the token step) is
    # left alone
    src = open(SRC).read()
    cut = src.index("/*\n * Backward pass")
    head, tail = src[:cut], src[cut:]
    assert head.count(old) == 1, name
    path = tmp_path / (name + ".c")
    path.write_text(head.replace(old, new) + tail)
    so = tmp_path / (name + ".so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", str(path), "-o", str(so), "-lm"],
                   check=True)
    return oracle.load_library(str(so))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_mutant_fails_a_pin(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)

    def prefill(*args, **kw):
        return oracle.prefill(*args, lib=lib, **kw)

    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(prefill)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name
