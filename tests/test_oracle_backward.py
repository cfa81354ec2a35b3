"""The oracle's backward pass against its pins (finite differences of the
pinned forward map, Euler identities, the beta = 0 closed forms, split and
resume), and broken copies of it that the pins must catch.  CPU only."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import oracle_bwd_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")


@pytest.mark.parametrize("pin", P.ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin):
    pin(oracle.backward, oracle.prefill)


def test_bwd_threads_and_packing_are_bitwise():
    """One thread or many, packed or one sequence at a time: same bits."""
    c = P._case(34, [5, 0, 13, 1])
    g1 = P._grads(lambda *a: oracle.backward(*a, threads=1), c)
    g4 = P._grads(lambda *a: oracle.backward(*a, threads=4), c)
    for name in g1:
        assert np.array_equal(g1[name], g4[name])
    cu = c["cu"]
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        gn = oracle.backward(c["q"][s:e], c["k"][s:e], c["v"][s:e], c["la"][s:e], c["b"][s:e], [0, e - s],
                             c["S0"][n:n + 1], c["dO"][s:e], c["dST"][n:n + 1])
        for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
            assert np.array_equal(gn[name], g1[name][s:e])
        assert np.array_equal(gn["dS0"][0], g1["dS0"][n])


def test_bwd_no_state_cotangent_and_empty():
    """dS_T = None is a zero cotangent; an empty sequence passes dS_T to dS0."""
    c = P._case(35, [6, 0])
    z = dict(c)
    z["dST"] = np.zeros_like(c["dST"])
    gz = P._grads(oracle.backward, z)
    c["dST"] = None
    gn = P._grads(oracle.backward, c)
    for name in gz:
        assert np.array_equal(gz[name], gn[name])
    c2 = P._case(36, [0])
    g2 = P._grads(oracle.backward, c2)
    assert np.array_equal(g2["dS0"], c2["dST"])


# (name, original text, replacement) in the backward section of the C file
MUTANTS = [
    ("dla_from_undecayed", "acc += G[(size_t)i * dv + j] * Sd[(size_t)i * dv + j];",
     "acc += G[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];"),
    ("no_erase_cotangent", "G[(size_t)i * dv + j] -= kt[i] * de[j]; /* G is now dSd */", "/* dropped */"),
    ("dq_from_decayed", "acc += St[(size_t)i * dv + j] * dot[j];", "acc += Sd[(size_t)i * dv + j] * dot[j];"),
    ("state_cotangent_not_decayed", "G[(size_t)i * dv + j] *= a;\n", "(void)a;\n"),
    ("dbeta_sign", "db += acc * e[j];", "db -= acc * e[j];"),
    ("dk_missing_readback", "dkt[i] += acc;", "(void)acc;"),
    ("dv_sign", "dvt[j] = de[j];", "dvt[j] = -de[j];"),
    ("dk_without_beta", "dkt[i] = bt * acc;", "dkt[i] = acc;"),
    ("no_output_cotangent",  # the q dO^T term of the state cotangent dropped
     "          G[(size_t)i * dv + j] += qt[i] * dot[j];\n", "          G[(size_t)i * dv + j] += 0.0 * qt[i];\n"),
    ("checkpoint_state_shifted", "const double *Sp = span + (size_t)(t - t0) * SZ;     /* S_{t-1} */",
     "const double *Sp = span + (size_t)(t - t0 + (t > t0)) * SZ;"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    so = tmp_path / (name + ".so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", str(path), "-o", str(so), "-lm"],
                   check=True)
    return oracle.load_library(str(so))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_bwd_mutant_fails_a_pin(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)

    def backward(*a, **kw):
        return oracle.backward(*a, lib=lib, **kw)

    caught = []
    for pin in P.ALL_BWD_PINS:
        try:
            pin(backward, oracle.prefill)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name
