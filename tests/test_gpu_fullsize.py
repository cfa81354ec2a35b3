"""Parity at the full sizes of the standard workloads, in the launch
configuration the benchmark times.  The GPU computes every head; the oracle
recomputes a sample of heads (each over its whole sequence), and every output
element of those heads is compared."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import TOL, assert_overlapped_ok, check, gpu_prefill, have_gpu, log, oracle_prefill

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _run(name, heads, overlapped=False):
    w = synth.workload_prefill(name)
    log("full-size %s: T=%d H=%d, oracle heads %s" % (name, w.total_tokens, w.num_heads, heads))
    o, S = gpu_prefill(w)
    if overlapped:
        assert_overlapped_ok()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    hs = list(range(w.num_heads)) if heads is None else heads
    o_ref, S_ref = oracle_prefill(w, heads=hs)
    check("o (%d heads)" % len(hs), o[:, hs], o_ref, TOL[w.io_dtype])
    check("S_T (%d heads)" % len(hs), S[:, hs], S_ref, TOL[w.io_dtype])


def test_batch4x4096_all_heads():
    _run("batch4x4096_bf16", None)


def test_long131072_sampled_heads():
    _run("long131072_bf16", [0, 5, 17, 31], overlapped=True)


def test_varlen64_sampled_heads():
    _run("varlen64_bf16", [3, 22])
