"""Backward pass on the GPU against the fp64 oracle's backward (reverse-mode
through the token recurrence), every element of every gradient: dq, dk, dv,
dlog_alpha, dbeta, dS0.  Shapes span several chunks with ragged tails, empty
and one-token sequences, both io dtypes, all head-dim pairs, the three gate
forms and gates far outside the range a plain per-chunk factorisation could
hold."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import check, dev, have_gpu, host, log, torch_mod

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

# Error budget (global max |err| / max |ref| per gradient).  fp32 io: every
# product is formed in fp32 (fp32 MFMA, fp32 exponentials); bf16 io: dq, dk,
# dv are rounded to bf16 on output (relative 2^-9 each), the rest is fp32.
TOL = {"f32": 1e-4, "bf16": 1e-2}


def gpu_backward(w, cot, S0=None, dS_T="w", want_dS0=True):
    import gated_delta_rule_33_amd as kda
    torch = torch_mod()
    dt = w.io_dtype
    la = dev(w.log_alpha) if w.log_alpha is not None else None
    s0 = w.S0 if S0 is None else S0
    dst = cot.dS_T if isinstance(dS_T, str) else dS_T
    g = kda.prefill_backward(dev(w.q, dt), dev(w.k, dt), dev(w.v, dt), la, dev(w.beta), dev(w.cu_seqlens),
                             dev(s0) if s0 is not None else None, dev(cot.dO, dt),
                             dev(dst) if dst is not None else None, want_dS0=want_dS0,
                             cu_seqlens_host=w.cu_seqlens.tolist())
    torch.cuda.synchronize()
    return {k_: (host(v_) if v_ is not None else None) for k_, v_ in g.items()}


def oracle_backward(w, cot, S0=None, dS_T="w"):
    s0 = w.S0 if S0 is None else S0
    dst = cot.dS_T if isinstance(dS_T, str) else dS_T
    g = oracle.backward(w.q, w.k, w.v, w.log_alpha_channels(), w.beta, w.cu_seqlens, s0, cot.dO, dst)
    if w.gate == "scalar":
        g["dlog_alpha"] = g["dlog_alpha"].sum(axis=-1)
    elif w.gate == "none":
        g["dlog_alpha"] = None
    return g


def compare(got, ref, tol, label=""):
    errs = {}
    for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"):
        if ref[name] is None:
            assert got[name] is None, name
            continue
        errs[name] = check(label + name, got[name], ref[name], tol)
    return errs


CASES = [
    # (lengths, H, dk, dv, io, gate, S0_std, seed)
    ([130, 0, 70, 1], 2, 64, 64, "f32", "channel", 0.5, 1),
    ([200, 64], 2, 128, 128, "f32", "channel", 0.5, 2),
    ([129], 3, 128, 64, "f32", "channel", None, 3),
    ([65, 191], 2, 64, 128, "f32", "channel", 0.5, 4),
    ([130, 0, 70, 1], 2, 128, 128, "bf16", "channel", 0.5, 5),
    ([300], 2, 64, 64, "bf16", "channel", 0.5, 6),
    ([150, 33], 2, 128, 128, "f32", "scalar", 0.5, 7),
    ([150, 33], 2, 128, 128, "bf16", "scalar", 0.5, 8),
    ([150, 33], 2, 128, 128, "f32", "none", 0.5, 9),
    ([100], 2, 64, 64, "bf16", "none", None, 10),
]


@pytest.mark.parametrize("lengths,H,dk,dv,io,gate,s0std,seed", CASES,
                         ids=["%s-%dx%d-%s-%s-%s" % ("_".join(map(str, c[0])), c[2], c[3], c[4], c[5], c[7])
                              for c in CASES])
def test_backward_matches_oracle(lengths, H, dk, dv, io, gate, s0std, seed):
    log("backward parity: lengths %s H %d dk %d dv %d %s gate %s S0 %s" % (lengths, H, dk, dv, io, gate, s0std))
    w = synth.make_prefill(lengths, H, dk, dv, io, seed, S0_std=s0std, gate=gate)
    cot = synth.make_cotangents(w, seed + 100)
    compare(gpu_backward(w, cot), oracle_backward(w, cot), TOL[io])


@pytest.mark.parametrize("la_kind", ["const-11", "const-60", "mixed-30", "const-3.7"])
def test_backward_extreme_gates(la_kind):
    """Constant log alpha of -11 and -60 per token (a 16-token block decays by
    e^-176 and e^-960: far past fp32), half the channels at -30, the rest at 0
    (no decay), and -3.7 (a 16-token block decays by e^-59.2, just inside the
    range where a block's own products use operands scaled at the row before
    it, so the column factors reach e^59): exact for every finite gate."""
    log("backward gates: %s" % la_kind)
    w = synth.make_prefill([150, 70], 2, 64, 64, "f32", 11, S0_std=0.5)
    if la_kind.startswith("const-"):
        w.log_alpha[:] = -float(la_kind[len("const-"):])
    else:
        w.log_alpha[:] = 0.0
        w.log_alpha[:, :, ::2] = -30.0
    cot = synth.make_cotangents(w, 111)
    compare(gpu_backward(w, cot), oracle_backward(w, cot), TOL["f32"])


def test_backward_beta_extremes_and_no_state():
    """beta = 0 on some tokens and 1 on others; no S0 and no dS_T."""
    log("backward: beta in {0, 1}, no S0, no dS_T")
    w = synth.make_prefill([90, 40], 2, 128, 128, "f32", 12)
    w.beta[::3] = 0.0
    w.beta[1::3] = 1.0
    cot = synth.make_cotangents(w, 112, dS_T_std=None)
    compare(gpu_backward(w, cot), oracle_backward(w, cot), TOL["f32"])


def test_backward_without_dS0_and_empty_batch():
    """dS0 may be skipped; a batch of only empty sequences passes dS_T to dS0."""
    log("backward: dS0 skipped; all-empty batch")
    w = synth.make_prefill([77], 2, 64, 64, "f32", 13, S0_std=0.5)
    cot = synth.make_cotangents(w, 113)
    got = gpu_backward(w, cot, want_dS0=False)
    ref = oracle_backward(w, cot)
    assert got["dS0"] is None
    for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
        check(name, got[name], ref[name], TOL["f32"])
    w0 = synth.make_prefill([0, 0], 2, 64, 64, "f32", 14, S0_std=0.5)
    c0 = synth.make_cotangents(w0, 114)
    g0 = gpu_backward(w0, c0)
    assert np.array_equal(g0["dS0"], c0.dS_T.astype(np.float64))


def test_backward_deterministic():
    log("backward: two calls, same bits")
    w = synth.make_prefill([300, 17], 4, 128, 128, "bf16", 15, S0_std=0.1)
    cot = synth.make_cotangents(w, 115)
    a, b = gpu_backward(w, cot), gpu_backward(w, cot)
    for name in a:
        assert np.array_equal(a[name], b[name]), name


def test_backward_4096_tokens_bf16():
    """One 4096-token sequence (64 chunks), 4 heads, dk = dv = 128, bf16,
    with S0 and dS_T: the reverse state chain over many chunks."""
    log("backward: 1 x 4096 x 4 heads bf16")
    w = synth.make_prefill([4096], 4, 128, 128, "bf16", 16, S0_std=0.05)
    cot = synth.make_cotangents(w, 116, dS_T_std=0.1)
    compare(gpu_backward(w, cot), oracle_backward(w, cot), TOL["bf16"])


def test_backward_varlen_many_items_bf16():
    """Three ragged sequences (2500, 1700, 900 tokens: 82 chunks), 6 heads,
    bf16: more (chunk, head) items than a GPU has CUs, so the persistent
    workgroups each take several items in turn, across sequence and head
    boundaries."""
    log("backward: lengths [2500, 1700, 900] x 6 heads bf16")
    w = synth.make_prefill([2500, 1700, 900], 6, 128, 128, "bf16", 17, S0_std=0.05)
    cot = synth.make_cotangents(w, 117, dS_T_std=0.1)
    compare(gpu_backward(w, cot), oracle_backward(w, cot), TOL["bf16"])
