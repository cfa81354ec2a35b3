"""GPU parity of kda_prefill against the fp64 oracle, element by element on
the same seeded inputs, plus invariants (chunk-size independence, in-place
state, split/resume, decode equivalence, pure decay)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import (TOL, assert_not_recovered, check, dev, gpu_prefill, have_gpu, host, log,
                                oracle_prefill)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def test_tiny_f32_workload():
    """1 x 256 tokens, H=2, d=64, fp32, chunk 64, S0 = 0."""
    w = synth.workload_prefill("tiny_f32")
    log("prefill tiny_f32")
    o, S = gpu_prefill(w)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL["f32"])
    check("S_T", S, S_ref, TOL["f32"])


RAGGED = [1, 63, 64, 65, 200, 0, 31, 129]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("chunk", [64, 32, 16])
def test_ragged_varlen(dt, dk, dv, chunk):
    """Packed sequences of ragged lengths (incl. 0, 1, C-1, C, C+1) with a
    nonzero initial state."""
    log("prefill ragged dt=%s dk=%d dv=%d chunk=%d" % (dt, dk, dv, chunk))
    w = synth.make_prefill(RAGGED, H=3, dk=dk, dv=dv, io_dtype=dt, seed=11, S0_std=0.05, chunk=chunk)
    o, S = gpu_prefill(w)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL[dt])
    check("S_T", S, S_ref, TOL[dt])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_device_offsets_without_host_mirror(dt):
    w = synth.make_prefill([70, 0, 5, 300], H=2, dk=128, dv=128, io_dtype=dt, seed=12, S0_std=0.02)
    log("prefill no-host-offsets dt=%s" % dt)
    o, S = gpu_prefill(w, host_offsets=False)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL[dt])
    check("S_T", S, S_ref, TOL[dt])


def test_in_place_state_and_zero_tokens():
    w = synth.make_prefill([0, 0, 0], H=2, dk=64, dv=64, io_dtype="bf16", seed=13, S0_std=0.1)
    log("prefill all-empty in-place")
    o, S = gpu_prefill(w, in_place=True)
    assert o.shape == (0, 2, 64)
    assert np.array_equal(S, w.S0.astype(np.float64))
    w = synth.make_prefill([100, 37], H=2, dk=128, dv=128, io_dtype="bf16", seed=14, S0_std=0.1)
    o, S = gpu_prefill(w, in_place=True)
    o_ref, S_ref = oracle_prefill(w)
    check("o (in place)", o, o_ref, TOL["bf16"])
    check("S_T (in place)", S, S_ref, TOL["bf16"])


def test_chunk_size_independence_and_resume():
    """C = 16, 32 and 64 agree; a split at t then resume from S_t equals the whole."""
    w = synth.make_prefill([333], H=2, dk=128, dv=128, io_dtype="f32", seed=15, S0_std=0.05)
    log("prefill chunk independence + resume")
    o64, S64 = gpu_prefill(w, chunk=64)
    for c in (32, 16):
        oc, Sc = gpu_prefill(w, chunk=c)
        assert np.max(np.abs(o64 - oc)) <= 1e-4 * np.max(np.abs(o64)), c
        assert np.max(np.abs(S64 - Sc)) <= 1e-4 * np.max(np.abs(S64)), c
    t = 150
    a = synth.PrefillInputs(w.q[:t], w.k[:t], w.v[:t], w.log_alpha[:t], w.beta[:t], np.array([0, t], np.int32),
                            w.S0, "f32")
    oa, Sa = gpu_prefill(a)
    b = synth.PrefillInputs(w.q[t:], w.k[t:], w.v[t:], w.log_alpha[t:], w.beta[t:], np.array([0, 333 - t], np.int32),
                            Sa.astype(np.float32), "f32")
    ob, Sb = gpu_prefill(b)
    assert np.max(np.abs(np.concatenate([oa, ob]) - o64)) <= 1e-4 * np.max(np.abs(o64))
    assert np.max(np.abs(Sb - S64)) <= 1e-4 * np.max(np.abs(S64))


def test_pure_decay_closed_form_on_gpu():
    """beta = 0: o_t = S0^T (exp(g_t) q_t) for each sequence."""
    w = synth.make_prefill([150, 77], H=2, dk=128, dv=64, io_dtype="f32", seed=16, S0_std=0.3)
    w.beta[:] = 0.0
    log("prefill pure decay")
    o, S = gpu_prefill(w)
    for n in range(2):
        s, e = int(w.cu_seqlens[n]), int(w.cu_seqlens[n + 1])
        for h in range(2):
            g = np.cumsum(w.log_alpha[s:e, h].astype(np.float64), axis=0)
            ref = (np.exp(g) * w.q[s:e, h]) @ w.S0[n, h].astype(np.float64)
            check("o seq%d head%d" % (n, h), o[s:e, h], ref, 1e-4)


GATE_CASES = [
    # (name, per-channel log_alpha pattern); beta = 1
    ("all-5", "all", -5.0), ("all-11", "all", -11.0), ("all-20", "all", -20.0), ("all-60", "all", -60.0),
    ("half-8", "half", -8.0), ("half-30", "half", -30.0), ("half-60", "half", -60.0),
    ("spikes-1000", "spikes", -1000.0), ("spikes-1e4", "spikes", -1e4),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", GATE_CASES, ids=[c[0] for c in GATE_CASES])
def test_gate_decay_extremes(dt, case):
    """Any finite log_alpha <= 0: held constant on every channel ("all") or
    on every other channel with no decay on the rest ("half"), or a cfg-like
    gate with isolated huge decays (5% of the (token, channel) entries,
    "spikes").  Strong decay puts a diagonal 16-token block's decay beyond
    the fp32 range on the affected channels, so the prep forms those
    channels' ratios token by token."""
    name, pattern, la = case
    w = synth.make_prefill([200, 64, 17, 1], H=2, dk=128, dv=128, io_dtype=dt, seed=19, S0_std=0.05)
    if pattern == "half":
        w.log_alpha[:, :, 0::2] = la
        w.log_alpha[:, :, 1::2] = 0.0
    elif pattern == "all":
        w.log_alpha[:] = la
    else:
        rng = np.random.default_rng(190)
        w.log_alpha[rng.random(w.log_alpha.shape) < 0.05] = la
    w.beta[:] = 1.0
    log("prefill gate extremes dt=%s case=%s" % (dt, name))
    o, S = gpu_prefill(w)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL[dt])
    check("S_T", S, S_ref, TOL[dt])


def test_gate_extremes_long_overlapped():
    """A 200-chunk-index batch (overlapped schedule) whose gates mix the
    workload distribution with isolated decays of -200 and a block of
    channels at -30, bf16."""
    w = synth.make_prefill([9000, 4000], H=2, dk=128, dv=128, io_dtype="bf16", seed=31, S0_std=0.05)
    rng = np.random.default_rng(310)
    w.log_alpha[rng.random(w.log_alpha.shape) < 0.01] = -200.0
    w.log_alpha[:, :, 64:80] = -30.0
    log("prefill gate extremes, overlapped schedule")
    rep = {}
    o, S = gpu_prefill(w, report=rep)
    assert_not_recovered(rep)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL["bf16"])
    check("S_T", S, S_ref, TOL["bf16"])


def test_prefill_equals_decode_steps():
    """T tokens through prefill and T decode steps on the same values: both
    against the oracle, and against each other."""
    import torch
    import gated_delta_rule_33_amd as kda
    w = synth.make_prefill([70], H=4, dk=128, dv=128, io_dtype="bf16", seed=17, S0_std=0.05)
    log("prefill vs decode steps")
    o, S = gpu_prefill(w)
    Sd = dev(w.S0)
    outs = []
    for t in range(70):
        sl = slice(t, t + 1)
        outs.append(host(kda.decode_step(dev(w.q[sl], "bf16"), dev(w.k[sl], "bf16"), dev(w.v[sl], "bf16"),
                                         dev(w.log_alpha[sl]), dev(w.beta[sl]), Sd)))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(w)
    od = np.concatenate(outs)
    check("o prefill vs oracle", o, o_ref, TOL["bf16"])
    check("o decode steps vs oracle", od, o_ref, TOL["bf16"])
    check("S prefill vs oracle", S, S_ref, TOL["bf16"])
    check("S decode steps vs oracle", host(Sd), S_ref, TOL["bf16"])
    # and the two GPU paths against each other (each within the bound of the
    # oracle, so within twice the bound of each other)
    check("o prefill vs decode", o, od, 2 * TOL["bf16"])
    check("S prefill vs decode", S, host(Sd), 2 * TOL["bf16"])


def test_deterministic():
    w = synth.make_prefill([500, 3], H=2, dk=128, dv=128, io_dtype="bf16", seed=18, S0_std=0.02)
    o1, S1 = gpu_prefill(w)
    o2, S2 = gpu_prefill(w)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_many_pairs_wide_tiles():
    """Enough (sequence, head) pairs that the scan uses its wide value tiles."""
    rng = np.random.default_rng(19)
    lengths = [int(x) for x in rng.integers(0, 200, size=64)]
    w = synth.make_prefill(lengths, H=8, dk=128, dv=128, io_dtype="bf16", seed=19, S0_std=0.05)
    log("prefill many pairs: %d seqs x 8 heads" % len(lengths))
    o, S = gpu_prefill(w)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL["bf16"])
    check("S_T", S, S_ref, TOL["bf16"])


SEG_LENGTHS = [5000, 0, 3000, 777, 4096]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [64, 32, 16])
@pytest.mark.parametrize("mode", ["state", "nostate", "inplace"])
def test_segmented_schedule(dt, chunk, mode):
    """Few (sequence, head) pairs and 200+ chunk indices: one scan launch on
    half of the CUs beside the prep of 4 (chunk 64) or 7 (chunk 32) segments
    of 64 chunk indices on the other half.  Sequences straddle segment
    boundaries, so the scan waits on the segment counter mid-sequence; the
    final state is written to S_T, to S0 in place, or not at all."""
    import torch
    import gated_delta_rule_33_amd as kda
    log("prefill segmented dt=%s chunk=%d mode=%s" % (dt, chunk, mode))
    w = synth.make_prefill(SEG_LENGTHS, H=4, dk=128, dv=128, io_dtype=dt, seed=20, S0_std=0.05, chunk=chunk)
    o_ref, S_ref = oracle_prefill(w)
    rep = {}
    if mode == "state":
        o, S = gpu_prefill(w, report=rep)
    elif mode == "inplace":
        o, S = gpu_prefill(w, in_place=True, report=rep)
    else:
        o, S = gpu_prefill(w, want_state=False, report=rep)
        assert S is None
    assert_not_recovered(rep)
    check("o", o, o_ref, TOL[dt])
    if S is not None:
        check("S_T", S, S_ref, TOL[dt])


def test_segmented_schedule_many_segments():
    """674 chunk indices over 4 sequences x 2 heads: eleven segments of 64,
    with sequences (one of 3 tokens) straddling the boundaries."""
    lengths = [20000, 9000, 3, 14000]
    log("prefill segmented, 11 segments: %s x 2 heads" % lengths)
    w = synth.make_prefill(lengths, H=2, dk=128, dv=128, io_dtype="bf16", seed=23, S0_std=0.05)
    rep = {}
    o, S = gpu_prefill(w, report=rep)
    assert_not_recovered(rep)
    o_ref, S_ref = oracle_prefill(w)
    check("o", o, o_ref, TOL["bf16"])
    check("S_T", S, S_ref, TOL["bf16"])


def test_one_stream_schedule_is_bitwise_equal():
    """KDA_PREFILL_ONE_STREAM (every prep segment, then the scan, on the
    caller's stream) returns bitwise the same o and S_T as the overlapped
    two-stream schedule."""
    lengths = [5000, 0, 3000, 777, 4096]
    log("prefill one-stream vs overlapped schedule, %s x 4 heads" % lengths)
    w = synth.make_prefill(lengths, H=4, dk=128, dv=128, io_dtype="bf16", seed=20, S0_std=0.05)
    rep = {}
    o_ov, S_ov = gpu_prefill(w, report=rep)
    assert_not_recovered(rep)
    o_one, S_one = gpu_prefill(w, one_stream=True, report=rep)
    assert rep["recovered"] is False
    assert np.array_equal(o_one, o_ov)
    assert np.array_equal(S_one, S_ov)


@pytest.mark.parametrize("mode", ["state", "inplace", "nostate"])
def test_overlapped_recovery_path(mode):
    """The overlapped schedule's fail-safe: with the state pass's wait bound
    set to zero from the host, every loader wave gives up at its first
    unpublished segment (all kernels still run to their end), the call's
    guarded recovery launches recompute everything on the caller's stream,
    kda_prefill_recovered reports it, and the results match the oracle --
    including an in-place update, whose S0 must survive the abandoned pass."""
    import gated_delta_rule_33_amd as kda
    lengths = [5000, 0, 3000, 777, 4096]
    log("prefill overlapped recovery path mode=%s" % mode)
    w = synth.make_prefill(lengths, H=4, dk=128, dv=128, io_dtype="bf16", seed=21, S0_std=0.05)
    o_ref, S_ref = oracle_prefill(w)
    rep = {}
    prev = kda.set_wait_limit(0)
    try:
        if mode == "state":
            o, S = gpu_prefill(w, report=rep)
        elif mode == "inplace":
            o, S = gpu_prefill(w, in_place=True, report=rep)
        else:
            o, S = gpu_prefill(w, want_state=False, report=rep)
    finally:
        kda.set_wait_limit(prev)
    log("  recovered: %s" % rep["recovered"])
    assert rep["recovered"] is True
    check("o", o, o_ref, TOL["bf16"])
    if S is not None:
        check("S_T", S, S_ref, TOL["bf16"])
    # the next call, with the default bound, runs the overlapped schedule again
    o2, S2 = gpu_prefill(w, report=rep)
    assert_not_recovered(rep)
    check("o (after)", o2, o_ref, TOL["bf16"])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sequence_order_permutation(dt):
    """The same sequences packed in two different orders (so the chunk
    offsets, the longest-first processing order and the workgroups that
    take each (sequence, head) all change) give bitwise the same per-sequence
    o and S_T."""
    lengths = [300, 0, 1, 777, 64, 129, 2000, 65]
    w = synth.make_prefill(lengths, H=3, dk=128, dv=64, io_dtype=dt, seed=24, S0_std=0.05)
    perm = [6, 3, 0, 7, 2, 5, 1, 4]
    log("prefill sequence-order permutation dt=%s perm=%s" % (dt, perm))
    cu = w.cu_seqlens
    segs = [slice(int(cu[i]), int(cu[i + 1])) for i in range(len(lengths))]
    cat = lambda x: np.concatenate([x[segs[i]] for i in perm], axis=0)
    wp = synth.PrefillInputs(cat(w.q), cat(w.k), cat(w.v), cat(w.log_alpha), cat(w.beta),
                             np.concatenate([[0], np.cumsum([lengths[i] for i in perm])]).astype(np.int32),
                             w.S0[perm].copy(), dt)
    o, S = gpu_prefill(w)
    op, Sp = gpu_prefill(wp)
    cup = wp.cu_seqlens
    for j, i in enumerate(perm):
        assert np.array_equal(op[int(cup[j]):int(cup[j + 1])], o[segs[i]]), "sequence %d" % i
        assert np.array_equal(Sp[j], S[i]), "state %d" % i


def test_packed_equals_separate_calls():
    """A packed batch equals one call per sequence (bf16, 2 heads)."""
    lengths = [700, 3, 0, 1500]
    w = synth.make_prefill(lengths, H=2, dk=128, dv=128, io_dtype="bf16", seed=25, S0_std=0.05)
    log("prefill packed vs separate calls %s" % lengths)
    o, S = gpu_prefill(w)
    cu = w.cu_seqlens
    for i, L in enumerate(lengths):
        a, b = int(cu[i]), int(cu[i + 1])
        wi = synth.PrefillInputs(w.q[a:b], w.k[a:b], w.v[a:b], w.log_alpha[a:b], w.beta[a:b],
                                 np.array([0, L], np.int32), w.S0[i:i + 1].copy(), "bf16")
        oi, Si = gpu_prefill(wi)
        if L:
            assert np.max(np.abs(oi - o[a:b])) <= 1e-5 * max(np.max(np.abs(o[a:b])), 1e-30), i
        assert np.max(np.abs(Si[0] - S[i])) <= 1e-5 * np.max(np.abs(S[i])), i


def _random_cases(n: int, seed: int):
    """Seeded random small prefill shapes: ragged and empty sequences, lengths
    around chunk boundaries, every (dk, dv), both chunk sizes and io dtypes,
    with and without an initial state, in place or not."""
    rng = np.random.Generator(np.random.PCG64([seed]))
    edge = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129]
    cases = []
    for i in range(n):
        nseq = int(rng.integers(1, 7))
        lengths = [int(rng.choice(edge)) if rng.random() < 0.5 else int(rng.integers(0, 700)) for _ in range(nseq)]
        if sum(lengths) == 0:
            lengths[0] = 5
        cases.append(dict(lengths=lengths, H=int(rng.integers(1, 4)),
                          dk=int(rng.choice([64, 128])), dv=int(rng.choice([64, 128])),
                          chunk=int(rng.choice([16, 32, 64])), dt=str(rng.choice(["bf16", "f32"])),
                          s0=bool(rng.random() < 0.6), in_place=bool(rng.random() < 0.3), seed=100 + i))
    return cases


@pytest.mark.parametrize("case", _random_cases(16, 2024), ids=lambda c: "%s-%dx%d-c%d-%s%s" % (
    c["dt"], c["dk"], c["dv"], c["chunk"], "-".join(map(str, c["lengths"])), "-s0" if c["s0"] else ""))
def test_random_shapes(case):
    """Element-by-element parity with the fp64 oracle over seeded random
    shapes (the bound of the io dtype)."""
    c = case
    log("prefill random case %s" % c)
    w = synth.make_prefill(c["lengths"], H=c["H"], dk=c["dk"], dv=c["dv"], io_dtype=c["dt"], seed=c["seed"],
                           S0_std=0.05 if c["s0"] else None, chunk=c["chunk"])
    o_ref, S_ref = oracle_prefill(w)
    o, S = gpu_prefill(w, in_place=c["in_place"] and c["s0"])
    check("o", o, o_ref, TOL[c["dt"]])
    check("S_T", S, S_ref, TOL[c["dt"]])
