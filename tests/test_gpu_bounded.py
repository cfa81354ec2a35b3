"""The bounded-workspace schedule (KDA_PREFILL_BOUNDED) on the GPU: with a
workspace far smaller than the one-stream schedule's, the chunks run in
segments of global chunk indices whose boundaries fall inside sequences; the
states carried between segments pass through fp32 memory unchanged, so o and
S_T must equal the one-stream schedule's bit for bit, and match the oracle.
With few (sequence, head) pairs and room for two or more segments of 64+
chunk indices, the segments rotate through a ring of block slots, prepared
on one half of the CUs while the state pass runs on the other."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import TOL, check, gpu_prefill, have_gpu, log, oracle_prefill

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _min_bytes(w):
    import gated_delta_rule_33_amd as kda
    T, H, dk = w.q.shape
    d, keep = kda.make_desc(w.num_seqs, T, H, dk, w.v.shape[2], w.chunk,
                            kda.KDA_BF16 if w.io_dtype == "bf16" else kda.KDA_F32, w.cu_seqlens.tolist(),
                            kda.KDA_PREFILL_BOUNDED)
    return kda.prefill_workspace_size(d)


def _block_bytes(w):
    es = 2 if w.io_dtype == "bf16" else 4
    C = max(w.chunk, 32)
    dk = w.q.shape[2]
    tri = 32 * (C // 2) * es + (C - 32) * C * es if C == 64 else C * C * es
    return (3 * C * dk * es + 2 * tri + dk * 4 + C * 4 + 1023) // 1024 * 1024


CASES = [
    # (lengths, H, dk, dv, dtype, chunk, extra chunk indices per segment beyond one)
    ([700, 1, 0, 1300, 64, 257], 4, 128, 128, "bf16", 64, 3),
    ([700, 1, 0, 1300, 64, 257], 4, 128, 128, "bf16", 64, 0),   # the smallest workspace
    ([300, 129, 33], 2, 64, 128, "f32", 32, 4),
    ([2000], 2, 128, 64, "bf16", 16, 10),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bounded_equals_one_stream(case):
    lengths, H, dk, dv, dt, chunk, extra = CASES[case]
    w = synth.make_prefill(lengths, H=H, dk=dk, dv=dv, io_dtype=dt, seed=900 + case, S0_std=0.05, chunk=chunk)
    cap = _min_bytes(w) + extra * H * _block_bytes(w)
    log("prefill bounded case %d: %s H=%d dk=%d dv=%d %s chunk %d, workspace %d bytes" %
        (case, lengths, H, dk, dv, dt, chunk, cap))
    o_b, S_b = gpu_prefill(w, max_workspace_bytes=cap)
    o_1, S_1 = gpu_prefill(w, one_stream=True)
    assert np.array_equal(o_b, o_1)
    assert np.array_equal(S_b, S_1)
    o_ref, S_ref = oracle_prefill(w)
    check("o bounded", o_b, o_ref, TOL[dt])
    check("S_T bounded", S_b, S_ref, TOL[dt])


def test_bounded_without_state_and_in_place():
    w = synth.make_prefill([900, 5, 1100], H=4, dk=128, dv=128, io_dtype="bf16", seed=911, S0_std=0.05)
    cap = _min_bytes(w) + 2 * 4 * _block_bytes(w)
    log("prefill bounded: no S_T (carry in the workspace), then in place")
    o_n, S_n = gpu_prefill(w, max_workspace_bytes=cap, want_state=False)
    o_1, S_1 = gpu_prefill(w, one_stream=True)
    assert S_n is None
    assert np.array_equal(o_n, o_1)
    o_i, S_i = gpu_prefill(w, max_workspace_bytes=cap, in_place=True)
    assert np.array_equal(o_i, o_1)
    assert np.array_equal(S_i, S_1)


RING_CASES = [
    # (lengths, H, dtype, slots of 64 chunk indices the workspace holds)
    ([16384], 4, "bf16", 2),
    ([5000, 3000, 9000], 2, "bf16", 3),
    ([9000, 700], 2, "f32", 2),
]


@pytest.mark.parametrize("case", range(len(RING_CASES)))
def test_bounded_ring_equals_one_stream(case):
    lengths, H, dt, slots = RING_CASES[case]
    w = synth.make_prefill(lengths, H=H, dk=128, dv=128, io_dtype=dt, seed=950 + case, S0_std=0.05)
    carry = w.num_seqs * H * 128 * 128 * 4
    cap = _min_bytes(w) - carry - H * _block_bytes(w) + (slots * 64 + 5) * H * _block_bytes(w)
    log("prefill bounded ring case %d: %s H=%d %s, %d slots (workspace %d bytes)" % (case, lengths, H, dt, slots, cap))
    o_b, S_b = gpu_prefill(w, max_workspace_bytes=cap)
    o_1, S_1 = gpu_prefill(w, one_stream=True)
    assert np.array_equal(o_b, o_1)
    assert np.array_equal(S_b, S_1)
    o_i, S_i = gpu_prefill(w, max_workspace_bytes=cap, in_place=True)
    assert np.array_equal(o_i, o_1)
    assert np.array_equal(S_i, S_1)
    o_ref, S_ref = oracle_prefill(w)
    check("o bounded ring", o_b, o_ref, TOL[dt])
    check("S_T bounded ring", S_b, S_ref, TOL[dt])


@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_bounded_gate_forms(gate):
    """The gate forms run the same segmented state pass."""
    w = synth.make_prefill([1500, 40, 700], H=2, dk=128, dv=128, io_dtype="bf16", seed=960, S0_std=0.05, gate=gate)
    cap = _min_bytes(w) + 4 * 2 * _block_bytes(w)
    log("prefill bounded, gate %s (workspace %d bytes)" % (gate, cap))
    o_b, S_b = gpu_prefill(w, max_workspace_bytes=cap)
    o_1, S_1 = gpu_prefill(w, one_stream=True)
    assert np.array_equal(o_b, o_1)
    assert np.array_equal(S_b, S_1)


def test_two_streams_overlapped_and_ring():
    """An overlapped call and a bounded ring call enqueued on two caller
    streams at once, three times, with nothing synchronised in between: both
    share the library's per-device streams and events, each keeps its own
    workspace (one per caller stream), and each result equals its one-stream
    result bit for bit."""
    import torch
    import gated_delta_rule_33_amd as kda
    from tests.gpu_helpers import dev, host
    w1 = synth.make_prefill([9000], H=4, dk=128, dv=128, io_dtype="bf16", seed=970, S0_std=0.05)
    w2 = synth.make_prefill([5000, 4000], H=2, dk=128, dv=128, io_dtype="bf16", seed=971, S0_std=0.05)
    carry2 = w2.num_seqs * 2 * 128 * 128 * 4
    cap2 = _min_bytes(w2) - carry2 - 2 * _block_bytes(w2) + (2 * 64 + 3) * 2 * _block_bytes(w2)
    log("two streams: overlapped %s x 4 heads, bounded ring %s x 2 heads" % ([9000], [5000, 4000]))
    o1_ref, S1_ref = gpu_prefill(w1, one_stream=True)
    o2_ref, S2_ref = gpu_prefill(w2, one_stream=True)

    def up(w):
        return dict(q=dev(w.q, "bf16"), k=dev(w.k, "bf16"), v=dev(w.v, "bf16"), la=dev(w.log_alpha),
                    b=dev(w.beta), cu=dev(w.cu_seqlens), S0=dev(w.S0), hc=w.cu_seqlens.tolist())
    a, b = up(w1), up(w2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            r1 = kda.prefill(a["q"], a["k"], a["v"], a["la"], a["b"], a["cu"], a["S0"], cu_seqlens_host=a["hc"],
                             stream=s1)
        with torch.cuda.stream(s2):
            r2 = kda.prefill(b["q"], b["k"], b["v"], b["la"], b["b"], b["cu"], b["S0"], cu_seqlens_host=b["hc"],
                             stream=s2, max_workspace_bytes=cap2)
        outs.append((r1, r2))
    torch.cuda.synchronize()
    for (o1, S1), (o2, S2) in outs:
        assert np.array_equal(host(o1), o1_ref)
        assert np.array_equal(host(S1), S1_ref)
        assert np.array_equal(host(o2), o2_ref)
        assert np.array_equal(host(S2), S2_ref)
