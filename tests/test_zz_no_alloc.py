"""kda_prefill_noalloc -- the prefill whose workspace is the library's static
per-GPU scratch array -- against kda_prefill on the same inputs: two calls in
a row, the second smaller (the array keeps the first call's contents), then
problems whose one-stream workspace exceeds the array, which run the bounded
schedule inside it with identical results, and one that does not fit even
so, which must be refused."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import TOL, check, dev, gpu_prefill, have_gpu, host, log, oracle_prefill

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def _noalloc(w, in_place=False):
    import torch
    import gated_delta_rule_33_amd as kda
    dt = w.io_dtype
    S0 = dev(w.S0) if w.S0 is not None else None
    kw = {"S_T": S0} if in_place else {}
    o, S = kda.prefill_noalloc(dev(w.q, dt), dev(w.k, dt), dev(w.v, dt), dev(w.log_alpha), dev(w.beta),
                               dev(w.cu_seqlens), S0, chunk=w.chunk, cu_seqlens_host=w.cu_seqlens.tolist(), **kw)
    torch.cuda.synchronize()
    return host(o), host(S)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_matches_prefill_two_calls(dt):
    big = synth.make_prefill([2000, 0, 777, 3000, 65], H=4, dk=128, dv=128, io_dtype=dt, seed=41, S0_std=0.05)
    small = synth.make_prefill([100, 33], H=2, dk=64, dv=128, io_dtype=dt, seed=42, S0_std=0.05, chunk=32)
    for name, w in (("large", big), ("smaller", small)):
        log("noalloc %s dt=%s T=%d H=%d" % (name, dt, w.total_tokens, w.num_heads))
        o_na, S_na = _noalloc(w)
        o_ws, S_ws = gpu_prefill(w, one_stream=True)
        assert np.array_equal(o_na, o_ws), name
        assert np.array_equal(S_na, S_ws), name
        o_ref, S_ref = oracle_prefill(w)
        check("o " + name, o_na, o_ref, TOL[dt])
        check("S_T " + name, S_na, S_ref, TOL[dt])


def test_noalloc_in_place_and_size_limit():
    import torch
    import gated_delta_rule_33_amd as kda
    w = synth.make_prefill([500, 64], H=2, dk=128, dv=128, io_dtype="bf16", seed=43, S0_std=0.05)
    log("noalloc in place")
    o, S = _noalloc(w, in_place=True)
    o_ref, S_ref = oracle_prefill(w)
    check("o (in place)", o, o_ref, TOL["bf16"])
    check("S_T (in place)", S, S_ref, TOL["bf16"])
    # 16384 tokens x 32 heads need ~ 500 MB of one-stream workspace: the
    # call runs the bounded schedule inside the array, with the same bits
    T, H = 16384, 32
    desc, keep = kda.make_desc(1, T, H, 128, 128, 64, kda.KDA_BF16, [0, T], kda.KDA_PREFILL_ONE_STREAM)
    assert kda.prefill_workspace_size(desc) > kda.NOALLOC_SCRATCH_BYTES
    w = synth.make_prefill([T], H=H, dk=128, dv=128, io_dtype="bf16", seed=44, S0_std=0.05)
    log("noalloc bounded: %d tokens x %d heads" % (T, H))
    o_na, S_na = _noalloc(w)
    o_ws, S_ws = gpu_prefill(w, one_stream=True)
    assert np.array_equal(o_na, o_ws)
    assert np.array_equal(S_na, S_ws)
    # 160 one-token sequences x 32 heads: with S_T the carried states live
    # there and the call runs; without it they would need 320 MiB of the
    # array: refused, nothing launched
    N = 160
    w = synth.make_prefill([1] * N, H=H, dk=128, dv=128, io_dtype="bf16", seed=45, S0_std=0.05)
    log("noalloc bounded: %d one-token sequences x %d heads, then refused without S_T" % (N, H))
    o_na, S_na = _noalloc(w)
    o_ws, S_ws = gpu_prefill(w, one_stream=True)
    assert np.array_equal(o_na, o_ws)
    assert np.array_equal(S_na, S_ws)
    q = dev(w.q, "bf16")
    with pytest.raises(kda.KdaError) as ei:
        kda.prefill_noalloc(q, dev(w.k, "bf16"), dev(w.v, "bf16"), dev(w.log_alpha), dev(w.beta), dev(w.cu_seqlens),
                            dev(w.S0), cu_seqlens_host=w.cu_seqlens.tolist(), want_state=False)
    assert ei.value.status == kda.KDA_ERR_WORKSPACE_TOO_SMALL
