"""kda_prefill_noalloc: the prefill on the library's fixed per-GPU scratch,
for callers that cannot allocate.  Checked through the C ABI against
kda_prefill on the same inputs (the same kernels, so identical bits), on two
calls in a row, the second with a smaller batch; batches beyond the scratch
are rejected on the host."""
import ctypes

import pytest
import torch

import kda_inputs as ki
import kimi_delta_attention_07_amd as kda
import oracle
from kda_testlib import assert_chunk_close, to_dev
from kimi_delta_attention_07_amd import _lib

WORKSPACE, UNSUP = 6, 4
FAKE = [ctypes.c_void_p(0x10000 + 0x100 * i) for i in range(20)]   # aligned, never dereferenced
SCRATCH = 64 * 1024 * 1024


def _call_fake(H, cu_vals, chunk=64):
    cu = torch.tensor(cu_vals, dtype=torch.int32)
    g = _lib.geom(H, 128, 4)
    return kda.load().kda_prefill_noalloc(ctypes.byref(g), len(cu_vals) - 1, cu_vals[-1], FAKE[15],
                                          ctypes.cast(cu.data_ptr(), ctypes.c_void_p), 1, chunk, *FAKE[:12], None)


def test_noalloc_rejects_beyond_scratch_on_host():
    """Nothing is launched (no device is touched) for a batch whose chunk
    workspace exceeds the scratch, or for a chunk length other than 64."""
    assert _call_fake(32, [0, 4096]) == WORKSPACE            # 64 chunks x 32 heads
    assert "scratch" in kda.load().kda_last_error_detail().decode()
    assert _call_fake(4, [0, 14464]) == WORKSPACE            # 226 chunks x 4 heads = 904 pairs
    assert _call_fake(32, [0, 1792], chunk=32) == UNSUP
    # the documented limit: 903 (chunk, head) pairs fit, with the table
    al = lambda x: (x + 255) // 256 * 256
    assert al(8) + al(16 * 28) + 28 * 32 * 74240 <= SCRATCH
    assert al(8) + al(16 * 225) + 225 * 4 * 74240 <= SCRATCH


def _run(inp, noalloc):
    g = to_dev(inp)
    cache_out = torch.empty_like(g["conv_cache"])
    fn = kda.prefill_noalloc if noalloc else kda.prefill
    y, S = fn(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["log_alpha"], g["beta_logit"], g["gate_logit"],
              g["cu_seqlens"], g["initial_state"], g["conv_cache"], cache_out, cu_seqlens_host=inp["cu_seqlens"])
    torch.cuda.synchronize()
    return y, S, cache_out


@pytest.mark.gpu
def test_noalloc_matches_prefill_two_calls():
    """Two calls in a row (the second smaller, so it runs over what the first
    left in the scratch): each equals kda_prefill bit for bit, and the oracle
    within the chunk path's bar."""
    orc = oracle.get()
    cases = [ki.prefill_inputs(120, [300, 1000, 77, 0, 129], H=4, d=128, K=4, cache_std=1.0),
             ki.prefill_inputs(121, [130], H=2, d=128, K=4, cache_std=1.0)]
    for i, inp in enumerate(cases):
        y, S, cc = _run(inp, noalloc=True)
        y2, S2, cc2 = _run(inp, noalloc=False)
        assert torch.equal(y, y2), f"call {i}: y differs from kda_prefill"
        assert torch.equal(S, S2), f"call {i}: final state differs from kda_prefill"
        assert torch.equal(cc, cc2), f"call {i}: conv cache differs from kda_prefill"
        ref = orc.prefill(inp)
        assert_chunk_close(y, ref["y"], f"noalloc call {i} y")
        assert_chunk_close(S, ref["final_state"], f"noalloc call {i} final state")


@pytest.mark.gpu
def test_noalloc_rejects_beyond_scratch_on_gpu():
    """Over the limit with real tensors: rejected, outputs untouched."""
    inp = ki.prefill_inputs(122, [64 * 226], H=4, d=128, K=4)
    g = to_dev(inp)
    out = torch.full_like(g["v_raw"], 3.0)
    with pytest.raises(kda.KdaError) as e:
        kda.prefill_noalloc(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["log_alpha"], g["beta_logit"],
                            g["gate_logit"], g["cu_seqlens"], g["initial_state"], out=out,
                            cu_seqlens_host=inp["cu_seqlens"])
    assert e.value.code == WORKSPACE and "scratch" in e.value.detail
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
