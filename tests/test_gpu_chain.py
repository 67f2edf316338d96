"""GPU parity of the composed layer gradient: kda_chunk_backward, then
kda_prologue_backward on the gradients it produces, against the oracle's
recurrence and prologue gradients composed the same way (the composition is
pinned by finite differences in test_oracle_chain.py).  Both chains start
from the oracle's forward prologue outputs rounded to bf16, the point the
chunk backward differentiates at (the forward prologue kernel's own parity
is tested on its own); both prologue gradients work from the raw inputs.
The oracle is given seeded inputs and its own results only.  Bar per tensor
and element, as for each stage: |gpu - oracle| <= 1e-4 max|oracle| +
1e-3 |oracle|."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import kimi_delta_attention_07_amd as kda
import oracle

pytestmark = pytest.mark.gpu
ORC = oracle.get()


def close(got, ref, what):
    g = got.double().cpu().numpy()
    w = np.asarray(ref)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    err = np.abs(g - w)
    bad = err > 1e-4 * np.abs(w).max() + 1e-3 * np.abs(w)
    assert not bad.any(), f"{what}: {int(bad.sum())} off (max err {err.max():.3e}, max |ref| {np.abs(w).max():.3e})"


@pytest.mark.parametrize("seed,lengths,H", [(41, [70, 0, 130], 2), (43, [1, 64, 65], 3)])
def test_layer_gradient_chain(seed, lengths, H):
    inp = ki.prefill_inputs(seed, lengths, H=H, d=128, K=4, cache_std=1.0)
    cu = inp["cu_seqlens"]
    dev = lambda t: t.cuda() if t is not None else None
    raw = [dev(inp[k]) for k in ("q_raw", "k_raw", "v_raw")]
    # the forward prologue's outputs from the oracle, rounded to the chunk
    # path's bf16 (beta fp32): both backward chains start from these values
    po = ORC.prologue(inp)
    bf = lambda a: torch.tensor(a).to(torch.bfloat16)
    host = dict(q=bf(po["q"]), k=bf(po["k"]), v=bf(po["v"]), gate=bf(po["gate"]), beta=torch.tensor(po["beta"]).float())
    pro = {k: dev(v) for k, v in host.items()}
    g = torch.Generator().manual_seed(seed + 1)
    dy = torch.randn(inp["T"], H, 128, generator=g).to(torch.bfloat16)
    dsf = torch.randn(inp["N"], H, 128, 128, generator=g) * 0.1
    gb = kda.chunk_backward(pro["q"], pro["k"], pro["v"], dev(inp["log_alpha"]), pro["beta"], pro["gate"], dev(cu),
                            dev(dy), dev(inp["initial_state"]), dev(dsf), cu_seqlens_host=cu)
    gr = kda.prologue_backward(*raw, dev(inp["conv_w"]), dev(cu), dev(inp["beta_logit"]), dev(inp["gate_logit"]),
                               dev(inp["conv_cache"]), gb["dq"], gb["dk"], gb["dv"], gb["dbeta"], gb["dgate"],
                               act="silu", cu_seqlens_host=cu)
    torch.cuda.synchronize()
    ro = ORC.recurrence_backward(host["q"], host["k"], host["v"], inp["log_alpha"], host["beta"], host["gate"], cu,
                                 dy, dsf, 1.0, inp["initial_state"])
    rr = ORC.prologue_backward(inp, {k: torch.from_numpy(ro[k]) for k in ("dq", "dk", "dv", "dbeta", "dgate")})
    close(gb["dlog_alpha"], ro["dla"], "dlog_alpha")
    close(gb["d_initial_state"], ro["ds0"], "d_initial_state")
    for key in ("dq_raw", "dk_raw", "dv_raw", "dconv_w", "dconv_cache", "dbeta_logit", "dgate_logit"):
        close(gr[key], rr[key], key)
