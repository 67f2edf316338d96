"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, slice workloads by head or
sequence (pure re-layout), and the tolerance checks.

Tolerances (written into the tests that use them):
  * fp32 decode path: max |gpu - oracle| <= 1e-5;
  * bf16-input chunked path: |gpu - oracle| <= 2e-2 + 1e-2 |oracle| elementwise,
    on outputs and on the final state;
  * bf16 prologue outputs: one bf16 rounding of the fp32 result,
    |gpu - oracle| <= 2^-8 |oracle| + 1e-5.
"""
import numpy as np
import torch

import kimi_delta_attention_07_amd as kda

PREFILL_KEYS = ("q_raw", "k_raw", "v_raw", "beta_logit", "log_alpha", "gate_logit")


def to_dev(inp, dev="cuda"):
    return {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}


def gpu_prefill(inp, dev="cuda", scale=1.0, with_cache=True):
    """prologue + chunk_forward on the GPU; returns numpy (fp64) results."""
    g = to_dev(inp, dev)
    cu_h = inp["cu_seqlens"]
    cache_out = torch.empty_like(g["conv_cache"])
    pro = kda.prologue(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["cu_seqlens"], g["beta_logit"],
                       g["gate_logit"], g["conv_cache"] if with_cache else None, cache_out, cu_seqlens_host=cu_h)
    y, S = kda.chunk_forward(pro["q"], pro["k"], pro["v"], g["log_alpha"], pro["beta"], pro["gate"],
                             g["cu_seqlens"], g["initial_state"], scale=scale, cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    return dict(y=y, final_state=S, conv_cache=cache_out, pro=pro)


def gpu_prefill_fused(inp, dev="cuda", scale=1.0, alias_cache=False, gated=True):
    """kda_prefill (fused prologue) on the GPU."""
    g = to_dev(inp, dev)
    cache_out = g["conv_cache"] if alias_cache else torch.empty_like(g["conv_cache"])
    y, S = kda.prefill(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["log_alpha"], g["beta_logit"],
                       g["gate_logit"] if gated else None, g["cu_seqlens"], g["initial_state"], g["conv_cache"],
                       cache_out, scale=scale, cu_seqlens_host=inp["cu_seqlens"])
    torch.cuda.synchronize()
    return dict(y=y, final_state=S, conv_cache=cache_out)


def np64(t):
    return t.detach().double().cpu().numpy()


def chunk_tol_violations(got, want):
    got, want = np64(got) if torch.is_tensor(got) else got, want
    err = np.abs(got - want)
    bad = err > 2e-2 + 1e-2 * np.abs(want)
    return int(bad.sum()), float(err.max()) if err.size else 0.0, float((err / (np.abs(want) + 1e-6)).max()) if err.size else 0.0


def assert_chunk_close(got, want, what):
    nbad, maxabs, maxrel = chunk_tol_violations(got, want)
    assert nbad == 0, f"{what}: {nbad} elements outside 2e-2 + 1e-2|ref| (max abs {maxabs:.3e})"
    report(what, got, want)
    return maxabs


def report(what, got, want, bar="chunk"):
    """Print one line of error figures for the log of a GPU run: max abs error,
    max abs of the reference, and the largest fraction of the bar any element
    uses (bar "chunk": 2e-2 + 1e-2|ref|; "fp32": 1e-5)."""
    got = np64(got) if torch.is_tensor(got) else got
    if got.size == 0:
        return
    err = np.abs(got - want)
    lim = 2e-2 + 1e-2 * np.abs(want) if bar == "chunk" else np.full_like(want, 1e-5)
    print(f"PARITY {what}: max_abs {err.max():.3e} max_ref {np.abs(want).max():.3e} "
          f"bar_frac {(err / lim).max():.3f}", flush=True)


def assert_fp32_close(got, want, what, tol=1e-5):
    got = np64(got) if torch.is_tensor(got) else got
    err = float(np.abs(got - want).max()) if got.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol}"
    return err


def assert_bf16_rounding(got, want, what):
    got = np64(got) if torch.is_tensor(got) else got
    err = np.abs(got - want)
    bad = err > 2.0 ** -8 * np.abs(want) + 1e-5
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond one bf16 rounding (max abs {err.max():.3e})"


def slice_heads(inp, heads):
    """Keep the listed heads (heads are independent in every step)."""
    H, d = inp["H"], inp["d"]
    hs = torch.tensor(heads)
    ch = (hs[:, None] * d + torch.arange(d)[None]).reshape(-1)
    out = dict(inp)
    for k in PREFILL_KEYS:
        out[k] = inp[k][:, hs].contiguous()
    out["conv_w"] = inp["conv_w"][:, ch].contiguous()
    out["conv_cache"] = inp["conv_cache"][:, :, :, ch].contiguous()
    out["initial_state"] = inp["initial_state"][:, hs].contiguous()
    out["H"] = len(heads)
    return out


def slice_seqs(inp, seqs):
    """Keep the listed sequences, re-packed in the given order."""
    cu = inp["cu_seqlens"].tolist()
    parts = [(cu[n], cu[n + 1]) for n in seqs]
    out = dict(inp)
    for k in PREFILL_KEYS:
        out[k] = torch.cat([inp[k][a:b] for a, b in parts]).contiguous()
    lens = [b - a for a, b in parts]
    out["lengths"] = lens
    out["N"] = len(seqs)
    out["T"] = sum(lens)
    c = torch.zeros(len(seqs) + 1, dtype=torch.int32)
    c[1:] = torch.cumsum(torch.tensor(lens), 0)
    out["cu_seqlens"] = c
    out["initial_state"] = inp["initial_state"][list(seqs)].contiguous()
    out["conv_cache"] = inp["conv_cache"][list(seqs)].contiguous()
    return out
