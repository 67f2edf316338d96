"""GPU parity of kda_prologue_backward against the oracle's prologue gradient
(pinned by finite differences in test_oracle_prologue_backward.py).  Both
sides get the same raw inputs (bf16 or fp32) and the same fp32 upstream
gradients; the kernels compute in fp32.  Bar, per gradient tensor and
element: |gpu - oracle| <= 1e-4 max|oracle| + 1e-3 |oracle| (fp32 sums of at
most K products per element, or of one product per token for the taps)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import kimi_delta_attention_07_amd as kda
import oracle

pytestmark = pytest.mark.gpu
ORC = oracle.get()
KEYS = ("dq_raw", "dk_raw", "dv_raw", "dconv_w", "dconv_cache", "dbeta_logit", "dgate_logit")


def make(seed, lengths, H, d, K, dtype, gate=True, cache=True):
    inp = ki.prefill_inputs(seed, lengths, H=H, d=d, K=K, dtype=dtype, cache_std=1.0 if cache else None)
    if not gate:
        inp["gate_logit"] = None
    g = torch.Generator().manual_seed(seed + 500)
    T = inp["T"]
    grads = dict(dq=torch.randn(T, H, d, generator=g), dk=torch.randn(T, H, d, generator=g),
                 dv=torch.randn(T, H, d, generator=g), dbeta=torch.randn(T, H, generator=g),
                 dgate=torch.randn(T, H, d, generator=g) if gate else None)
    return inp, grads


def run_gpu(inp, grads, act):
    dv = lambda t: t.cuda() if t is not None else None
    out = kda.prologue_backward(dv(inp["q_raw"]), dv(inp["k_raw"]), dv(inp["v_raw"]), dv(inp["conv_w"]),
                                dv(inp["cu_seqlens"]), dv(inp["beta_logit"]), dv(inp["gate_logit"]),
                                dv(inp["conv_cache"]), dv(grads["dq"]), dv(grads["dk"]), dv(grads["dv"]),
                                dv(grads["dbeta"]), dv(grads["dgate"]), act=act, cu_seqlens_host=inp["cu_seqlens"])
    torch.cuda.synchronize()
    return out


def check(got, ref, what):
    for key in KEYS:
        if ref[key] is None or got[key] is None:
            assert got[key] is None or ref[key] is None or ref[key].size == 0, (what, key)
            continue
        g = got[key].double().cpu().numpy()
        w = np.asarray(ref[key])
        assert g.shape == w.shape, (what, key, g.shape, w.shape)
        if w.size == 0:
            continue
        err = np.abs(g - w)
        bad = err > 1e-4 * np.abs(w).max() + 1e-3 * np.abs(w)
        assert not bad.any(), f"{what} {key}: {int(bad.sum())} off (max err {err.max():.3e}, max |ref| " \
                              f"{np.abs(w).max():.3e})"


@pytest.mark.parametrize("seed,lengths,H,d,K,dtype,act,gate,cache", [
    (1, [3, 0, 5], 2, 4, 2, torch.float32, "silu", True, True),
    (2, [0, 1, 70, 300], 4, 128, 4, torch.bfloat16, "silu", True, True),
    (3, [40, 9], 3, 64, 1, torch.float32, "none", False, False),
    (4, [2, 130, 1, 600], 2, 32, 3, torch.bfloat16, "none", True, False),
    (5, [513, 0, 2], 1, 16, 4, torch.float32, "silu", False, True),
])
def test_prologue_backward_matches_oracle(seed, lengths, H, d, K, dtype, act, gate, cache):
    inp, grads = make(seed, lengths, H, d, K, dtype, gate, cache)
    ref = ORC.prologue_backward(inp, grads, act=1 if act == "silu" else 0)
    check(run_gpu(inp, grads, act), ref, f"seed {seed}")


@pytest.mark.parametrize("seed,lengths,K,dtype,act,gate,cache", [
    (21, [2, 65, 0, 130], 1, torch.float32, "silu", True, True),
    (22, [1, 2, 64, 3, 200], 2, torch.bfloat16, "none", False, True),
    (23, [129, 0, 66], 3, torch.float32, "silu", True, False),
    (24, [63, 1, 64, 1], 4, torch.float32, "none", True, True),
])
def test_prologue_backward_head_dim_128_variants(seed, lengths, K, dtype, act, gate, cache):
    """Head dim 128 runs the streaming kernel: every conv width, fp32 and
    bf16 inputs, with and without activation, gate and cache, sequences
    shorter than the window and ones crossing its 64-token blocks."""
    inp, grads = make(seed, lengths, 2, 128, K, dtype, gate, cache)
    ref = ORC.prologue_backward(inp, grads, act=1 if act == "silu" else 0)
    check(run_gpu(inp, grads, act), ref, f"seed {seed}")


def test_prologue_backward_empty_batch_and_odd_heads():
    """No tokens at all (the tap and cache gradients come out as zeros), and
    H = 5 at d = 128 (the four-heads-per-block kernel has idle waves)."""
    inp, grads = make(9, [0, 0], 2, 128, 4, torch.bfloat16)
    got = run_gpu(inp, grads, "silu")
    assert not got["dconv_w"].any() and not got["dconv_cache"].any()
    inp, grads = make(10, [33, 0, 64], 5, 128, 4, torch.bfloat16)
    check(run_gpu(inp, grads, "silu"), ORC.prologue_backward(inp, grads), "H=5")


def test_prologue_backward_T4096_full():
    """The benchmark's prefill shapes: T = 4096, H = 32, d = 128, K = 4, bf16."""
    inp, grads = make(7, [4096], 32, 128, 4, torch.bfloat16)
    ref = ORC.prologue_backward(inp, grads)
    check(run_gpu(inp, grads, "silu"), ref, "T=4096")


def test_prologue_backward_deterministic():
    inp, grads = make(8, [300, 77], 2, 128, 4, torch.bfloat16)
    a, b = run_gpu(inp, grads, "silu"), run_gpu(inp, grads, "silu")
    for key in KEYS:
        if a[key] is not None:
            assert torch.equal(a[key], b[key]), key
