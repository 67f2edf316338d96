"""GPU parity of the KDA mixer's linear maps and of the whole mixer prefill
(input projection, the fused chunked prefill, output projection), through
the C ABI, against the CPU oracle on the same seeded inputs.

Bars:
  projections: |gpu - oracle| <= 2^-8 |oracle| + (1 + 2^-8) K 2^-24 S + 1e-6
    per element, S = sum_k |x_k w_k| (the fp32 accumulation bound over K
    terms in any order, then one bf16 rounding of that fp32 value); the decay segment
    carries the bound of its pre-activation through -exp(a_log) softplus
    (slope <= exp(a_log)) plus one bf16 rounding;
  the operator inside the mixer: the chunked path's 2e-2 + 1e-2 |oracle|,
    on the oracle's projections rounded to bf16 (both sides take them; the
    oracle is only ever given seeded inputs and its own results);
  the mixer itself: bit-identical to its three stages called one by one.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import kimi_delta_attention_07_amd as kda
import oracle
from kda_testlib import assert_chunk_close, np64, report

pytestmark = pytest.mark.gpu
ORC = oracle.get()
U = 2.0 ** -24


def assert_gemm_close(got, want, S, K, what, slope=None):
    got = np64(got)
    err = np.abs(got - want)
    acc = K * U * S * (1.0 if slope is None else slope)
    # the bf16 rounding acts on the fp32 result, which may already sit acc
    # away from the exact value: 2^-8 (|want| + acc)
    bar = 2.0 ** -8 * np.abs(want) + (1.0 + 2.0 ** -8) * acc + 1e-6
    bad = err > bar
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the bar (max abs {err.max():.3e})"
    print(f"PARITY {what}: max_abs {err.max():.3e} max_ref {np.abs(want).max():.3e} "
          f"bar_frac {(err / bar).max():.3f}", flush=True)


def check_in_projection(inp, res):
    """GPU input projection against the oracle's on the same bf16 x and w_in."""
    H, d, hidden = inp["H"], inp["d"], inp["hidden"]
    x, w = np64(inp["x"]), np64(inp["w_in"])
    ref = ORC.in_projection(x, w, H, d, np64(inp["a_log"]), np64(inp["dt_bias"]))
    S = np.abs(x) @ np.abs(w).T
    C = H * d
    T = x.shape[0]
    segS = lambda i: S[:, i * C:(i + 1) * C].reshape(T, H, d)
    for i, key in enumerate(("q_raw", "k_raw", "v_raw", "gate_logit")):
        assert_gemm_close(res[key], ref[key], segS(i), hidden, f"in projection {key}")
    slope = np.exp(np64(inp["a_log"]))[None, :, None]
    assert_gemm_close(res["log_alpha"], ref["log_alpha"], segS(4), hidden, "in projection log_alpha", slope)
    assert_gemm_close(res["beta_logit"], ref["beta_logit"], S[:, 5 * C:5 * C + H], hidden, "in projection beta_logit")
    assert (np64(res["log_alpha"]) <= 0).all()


@pytest.mark.parametrize("T,hidden,H,d", [(7, 16, 2, 4), (300, 16, 2, 4), (300, 1032, 4, 128), (513, 512, 3, 32),
                                         (130, 1064, 40, 4)])
def test_in_projection(T, hidden, H, d):
    """The tiny K3Config widths (hidden 16, 2 heads of 4; the k3 README's
    Tutorial 3), a production-like head dim with a ragged output width
    (5*4*128 + 4 = 2564 columns) and hidden 1032 (K tail), and an odd mix;
    row counts span several 256-row tiles and a ragged one.  40 heads give
    the beta columns' narrow kernel two column blocks, the second partial,
    with a K that is not a multiple of its 32-wide steps."""
    inp = ki.mixer_inputs(140 + T + hidden, [T], hidden, H, d, 4)
    res = kda.in_projection(inp["x"].cuda(), inp["w_in"].cuda(), H, d, inp["a_log"].cuda(), inp["dt_bias"].cuda())
    torch.cuda.synchronize()
    check_in_projection(inp, res)


def test_in_projection_no_decay_parameters():
    """a_log and dt_bias absent: log alpha = -softplus(z)."""
    inp = ki.mixer_inputs(150, [64], 64, 2, 8, 4)
    res = kda.in_projection(inp["x"].cuda(), inp["w_in"].cuda(), 2, 8)
    torch.cuda.synchronize()
    x, w = np64(inp["x"]), np64(inp["w_in"])
    ref = ORC.in_projection(x, w, 2, 8)
    S = (np.abs(x) @ np.abs(w).T)[:, 64:80].reshape(64, 2, 8)
    assert_gemm_close(res["log_alpha"], ref["log_alpha"], S, 64, "log_alpha without a_log, dt_bias")


@pytest.mark.parametrize("T,C,hidden", [(300, 512, 1032), (5, 8, 16), (1024, 4096, 256), (4096, 512, 4096)])
def test_out_projection(T, C, hidden):
    """Ragged shapes take the 224-wide tile; 4096 x 4096 outputs fill 256
    CUs once with 256-wide tiles (16 x 16) and would need a second round
    with 224-wide ones (16 x 19), so they take the 256-wide tile."""
    g = torch.Generator().manual_seed(160 + T)
    y = torch.randn(T, C, generator=g).to(torch.bfloat16)
    w = (torch.randn(hidden, C, generator=g) * C ** -0.5).to(torch.bfloat16)
    out = kda.out_projection(y.cuda(), w.cuda())
    torch.cuda.synchronize()
    ref = ORC.linear(np64(y), np64(w))
    assert_gemm_close(out, ref, np.abs(np64(y)) @ np.abs(np64(w)).T, C, f"out projection {T}x{C}->{hidden}")


@pytest.mark.parametrize("i", range(6))
def test_projections_random_shapes(i):
    """Six seeded random shapes for each projection: rows 1..700, inner
    dimension any multiple of 8 up to 1280 (2048 for the output projection),
    1..12 heads of 4..128 channels (any output width for the output
    projection), decay parameters present or absent."""
    rng = np.random.default_rng(9700 + i)
    T, hidden = int(rng.integers(1, 701)), 8 * int(rng.integers(1, 161))
    H, d = int(rng.integers(1, 13)), int(rng.choice([4, 8, 16, 32, 64, 128]))
    inp = ki.mixer_inputs(9700 + i, [T], hidden, H, d, 4)
    if rng.random() < 0.5:
        res = kda.in_projection(inp["x"].cuda(), inp["w_in"].cuda(), H, d, inp["a_log"].cuda(),
                                inp["dt_bias"].cuda())
        torch.cuda.synchronize()
        check_in_projection(inp, res)
    else:
        res = kda.in_projection(inp["x"].cuda(), inp["w_in"].cuda(), H, d)
        torch.cuda.synchronize()
        x, w = np64(inp["x"]), np64(inp["w_in"])
        ref = ORC.in_projection(x, w, H, d)
        S = np.abs(x) @ np.abs(w).T
        C = H * d
        for j, key in enumerate(("q_raw", "k_raw", "v_raw", "gate_logit", "log_alpha")):
            assert_gemm_close(res[key], ref[key], S[:, j * C:(j + 1) * C].reshape(T, H, d), hidden,
                              f"random {i} in projection {key} (no decay parameters)")
        assert_gemm_close(res["beta_logit"], ref["beta_logit"], S[:, 5 * C:5 * C + H], hidden,
                          f"random {i} in projection beta_logit")
    C, N = 8 * int(rng.integers(1, 257)), int(rng.integers(1, 1501))
    g = torch.Generator().manual_seed(9700 + i)
    y = torch.randn(T, C, generator=g).to(torch.bfloat16)
    w = (torch.randn(N, C, generator=g) * C ** -0.5).to(torch.bfloat16)
    out = kda.out_projection(y.cuda(), w.cuda())
    torch.cuda.synchronize()
    ref = ORC.linear(np64(y), np64(w))
    assert_gemm_close(out, ref, np.abs(np64(y)) @ np.abs(np64(w)).T, C, f"random {i} out projection {T}x{C}->{N}")


def test_mixer_prefill():
    """The whole mixer on a packed batch (ragged, an empty sequence): equal to
    its three stages called one by one, and each stage against the oracle."""
    inp = ki.mixer_inputs(170, [300, 77, 0, 130], 512, 4, 128, 4)
    H, d, hidden = 4, 128, 512
    dev = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    cu_h = inp["cu_seqlens"]
    cache_out = torch.empty_like(dev["conv_cache"])
    out, S = kda.mixer_prefill(dev["x"], dev["w_in"], dev["w_out"], dev["conv_w"], dev["cu_seqlens"], dev["a_log"],
                               dev["dt_bias"], dev["initial_state"], dev["conv_cache"], cache_out, H=H, d=d,
                               cu_seqlens_host=cu_h)
    # the same three stages, one call each
    pro = kda.in_projection(dev["x"], dev["w_in"], H, d, dev["a_log"], dev["dt_bias"])
    cache2 = torch.empty_like(dev["conv_cache"])
    y, S2 = kda.prefill(pro["q_raw"], pro["k_raw"], pro["v_raw"], dev["conv_w"], pro["log_alpha"], pro["beta_logit"],
                        pro["gate_logit"], dev["cu_seqlens"], dev["initial_state"], dev["conv_cache"], cache2,
                        cu_seqlens_host=cu_h)
    out2 = kda.out_projection(y.reshape(inp["T"], H * d), dev["w_out"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(S, S2) and torch.equal(cache_out, cache2)
    check_in_projection(inp, {k: v.cpu() for k, v in pro.items()})
    # the operator and the output projection, each on the oracle's own
    # results rounded to bf16 (the operator's input and output precision):
    # the oracle's projections for the prefill, its prefill output for the
    # output projection; the GPU stages take the same values
    refp = ORC.in_projection(np64(inp["x"]), np64(inp["w_in"]), H, d, np64(inp["a_log"]), np64(inp["dt_bias"]))
    bf = lambda a: torch.tensor(a).to(torch.bfloat16)
    keys = ("q_raw", "k_raw", "v_raw", "log_alpha", "beta_logit", "gate_logit")
    op_inp = dict(H=H, d=d, K=4, N=inp["N"], T=inp["T"], lengths=inp["lengths"], cu_seqlens=cu_h,
                  conv_w=inp["conv_w"], initial_state=inp["initial_state"], conv_cache=inp["conv_cache"],
                  **{k: bf(refp[k]) for k in keys})
    ref = ORC.prefill(op_inp)
    g = {k: op_inp[k].cuda() for k in keys}
    y3, S3 = kda.prefill(g["q_raw"], g["k_raw"], g["v_raw"], dev["conv_w"], g["log_alpha"], g["beta_logit"],
                         g["gate_logit"], dev["cu_seqlens"], dev["initial_state"], dev["conv_cache"],
                         cu_seqlens_host=cu_h)
    yb = bf(ref["y"]).reshape(inp["T"], H * d)
    out3 = kda.out_projection(yb.cuda(), dev["w_out"])
    torch.cuda.synchronize()
    assert_chunk_close(y3, ref["y"], "mixer operator y")
    assert_chunk_close(S3, ref["final_state"], "mixer operator final state")
    yn, wn = np64(yb), np64(dev["w_out"])
    assert_gemm_close(out3, ORC.linear(yn, wn), np.abs(yn) @ np.abs(wn).T, H * d, "mixer out projection")
