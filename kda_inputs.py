"""Seeded synthetic inputs for the KDA hot path (prefill and decode).

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no convolution, normalisation, gating or recurrence).  It
is the one module shared by the CPU oracle side (tests, the CPU baseline) and
the HIP side (parity tests, bench), so both consume bit-identical inputs.

Shapes and distributions follow the five workloads the method is measured on
(Kimi K3 KDA layers: head dim 128, short-conv kernel 4, 32 heads; plus a tiny
fp32 case with head dim 4 and conv kernel 2).  Everything is drawn on the CPU
from ``torch.Generator().manual_seed(seed)`` in a fixed order:

  1. sequence lengths (varlen only)      5. log-alpha  = -exp(U(a, b))
  2. conv weights      N(0, 0.5)         6. gate logit N(0, 1)
  3. raw q, k, v       N(0, 1)           7. initial state
  4. beta logit        N(0, 1)           8. conv cache
                                         9. decode-step inputs, step by step

N(mu, s) names a normal with standard deviation s.  Inputs meant to be bf16 are
drawn in fp32 and rounded to bf16 with round-to-nearest-even (torch's cast); the
oracle consumes exactly those rounded values.

Layouts (row-major, last index fastest):
  q_raw, k_raw [T, H, dk]; v_raw [T, H, dv]; log_alpha [T, H, dk];
  beta_logit [T, H]; gate_logit [T, H, dv];
  conv_w [3, H*d, K] fp32 (stream order q, k, v; tap K-1 multiplies the current token);
  conv_cache [N, 3, K-1, H*d] fp32 (oldest tap first);
  initial_state [N, H, dk, dv] fp32; cu_seqlens [N+1] int32.
"""
from __future__ import annotations

import torch

__all__ = [
    "prefill_inputs",
    "decode_inputs",
    "config_prefill",
    "config_decode",
    "mixer_inputs",
    "tokens_as_steps",
    "CONFIG_NAMES",
]

CONFIG_NAMES = {
    0: "tiny recurrent KDA fp32 (B=1 T=16 H=2 d=4 K=2)",
    1: "single-sequence chunked prefill (T=4096 H=32 d=128 K=4, chunk 64)",
    2: "batched decode step (256 slots x 1 token, H=32 d=128 K=4, 64 steps)",
    3: "packed varlen prefill (32 seqs, lengths U[256,8192], H=32 d=128 K=4)",
    4: "long-context prefill (T=65536 H=32 d=128 K=4) + 128 decode tokens",
}


def _normal(g, shape, std=1.0):
    return torch.randn(shape, generator=g, dtype=torch.float32) * std


def _uniform(g, shape, lo, hi):
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def _log_alpha(g, shape, lo, hi):
    # log-decay drawn as -exp(U(lo, hi)); part of the input recipe
    return -torch.exp(_uniform(g, shape, lo, hi))


def prefill_inputs(seed, lengths, H, d, K, dtype=torch.bfloat16,
                   la_range=(-5.0, 0.0), state_std=0.01, conv_w_std=0.5,
                   cache_std=None, draw_lengths=None, tail_steps=0):
    """Raw inputs for one packed prefill call.

    ``lengths``: list of per-sequence token counts (ignored when
    ``draw_lengths=(lo, hi, n)`` asks for n lengths drawn as integers
    U[lo, hi] inclusive, first in the draw order).  ``state_std=None`` means
    a zero initial state; ``cache_std=None`` a zero conv cache.
    ``tail_steps`` > 0 draws that many decode-step inputs (one token for each
    sequence) after everything else, for decoding on from the final state.
    """
    g = torch.Generator().manual_seed(seed)
    if draw_lengths is not None:
        lo, hi, n = draw_lengths
        lengths = torch.randint(lo, hi + 1, (n,), generator=g).tolist()
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    T = sum(lengths)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    if N:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    conv_w = _normal(g, (3, H * d, K), conv_w_std)
    q = _normal(g, (T, H, d)).to(dtype)
    k = _normal(g, (T, H, d)).to(dtype)
    v = _normal(g, (T, H, d)).to(dtype)
    beta_logit = _normal(g, (T, H)).to(dtype)
    log_alpha = _log_alpha(g, (T, H, d), *la_range).to(dtype)
    gate_logit = _normal(g, (T, H, d)).to(dtype)
    if state_std is None:
        s0 = torch.zeros(N, H, d, d, dtype=torch.float32)
    else:
        s0 = _normal(g, (N, H, d, d), state_std)
    if cache_std is None:
        cache = torch.zeros(N, 3, max(K - 1, 0), H * d, dtype=torch.float32)
    else:
        cache = _normal(g, (N, 3, max(K - 1, 0), H * d), cache_std)
    tail = [_step(g, N, H, d, dtype, la_range) for _ in range(tail_steps)]
    return dict(
        seed=seed, H=H, d=d, K=K, N=N, T=T, lengths=lengths, cu_seqlens=cu,
        conv_w=conv_w, q_raw=q, k_raw=k, v_raw=v, beta_logit=beta_logit,
        log_alpha=log_alpha, gate_logit=gate_logit, initial_state=s0,
        conv_cache=cache, dtype=dtype, tail=tail,
    )


def _step(g, batch, H, d, dtype, la_range):
    return dict(
        q_raw=_normal(g, (batch, H, d)).to(dtype),
        k_raw=_normal(g, (batch, H, d)).to(dtype),
        v_raw=_normal(g, (batch, H, d)).to(dtype),
        beta_logit=_normal(g, (batch, H)).to(dtype),
        log_alpha=_log_alpha(g, (batch, H, d), *la_range).to(dtype),
        gate_logit=_normal(g, (batch, H, d)).to(dtype),
    )


def mixer_inputs(seed, lengths, hidden, H, d, K, state_std=0.01):
    """Hidden states and weights for the KDA mixer (input projection, the
    operator, output projection) on one packed batch.

    Draw order: conv weights N(0, 0.5); x [T, hidden] N(0, 1); w_in
    [5 H d + H, hidden] N(0, 1/sqrt(hidden)) (so the projected q, k, v and
    logits come out near unit scale); w_out [hidden, H d] N(0, 1/sqrt(H d));
    a_log [H] U(-4, -1); dt_bias [H d] N(0, 1); initial state N(0, state_std).
    bf16 tensors are drawn in fp32 and rounded; a_log, dt_bias, conv weights
    and state stay fp32; the conv cache is zero.  The pages give no hidden
    size or decay parameters: these are synthetic.
    """
    g = torch.Generator().manual_seed(seed)
    lengths = [int(x) for x in lengths]
    N, T = len(lengths), sum(lengths)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    if N:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    C = H * d
    conv_w = _normal(g, (3, C, K), 0.5)
    x = _normal(g, (T, hidden)).to(torch.bfloat16)
    w_in = _normal(g, (5 * C + H, hidden), hidden ** -0.5).to(torch.bfloat16)
    w_out = _normal(g, (hidden, C), C ** -0.5).to(torch.bfloat16)
    a_log = _uniform(g, (H,), -4.0, -1.0)
    dt_bias = _normal(g, (C,))
    s0 = _normal(g, (N, H, d, d), state_std)
    cache = torch.zeros(N, 3, max(K - 1, 0), C, dtype=torch.float32)
    return dict(seed=seed, H=H, d=d, K=K, N=N, T=T, hidden=hidden, lengths=lengths, cu_seqlens=cu,
                conv_w=conv_w, x=x, w_in=w_in, w_out=w_out, a_log=a_log, dt_bias=dt_bias,
                initial_state=s0, conv_cache=cache)


def mla_inputs(seed, batch, H, H_kv, d_qk, d_v, max_len, lens=None, len_range=None, gate=True):
    """One MLA decode token for a batch: q [B, H, d_qk], k_new [B, H_kv, d_qk],
    v_new [B, H_kv, d_v], gate_logit [B, H, d_v], caches [B, H_kv, max_len,
    d_qk / d_v] (every slot filled, written or not), cache_len [B] int32.

    Draw order: lengths (given, or U[len_range] inclusive), q, k_new, v_new,
    k_cache, v_cache, gate; all N(0, 1) drawn in fp32 and rounded to bf16.
    The pages give no MLA widths beyond the tiny config's; these are
    synthetic."""
    g = torch.Generator().manual_seed(seed)
    if lens is None:
        lo, hi = len_range
        lens = torch.randint(lo, hi + 1, (batch,), generator=g).tolist()
    cache_len = torch.tensor([int(x) for x in lens], dtype=torch.int32)
    bf = lambda shape: _normal(g, shape).to(torch.bfloat16)
    q = bf((batch, H, d_qk))
    k_new = bf((batch, H_kv, d_qk))
    v_new = bf((batch, H_kv, d_v))
    k_cache = bf((batch, H_kv, max_len, d_qk))
    v_cache = bf((batch, H_kv, max_len, d_v))
    gate_logit = bf((batch, H, d_v)) if gate else None
    return dict(seed=seed, batch=batch, H=H, H_kv=H_kv, d_qk=d_qk, d_v=d_v, max_len=max_len, cache_len=cache_len,
                q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, gate_logit=gate_logit)


def tokens_as_steps(inp):
    """Split a single-sequence prefill input into per-token decode steps
    (pure re-layout: token t becomes step t with batch 1)."""
    assert inp["N"] == 1
    keys = ("q_raw", "k_raw", "v_raw", "beta_logit", "log_alpha", "gate_logit")
    return [{kk: inp[kk][t:t + 1].clone() for kk in keys} for t in range(inp["T"])]


def decode_inputs(seed, batch, H, d, K, steps, dtype=torch.bfloat16,
                  la_range=(-5.0, 0.0), state_std=0.05, cache_std=1.0,
                  conv_w_std=0.5, n_slots=None, slot_perm=False, g=None,
                  draw_state=True):
    """Raw inputs for ``steps`` consecutive decode steps over ``batch`` rows.

    Per step: q/k/v raw [batch, H, d], beta_logit [batch, H], log_alpha
    [batch, H, d], gate_logit [batch, H, d].  ``slot_perm`` draws a random
    row->slot map (a permutation of a random subset of ``n_slots``).
    Pass ``g`` to continue an existing generator (decode after prefill).
    """
    if g is None:
        g = torch.Generator().manual_seed(seed)
    n_slots = batch if n_slots is None else n_slots
    conv_w = _normal(g, (3, H * d, K), conv_w_std) if conv_w_std is not None else None
    state = cache = None
    if draw_state:
        state = _normal(g, (n_slots, H, d, d), state_std) if state_std else \
            torch.zeros(n_slots, H, d, d, dtype=torch.float32)
        cache = _normal(g, (n_slots, 3, max(K - 1, 0), H * d), cache_std) if cache_std else \
            torch.zeros(n_slots, 3, max(K - 1, 0), H * d, dtype=torch.float32)
    slot_idx = None
    if slot_perm:
        slot_idx = torch.randperm(n_slots, generator=g)[:batch].to(torch.int32)
    step_list = [_step(g, batch, H, d, dtype, la_range) for _ in range(steps)]
    return dict(seed=seed, batch=batch, n_slots=n_slots, H=H, d=d, K=K,
                conv_w=conv_w, state=state, conv_cache=cache, slot_idx=slot_idx,
                steps=step_list, dtype=dtype)


def config_prefill(i, scale_T=None):
    """Prefill inputs of workload ``i`` (0, 1, 3, 4).

    ``scale_T`` shrinks sequence lengths for reduced-size tests while keeping
    every distribution (for workload 3 it is the upper length bound).
    Workload 4 also carries its 128-token decode tail in ``tail``.
    """
    if i == 0:
        return prefill_inputs(0, [16], H=2, d=4, K=2, dtype=torch.float32,
                              state_std=None)
    if i == 1:
        T = 4096 if scale_T is None else scale_T
        return prefill_inputs(1, [T], H=32, d=128, K=4)
    if i == 3:
        if scale_T is None:
            return prefill_inputs(3, None, H=32, d=128, K=4,
                                  draw_lengths=(256, 8192, 32))
        return prefill_inputs(3, None, H=32, d=128, K=4,
                              draw_lengths=(max(1, scale_T // 32), scale_T, 32))
    if i == 4:
        T = 65536 if scale_T is None else scale_T
        return prefill_inputs(4, [T], H=32, d=128, K=4, la_range=(-8.0, -2.0),
                              tail_steps=128)
    raise ValueError(f"workload {i} has no prefill part")


def config_decode(i, steps=None, batch=None):
    """Decode inputs of workload ``i`` (0 or 2).

    Workload 0 is the tiny fp32 case: its 16 prefill tokens replayed one by
    one as decode steps from a zero state and a zero conv cache.  Workload 2
    is 256 resident slots, 64 steps.
    """
    if i == 0:
        inp = config_prefill(0)
        H, d, K = inp["H"], inp["d"], inp["K"]
        return dict(seed=0, batch=1, n_slots=1, H=H, d=d, K=K, conv_w=inp["conv_w"],
                    state=torch.zeros(1, H, d, d), conv_cache=torch.zeros(1, 3, K - 1, H * d),
                    slot_idx=None, steps=tokens_as_steps(inp)[:steps], dtype=torch.float32)
    if i == 2:
        return decode_inputs(2, 256 if batch is None else batch, H=32, d=128, K=4,
                             steps=64 if steps is None else steps)
    raise ValueError(f"workload {i} has no stand-alone decode part")
