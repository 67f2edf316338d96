"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars (from the method's stated accuracy targets):
  fp32 decode path ........ max |gpu - oracle| <= 1e-5
  bf16 chunked prefill .... |gpu - oracle| <= 2e-2 + 1e-2 |oracle| per element,
                            on the output y and on the final state
  bf16 prologue outputs ... one bf16 rounding: <= 2^-8 |oracle| + 1e-5
Reduced sizes span several 64-token chunks and ragged tails; the full-size
workloads run on the GPU exactly as the benchmark launches them and are
compared on every output the oracle can afford (all heads for T=4096,
sampled heads / sequences for T=65536 and the packed varlen batch).
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import kimi_delta_attention_07_amd as kda
import oracle
from kda_testlib import (assert_bf16_rounding, assert_chunk_close, assert_fp32_close, gpu_prefill,
                         gpu_prefill_fused, np64, report, slice_heads, slice_seqs, to_dev)

pytestmark = pytest.mark.gpu
ORC = oracle.get()


def _step_dev(step, dev="cuda"):
    return {k: v.to(dev) for k, v in step.items()}


def run_decode(dec, steps=None, out_dtype=torch.float32):
    """GPU and oracle decode over the given steps; returns per-step errors."""
    st = dec["state"].double().numpy().copy()
    ca = dec["conv_cache"].double().numpy().copy()
    gst, gca, cw = dec["state"].cuda(), dec["conv_cache"].cuda(), dec["conv_w"].cuda()
    si = dec["slot_idx"]
    gsi = si.cuda() if si is not None else None
    errs = []
    for step in (dec["steps"] if steps is None else steps):
        want = ORC.decode_step(st, ca, dec["conv_w"], step, slot_idx=si)
        s = _step_dev(step)
        got = kda.decode_step(s["q_raw"], s["k_raw"], s["v_raw"], cw, gca, gst, s["log_alpha"], s["beta_logit"],
                              s["gate_logit"], gsi, out_dtype=out_dtype)
        errs.append((got, want))
    torch.cuda.synchronize()
    return errs, (gst, st), (gca, ca)


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
def test_decode_tiny_fp32():
    """Tiny workload: B=1, T=16, H=2, d=4, K=2, fp32, zero state: 16 decode steps."""
    dec = ki.config_decode(0)
    errs, (gst, st), (gca, ca) = run_decode(dec)
    for t, (got, want) in enumerate(errs):
        assert_fp32_close(got, want, f"y step {t}")
    assert_fp32_close(gst, st, "state")
    assert_fp32_close(gca, ca, "conv cache", 0.0)
    # token-by-token decode equals the oracle's prefill of the same tokens
    ref = ORC.prefill(ki.config_prefill(0))
    assert_fp32_close(torch.cat([g for g, _ in errs]), ref["y"], "decode vs prefill y")


def test_decode_batched_full():
    """256 slots x 1 token, H=32, d=128, K=4, 64 consecutive steps, state in place."""
    dec = ki.config_decode(2)
    errs, (gst, st), (gca, ca) = run_decode(dec)
    worst = max(assert_fp32_close(got, want, f"y step {t}") for t, (got, want) in enumerate(errs))
    assert_fp32_close(gst, st, "state after 64 steps")
    assert_fp32_close(gca, ca, "conv cache after 64 steps", 0.0)
    print(f"decode 256x64: worst |y err| {worst:.2e}")


@pytest.mark.parametrize("d", [8, 16, 32, 64, 128])
def test_decode_slot_map_and_dims(d):
    dec = ki.decode_inputs(40 + d, 5, H=3, d=d, K=3, steps=3, n_slots=9, slot_perm=True, state_std=0.1)
    before = dec["state"].clone()
    errs, (gst, st), (gca, ca) = run_decode(dec)
    for t, (got, want) in enumerate(errs):
        assert_fp32_close(got, want, f"y step {t}")
    assert_fp32_close(gst, st, "state")
    untouched = sorted(set(range(9)) - set(dec["slot_idx"].tolist()))
    assert torch.equal(gst.cpu()[untouched], before[untouched])


def test_decode_out_of_range_slot_is_skipped():
    """Rows whose slot index lies outside [0, n_slots) (one past the end, one
    negative) are skipped: their output rows keep what was there, no slot's
    state or conv cache changes through them, and the other rows match the
    oracle."""
    dec = ki.decode_inputs(48, 4, H=2, d=64, K=4, steps=1, n_slots=6, state_std=0.1)
    step = dec["steps"][0]
    slot_idx = torch.tensor([2, 6, 5, -1], dtype=torch.int32)
    good = [0, 2]
    st = dec["state"].double().numpy().copy()
    ca = dec["conv_cache"].double().numpy().copy()
    sub = {k: v[good].contiguous() for k, v in step.items()}
    want = ORC.decode_step(st, ca, dec["conv_w"], sub, slot_idx=slot_idx[good])
    gst, gca = dec["state"].cuda(), dec["conv_cache"].cuda()
    s = _step_dev(step)
    out = torch.full((4, 2, 64), 7.0, device="cuda")
    kda.decode_step(s["q_raw"], s["k_raw"], s["v_raw"], dec["conv_w"].cuda(), gca, gst, s["log_alpha"],
                    s["beta_logit"], s["gate_logit"], slot_idx.cuda(), out=out)
    torch.cuda.synchronize()
    assert_fp32_close(out[good], want, "rows with valid slots")
    assert torch.all(out[[1, 3]].cpu() == 7.0), "a skipped row's output was written"
    assert_fp32_close(gst, st, "state")
    assert_fp32_close(gca, ca, "conv cache", 0.0)


@pytest.mark.parametrize("i", range(8))
def test_decode_random_configs(i):
    """Eight seeded random decode batches: rows, heads, head dim, conv width,
    step count, slot count and row-to-slot map, decay range, gate on or off.
    Every output row, the states and the conv caches against the oracle, fp32
    bar 1e-5."""
    rng = np.random.default_rng(8000 + i)
    batch, H = int(rng.integers(1, 41)), int(rng.integers(1, 7))
    d, K = int(rng.choice([4, 8, 16, 32, 64, 128])), int(rng.integers(1, 5))
    perm = bool(rng.random() < 0.6)
    n_slots = batch + int(rng.integers(0, 8)) if perm else None
    la = [(-5.0, 0.0), (-8.0, -2.0), (-1.0, 1.5)][int(rng.integers(0, 3))]
    gated = bool(rng.random() < 0.7)
    dec = ki.decode_inputs(8000 + i, batch, H=H, d=d, K=K, steps=int(rng.integers(1, 4)), la_range=la,
                           n_slots=n_slots, slot_perm=perm, state_std=0.1)
    what = f"random decode {i} (batch {batch}, H={H}, d={d}, K={K}, slots {n_slots}, la {la}, gated {gated})"
    si = dec["slot_idx"]
    st = dec["state"].double().numpy().copy()
    ca = dec["conv_cache"].double().numpy().copy()
    gst, gca, cw = dec["state"].cuda(), dec["conv_cache"].cuda(), dec["conv_w"].cuda()
    gsi = si.cuda() if si is not None else None
    for t, step in enumerate(dec["steps"]):
        if not gated:
            step = dict(step, gate_logit=None)
        want = ORC.decode_step(st, ca, dec["conv_w"], step, slot_idx=si)
        s = {k: (v.cuda() if v is not None else None) for k, v in step.items()}
        got = kda.decode_step(s["q_raw"], s["k_raw"], s["v_raw"], cw, gca, gst, s["log_alpha"], s["beta_logit"],
                              s["gate_logit"], gsi)
        torch.cuda.synchronize()
        assert_fp32_close(got, want, f"{what} y step {t}")
    assert_fp32_close(gst, st, what + " state")
    assert_fp32_close(gca, ca, what + " conv cache", 0.0)


def test_decode_bf16_output_and_no_gate():
    dec = ki.decode_inputs(50, 4, H=2, d=128, K=4, steps=2)
    for s in dec["steps"]:
        s["gate_logit"] = None
    st = dec["state"].double().numpy().copy()
    ca = dec["conv_cache"].double().numpy().copy()
    gst, gca, cw = dec["state"].cuda(), dec["conv_cache"].cuda(), dec["conv_w"].cuda()
    for step in dec["steps"]:
        want = ORC.decode_step(st, ca, dec["conv_w"], step)
        s = {k: (v.cuda() if v is not None else None) for k, v in step.items()}
        got = kda.decode_step(s["q_raw"], s["k_raw"], s["v_raw"], cw, gca, gst, s["log_alpha"], s["beta_logit"],
                              None, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert_bf16_rounding(got, want, "bf16 decode output")
    assert_fp32_close(gst, st, "state")


# ----------------------------------------------------------------------------
# prologue
# ----------------------------------------------------------------------------
def _gpu_prologue(inp, alias=False):
    g = to_dev(inp)
    cache_out = g["conv_cache"] if alias else torch.empty_like(g["conv_cache"])
    pro = kda.prologue(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["cu_seqlens"], g["beta_logit"],
                       g["gate_logit"], g["conv_cache"], cache_out, cu_seqlens_host=inp["cu_seqlens"])
    torch.cuda.synchronize()
    return pro, cache_out


def test_prologue_tiny_fp32():
    inp = ki.config_prefill(0)
    ref = ORC.prologue(inp)
    pro, cache_out = _gpu_prologue(inp)
    for k in ("q", "k", "v", "beta", "gate"):
        assert_fp32_close(pro[k], ref[k], f"prologue {k}")
    assert_fp32_close(cache_out, ref["conv_cache"], "conv cache", 0.0)


@pytest.mark.parametrize("alias", [False, True])
def test_prologue_bf16_varlen(alias):
    inp = ki.prefill_inputs(60, [0, 1, 2, 3, 70, 5, 129], H=4, d=128, K=4, cache_std=1.0)
    ref = ORC.prologue(inp)
    pro, cache_out = _gpu_prologue(inp, alias)
    for k in ("q", "k", "v", "gate"):
        assert_bf16_rounding(pro[k], ref[k], f"prologue {k}")
    assert_fp32_close(pro["beta"], ref["beta"], "beta")
    assert_fp32_close(cache_out, ref["conv_cache"], "conv cache out", 0.0)


@pytest.mark.parametrize("d,K,dtype", [(8, 1, torch.float32), (16, 2, torch.bfloat16), (32, 3, torch.float32),
                                       (64, 4, torch.bfloat16)])
def test_prologue_dims(d, K, dtype):
    inp = ki.prefill_inputs(61, [9, 0, 40], H=3, d=d, K=K, dtype=dtype, cache_std=1.0)
    ref = ORC.prologue(inp)
    pro, cache_out = _gpu_prologue(inp)
    check = assert_fp32_close if dtype == torch.float32 else assert_bf16_rounding
    for k in ("q", "k", "v", "gate"):
        check(pro[k], ref[k], f"prologue {k}")
    if K > 1:
        assert_fp32_close(cache_out, ref["conv_cache"], "conv cache", 0.0)


# ----------------------------------------------------------------------------
# chunked prefill, reduced sizes
# ----------------------------------------------------------------------------
def _check_prefill(inp, res, what, scale=1.0):
    ref = ORC.prefill(inp, scale=scale)
    e1 = assert_chunk_close(res["y"], ref["y"], f"{what} y")
    e2 = assert_chunk_close(res["final_state"], ref["final_state"], f"{what} final state")
    assert_fp32_close(res["conv_cache"], ref["conv_cache"], f"{what} conv cache", 0.0)
    return e1, e2


def _oracle_prologue_bf16(inp):
    """The oracle's prologue outputs, q^, k^, v^ and the gate rounded to bf16
    (the chunk path's input precision), beta in fp32: inputs that the chunk
    kernels and the oracle recurrence can both take."""
    pro = ORC.prologue(inp)
    bf = lambda a: torch.tensor(a).to(torch.bfloat16)
    return dict(q=bf(pro["q"]), k=bf(pro["k"]), v=bf(pro["v"]), gate=bf(pro["gate"]),
                beta=torch.tensor(pro["beta"]).float())


def _check_chunk_isolated(inp, what, scale=1.0):
    """The chunk kernels alone: kda_chunk_forward and the oracle recurrence on
    the same bf16 inputs (the oracle's own prologue outputs, rounded)."""
    pro = _oracle_prologue_bf16(inp)
    dev = lambda t: t.cuda() if t is not None else None
    yg, Sg = kda.chunk_forward(dev(pro["q"]), dev(pro["k"]), dev(pro["v"]), dev(inp["log_alpha"]), dev(pro["beta"]),
                               dev(pro["gate"]), dev(inp["cu_seqlens"]), dev(inp["initial_state"]), scale=scale,
                               cu_seqlens_host=inp["cu_seqlens"])
    torch.cuda.synchronize()
    y, S = ORC.recurrence(pro["q"], pro["k"], pro["v"], inp["log_alpha"], pro["beta"], pro["gate"],
                          inp["cu_seqlens"], scale, inp["initial_state"])
    assert_chunk_close(yg, y, f"{what} y (isolated)")
    assert_chunk_close(Sg, S, f"{what} final state (isolated)")
    return float(np.abs(np64(yg) - y).max()), float(np.abs(np64(Sg) - S).max())


def test_chunk_single_sequence_reduced():
    """T=4096 workload shape cut to T=300: 4 full chunks and a 44-token tail."""
    inp = ki.config_prefill(1, scale_T=300)
    res = gpu_prefill(inp)
    e = _check_prefill(inp, res, "T=300")
    iso = _check_chunk_isolated(inp, "T=300")
    print(f"T=300: end-to-end max |err| y {e[0]:.2e} S {e[1]:.2e}; chunk-only y {iso[0]:.2e} S {iso[1]:.2e}")


def test_chunk_varlen_edges():
    inp = ki.prefill_inputs(70, [0, 1, 63, 64, 65, 130, 0, 200], H=4, d=128, K=4, cache_std=1.0)
    res = gpu_prefill(inp)
    _check_prefill(inp, res, "varlen edges")
    _check_chunk_isolated(inp, "varlen edges")
    S = np64(res["final_state"])
    for n in (0, 6):   # empty sequences pass their state through exactly
        assert np.array_equal(S[n], inp["initial_state"][n].double().numpy())


def test_chunk_zero_state_alias_scale():
    inp = ki.prefill_inputs(71, [77, 150], H=2, d=128, K=4, state_std=None)
    g = to_dev(inp)
    pro = kda.prologue(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["cu_seqlens"], g["beta_logit"],
                       g["gate_logit"], cu_seqlens_host=inp["cu_seqlens"])
    scale = 128 ** -0.5
    # initial_state None means zeros
    y0, S0 = kda.chunk_forward(pro["q"], pro["k"], pro["v"], g["log_alpha"], pro["beta"], pro["gate"],
                               g["cu_seqlens"], None, scale=scale, cu_seqlens_host=inp["cu_seqlens"])
    # final_state aliasing initial_state
    st = torch.zeros(2, 2, 128, 128, device="cuda")
    y1, S1 = kda.chunk_forward(pro["q"], pro["k"], pro["v"], g["log_alpha"], pro["beta"], pro["gate"],
                               g["cu_seqlens"], st, final_state=st, scale=scale, cu_seqlens_host=inp["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(S0, st)
    ref = ORC.prefill(inp, scale=scale)
    assert_chunk_close(y0, ref["y"], "scaled y")
    assert_chunk_close(S0, ref["final_state"], "final state")


def test_chunk_no_gate_deterministic():
    """No gate, run twice: bit-identical, and within the bar of the oracle
    recurrence on the same bf16 inputs (the oracle's prologue outputs)."""
    inp = ki.prefill_inputs(72, [190], H=2, d=128, K=4)
    g = to_dev(inp)
    pro = {k: v.cuda() for k, v in _oracle_prologue_bf16(inp).items()}
    outs = [kda.chunk_forward(pro["q"], pro["k"], pro["v"], g["log_alpha"], pro["beta"], None, g["cu_seqlens"],
                              g["initial_state"], cu_seqlens_host=inp["cu_seqlens"]) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    pro = {k: v.cpu() for k, v in pro.items()}
    y, S = ORC.recurrence(pro["q"], pro["k"], pro["v"], inp["log_alpha"], pro["beta"], None, inp["cu_seqlens"],
                          1.0, inp["initial_state"])
    assert_chunk_close(outs[0][0], y, "ungated y")
    assert_chunk_close(outs[0][1], S, "ungated S")


def test_chunk_continuation():
    """prefill(T) == prefill(T1) then prefill(T - T1) from its final state and conv cache."""
    inp = ki.prefill_inputs(73, [260], H=2, d=128, K=4, cache_std=1.0)
    whole = gpu_prefill(inp)
    T1 = 100
    a = dict(inp, T=T1, lengths=[T1], cu_seqlens=torch.tensor([0, T1], dtype=torch.int32))
    b = dict(inp, T=260 - T1, lengths=[260 - T1], cu_seqlens=torch.tensor([0, 260 - T1], dtype=torch.int32))
    for k in ("q_raw", "k_raw", "v_raw", "beta_logit", "log_alpha", "gate_logit"):
        a[k], b[k] = inp[k][:T1].contiguous(), inp[k][T1:].contiguous()
    ra = gpu_prefill(a)
    b["initial_state"], b["conv_cache"] = ra["final_state"].cpu(), ra["conv_cache"].cpu()
    rb = gpu_prefill(b)
    ref = ORC.prefill(inp)
    assert_chunk_close(torch.cat([ra["y"], rb["y"]]), ref["y"], "split y")
    assert_chunk_close(rb["final_state"], ref["final_state"], "split final state")
    assert torch.equal(rb["conv_cache"], whole["conv_cache"])


# ----------------------------------------------------------------------------
# fused prefill (prologue inside the chunk path)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("K", [4, 2, 1])
def test_prefill_fused_varlen_edges(K):
    inp = ki.prefill_inputs(80 + K, [0, 1, 2, 3, 63, 64, 65, 130, 0, 200], H=4, d=128, K=K, cache_std=1.0)
    res = gpu_prefill_fused(inp)
    ref = ORC.prefill(inp)
    e1 = assert_chunk_close(res["y"], ref["y"], f"fused K={K} y")
    e2 = assert_chunk_close(res["final_state"], ref["final_state"], f"fused K={K} final state")
    assert_fp32_close(res["conv_cache"], ref["conv_cache"], "fused conv cache", 0.0)
    S = np64(res["final_state"])
    for n in (0, 8):   # empty sequences pass their state through exactly
        assert np.array_equal(S[n], inp["initial_state"][n].double().numpy())
    print(f"fused K={K}: max |err| y {e1:.2e} S {e2:.2e}")


@pytest.mark.parametrize("lens,alias", [([1, 2, 3, 63, 64, 65, 130, 200], False),
                                        ([0, 1, 2, 5, 64, 30, 0], True)])
def test_prefill_fused_conv_cache_out(lens, alias):
    """Outgoing conv cache written by the prepare kernel itself: out of place
    with no empty sequence, and in place with every sequence within one chunk
    (short sequences keep part of the incoming cache)."""
    inp = ki.prefill_inputs(96 + alias, lens, H=3, d=128, K=4, cache_std=1.0)
    res = gpu_prefill_fused(inp, alias_cache=alias)
    ref = ORC.prefill(inp)
    assert_chunk_close(res["y"], ref["y"], "y")
    assert_chunk_close(res["final_state"], ref["final_state"], "final state")
    assert_fp32_close(res["conv_cache"], ref["conv_cache"], "conv cache", 0.0)


def test_prefill_empty_batch_passes_states_through():
    """Three empty sequences (total_tokens = 0: every per-token tensor is
    empty and reaches the library as NULL).  The fused, no-alloc and
    three-call paths leave each final state equal to its initial state and
    each outgoing conv cache equal to the incoming one, bit for bit, as the
    oracle does."""
    inp = ki.prefill_inputs(90, [0, 0, 0], H=2, d=128, K=4, cache_std=1.0)
    ref = ORC.prefill(inp)
    g = to_dev(inp)
    cu_h = inp["cu_seqlens"]
    runs = {"fused": gpu_prefill_fused(inp), "unfused": gpu_prefill(inp)}
    cache_out = torch.full_like(g["conv_cache"], float("nan"))
    y, S = kda.prefill_noalloc(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["log_alpha"], g["beta_logit"],
                               g["gate_logit"], g["cu_seqlens"], g["initial_state"], g["conv_cache"], cache_out,
                               cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    runs["noalloc"] = dict(y=y, final_state=S, conv_cache=cache_out)
    for name, res in runs.items():
        assert res["y"].numel() == 0, name
        assert np.array_equal(np64(res["final_state"]), ref["final_state"]), name
        assert np.array_equal(np64(res["conv_cache"]), ref["conv_cache"]), name
        print(f"empty batch {name}: states and conv caches passed through exactly")


def test_prefill_many_sequences():
    """150 short sequences (0..90 tokens, empty ones included): more than the
    128 whose chunk table travels in the kernel arguments, so the table is
    built on the device; both the fused and the unfused path."""
    g = torch.Generator().manual_seed(95)
    lens = torch.randint(0, 91, (150,), generator=g).tolist()
    lens[3] = lens[77] = 0
    inp = ki.prefill_inputs(95, lens, H=2, d=128, K=4, cache_std=1.0)
    ref = ORC.prefill(inp)
    for name, res in (("fused", gpu_prefill_fused(inp)), ("unfused", gpu_prefill(inp))):
        assert_chunk_close(res["y"], ref["y"], f"150 seqs {name} y")
        assert_chunk_close(res["final_state"], ref["final_state"], f"150 seqs {name} final state")
        assert_fp32_close(res["conv_cache"], ref["conv_cache"], f"150 seqs {name} conv cache", 0.0)
        S = np64(res["final_state"])
        assert np.array_equal(S[3], inp["initial_state"][3].double().numpy())


def test_prefill_many_sequences_dealt_to_xcds():
    """136 short sequences x 2 heads: 272 (sequence, head) items, a multiple
    of 8, so the scan deals them to the XCDs in turn; with more than 128
    sequences the table is built on the device and the dispatch order is the
    sequences' own.  Fused and unfused path, every element checked."""
    g = torch.Generator().manual_seed(98)
    lens = torch.randint(0, 91, (136,), generator=g).tolist()
    lens[0], lens[50] = 0, 1
    inp = ki.prefill_inputs(98, lens, H=2, d=128, K=4, cache_std=1.0)
    ref = ORC.prefill(inp)
    for name, res in (("fused", gpu_prefill_fused(inp)), ("unfused", gpu_prefill(inp))):
        assert_chunk_close(res["y"], ref["y"], f"136 seqs {name} y")
        assert_chunk_close(res["final_state"], ref["final_state"], f"136 seqs {name} final state")
        assert_fp32_close(res["conv_cache"], ref["conv_cache"], f"136 seqs {name} conv cache", 0.0)


@pytest.mark.parametrize("n_seqs", [40, 33])
def test_prefill_two_tiles_per_block(n_seqs):
    """n sequences x 2 heads: 80 heads put four value tiles in each scan block,
    66 heads two (both with one chain operand set in flight and the chunk
    table in the kernel arguments); empty and one-token sequences included;
    fused and unfused path, every element checked."""
    g = torch.Generator().manual_seed(97)
    lens = torch.randint(0, 151, (n_seqs,), generator=g).tolist()
    lens[0], lens[9], lens[n_seqs - 1] = 0, 1, 64
    inp = ki.prefill_inputs(97, lens, H=2, d=128, K=4, cache_std=1.0)
    ref = ORC.prefill(inp)
    for name, res in (("fused", gpu_prefill_fused(inp)), ("unfused", gpu_prefill(inp))):
        assert_chunk_close(res["y"], ref["y"], f"{n_seqs} seqs {name} y")
        assert_chunk_close(res["final_state"], ref["final_state"], f"{n_seqs} seqs {name} final state")
        assert_fp32_close(res["conv_cache"], ref["conv_cache"], f"{n_seqs} seqs {name} conv cache", 0.0)
        assert np.array_equal(np64(res["final_state"])[0], inp["initial_state"][0].double().numpy())


def test_prefill_nonfinite_sequence_stays_isolated():
    """One sequence of a packed batch holds NaN / inf in every input; its
    neighbours' outputs, final states and conv caches still match the oracle
    run without it (a chunk never mixes rows past its end, which here belong
    to the poisoned sequence, into its results).  Fused and unfused paths."""
    lens = [37, 50, 64, 10]
    inp = ki.prefill_inputs(97, lens, H=2, d=128, K=4, cache_std=1.0)
    cu = inp["cu_seqlens"].tolist()
    bad = dict(inp)
    for key, val in (("q_raw", float("nan")), ("k_raw", float("inf")), ("v_raw", float("nan")),
                     ("log_alpha", float("nan")), ("beta_logit", float("nan")), ("gate_logit", float("-inf"))):
        t = inp[key].clone()
        t[cu[1]:cu[2]] = val
        bad[key] = t
    keep = [0, 2, 3]
    ref = ORC.prefill(slice_seqs(inp, keep))
    for name, res in (("fused", gpu_prefill_fused(bad)), ("unfused", gpu_prefill(bad))):
        y, S, cc = np64(res["y"]), np64(res["final_state"]), np64(res["conv_cache"])
        assert_chunk_close(np.concatenate([y[cu[n]:cu[n + 1]] for n in keep]), ref["y"], f"{name} y")
        assert_chunk_close(S[keep], ref["final_state"], f"{name} final state")
        assert_fp32_close(cc[keep], ref["conv_cache"], f"{name} conv cache", 0.0)


def test_prefill_fused_alias_nogate_scale_and_matches_unfused():
    inp = ki.prefill_inputs(90, [150, 77], H=2, d=128, K=4, cache_std=1.0)
    scale = 128 ** -0.5
    res = gpu_prefill_fused(inp, scale=scale, alias_cache=True, gated=False)
    ref = ORC.prefill(dict(inp, gate_logit=None), scale=scale)
    assert_chunk_close(res["y"], ref["y"], "fused ungated y")
    assert_chunk_close(res["final_state"], ref["final_state"], "fused final state")
    assert_fp32_close(res["conv_cache"], ref["conv_cache"], "aliased conv cache", 0.0)
    a = gpu_prefill_fused(inp)
    b = gpu_prefill(inp)   # unfused path on the same inputs: close (fused skips one bf16 rounding)
    assert_chunk_close(a["y"], np64(b["y"]), "fused vs unfused y")
    c = gpu_prefill_fused(inp)
    assert torch.equal(a["y"], c["y"]) and torch.equal(a["final_state"], c["final_state"])


def _random_prefill_config(i):
    """Configuration i of the randomised prefill cases: batch shape, heads,
    conv width, decay range, zero or drawn state and cache, gate, scale and
    cache aliasing, all from one seeded generator."""
    rng = np.random.default_rng(7000 + i)
    n = int(rng.integers(1, 13))
    lens = [int(x) for x in rng.integers(0, 300, n)]
    if rng.random() < 0.3:
        lens[int(rng.integers(0, n))] = 0
    la = [(-5.0, 0.0), (-8.0, -2.0), (-1.0, 1.5)][int(rng.integers(0, 3))]
    kw = dict(H=int(rng.integers(1, 6)), d=128, K=int(rng.integers(1, 5)), la_range=la,
              state_std=None if rng.random() < 0.3 else 0.05, cache_std=None if rng.random() < 0.3 else 1.0)
    opts = dict(gated=bool(rng.random() < 0.7), scale=float(rng.choice([1.0, 128 ** -0.5])),
                alias=bool(rng.random() < 0.5))
    return ki.prefill_inputs(7000 + i, lens, **kw), opts


@pytest.mark.parametrize("i", range(8))
def test_prefill_random_configs(i):
    """Eight seeded random batches through the fused path (and, gated, the
    three-call path) against the oracle: every element within the chunk
    bar, the conv cache exact."""
    inp, o = _random_prefill_config(i)
    ref = ORC.prefill(inp if o["gated"] else dict(inp, gate_logit=None), scale=o["scale"])
    res = gpu_prefill_fused(inp, scale=o["scale"], alias_cache=o["alias"], gated=o["gated"])
    what = f"random {i} (lens {inp['lengths']}, H={inp['H']}, K={inp['K']}, {o})"
    assert_chunk_close(res["y"], ref["y"], what + " fused y")
    assert_chunk_close(res["final_state"], ref["final_state"], what + " fused final state")
    assert_fp32_close(res["conv_cache"], ref["conv_cache"], what + " fused conv cache", 0.0)
    if o["gated"]:
        res = gpu_prefill(inp, scale=o["scale"])
        assert_chunk_close(res["y"], ref["y"], what + " unfused y")
        assert_chunk_close(res["final_state"], ref["final_state"], what + " unfused final state")
        assert_fp32_close(res["conv_cache"], ref["conv_cache"], what + " unfused conv cache", 0.0)


def test_prefill_fused_T4096_full():
    inp = ki.config_prefill(1)
    res = gpu_prefill_fused(inp)
    ref = ORC.prefill(inp)
    e1 = assert_chunk_close(res["y"], ref["y"], "fused T=4096 y")
    e2 = assert_chunk_close(res["final_state"], ref["final_state"], "fused T=4096 final state")
    assert_fp32_close(res["conv_cache"], ref["conv_cache"], "fused T=4096 conv cache", 0.0)
    print(f"fused T=4096 full: max |err| y {e1:.2e} S {e2:.2e}")


# ----------------------------------------------------------------------------
# strong decays: chunks whose decay is too large for the chunk-start reference
# take the 16-token sub-chunk form
# ----------------------------------------------------------------------------
def _both_paths(inp, what):
    ref = ORC.prefill(inp)
    for name, res in (("fused", gpu_prefill_fused(inp)), ("unfused", gpu_prefill(inp))):
        assert_chunk_close(res["y"], ref["y"], f"{what} {name} y")
        assert_chunk_close(res["final_state"], ref["final_state"], f"{what} {name} final state")
        assert_fp32_close(res["conv_cache"], ref["conv_cache"], f"{what} {name} conv cache", 0.0)


def test_prefill_strong_decay_range():
    """log alpha = -exp(U(-1, 1.5)) (per token -0.37 .. -4.5, about -105 per
    chunk): every full chunk takes the sub-chunk form; ragged tails, an empty
    and a one-chunk sequence."""
    inp = ki.prefill_inputs(130, [300, 64, 17, 0, 200], H=4, d=128, K=4, la_range=(-1.0, 1.5), cache_std=1.0)
    _both_paths(inp, "strong decay")


@pytest.mark.parametrize("la", [-2.0, -4.0, -5.0])
def test_prefill_constant_decay(la):
    """Constant log alpha: -2 and -4 (the values that overflowed the
    chunk-start form) and -5 (80 per 16-token sub-chunk, near that form's
    bound)."""
    inp = ki.prefill_inputs(131, [300, 45], H=2, d=128, K=4, cache_std=1.0)
    inp["log_alpha"] = torch.full_like(inp["log_alpha"], la)
    _both_paths(inp, f"log alpha = {la}")


def test_prefill_decay_forms_mixed():
    """One sequence whose chunks alternate between mild decay (chunk-start
    form) and strong decay (sub-chunk form), plus chunks where only one
    16-token sub-chunk decays strongly: the state passes between chunks of
    both forms."""
    mild = ki.prefill_inputs(132, [640], H=4, d=128, K=4, cache_std=1.0)
    strong = ki.prefill_inputs(132, [640], H=4, d=128, K=4, la_range=(-1.0, 1.5), cache_std=1.0)
    t = torch.arange(640)
    use_strong = ((t // 64) % 2 == 1) | ((t // 64 == 4) & ((t % 64) // 16 == 2))
    inp = dict(mild)
    inp["log_alpha"] = torch.where(use_strong[:, None, None], strong["log_alpha"], mild["log_alpha"])
    _both_paths(inp, "mixed decay forms")


def test_prefill_strong_decay_T4096():
    """The T=4096 launch shape (one sequence, 64 chunks) at 8 heads with
    strong decay, every element against the oracle (fused path, as the
    benchmark runs it)."""
    inp = ki.prefill_inputs(133, [4096], H=8, d=128, K=4, la_range=(-1.0, 1.5))
    res = gpu_prefill_fused(inp)
    ref = ORC.prefill(inp)
    assert_chunk_close(res["y"], ref["y"], "strong decay T=4096 y")
    assert_chunk_close(res["final_state"], ref["final_state"], "strong decay T=4096 final state")


# ----------------------------------------------------------------------------
# full-size workloads (the benchmark's launch configuration)
# ----------------------------------------------------------------------------
def test_prefill_T4096_full():
    """T=4096, H=32, d=128: every output against the oracle."""
    inp = ki.config_prefill(1)
    res = gpu_prefill(inp)
    e = _check_prefill(inp, res, "T=4096")
    print(f"T=4096 full: max |err| y {e[0]:.2e} final state {e[1]:.2e}")


@pytest.fixture(scope="module")
def varlen_case():
    """32 packed sequences (lengths U[256, 8192]); the oracle on the shortest,
    the longest, the first and one more sequence, each on three heads."""
    inp = ki.config_prefill(3)
    lens = inp["lengths"]
    seqs = sorted({0, int(np.argmax(lens)), int(np.argmin(lens)), 17})
    heads = [0, 13, 31]
    ref = ORC.prefill(slice_heads(slice_seqs(inp, seqs), heads))
    return inp, seqs, heads, ref


@pytest.mark.parametrize("path", ["fused", "unfused"])
def test_prefill_varlen_full_sampled(varlen_case, path):
    """The packed varlen workload in full, in the launch configuration the
    benchmark times (fused: kda_prefill) and through the three-call path;
    sampled sequences x heads against the oracle, conv cache of every
    sequence exactly."""
    inp, seqs, heads, ref = varlen_case
    res = gpu_prefill_fused(inp) if path == "fused" else gpu_prefill(inp)
    cu = inp["cu_seqlens"].tolist()
    y = torch.cat([res["y"][cu[n]:cu[n + 1]] for n in seqs])[:, heads]
    S = res["final_state"][seqs][:, heads]
    e1 = assert_chunk_close(y, ref["y"], f"varlen {path} y")
    e2 = assert_chunk_close(S, ref["final_state"], f"varlen {path} final state")
    # the outgoing conv cache of every sequence: the last 3 raw rows, exactly
    K1 = inp["conv_w"].shape[2] - 1
    cc = np64(res["conv_cache"])
    for n in range(inp["N"]):
        for X, key in enumerate(("q_raw", "k_raw", "v_raw")):
            want = inp[key][cu[n + 1] - K1:cu[n + 1]].double().reshape(K1, -1).numpy()
            assert np.array_equal(cc[n, X], want), f"conv cache of sequence {n}, stream {X}"
    print(f"varlen {path} T={inp['T']}: sampled max |err| y {e1:.2e} S {e2:.2e}")
    del res
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def long_case():
    """T=65536 with slow decay (1024 chunks); the oracle on heads 0 and 31."""
    inp = ki.config_prefill(4)
    heads = [0, 31]
    ref = ORC.prefill(slice_heads(inp, heads))
    return inp, heads, ref


@pytest.mark.parametrize("path", ["fused", "unfused"])
def test_prefill_T65536_full_sampled_and_decode_tail(long_case, path):
    """T=65536 in full (fused: the benchmark's kda_prefill launch), two heads
    against the oracle, the conv cache exactly; then 128 decode tokens that
    continue the long context from the oracle's final state on those heads,
    every output and the state after them against the oracle at the fp32
    bar."""
    inp, heads, ref = long_case
    res = gpu_prefill_fused(inp) if path == "fused" else gpu_prefill(inp)
    e1 = assert_chunk_close(res["y"][:, heads], ref["y"], f"T=65536 {path} y")
    e2 = assert_chunk_close(res["final_state"][:, heads], ref["final_state"], f"T=65536 {path} final state")
    K1 = inp["conv_w"].shape[2] - 1
    for X, key in enumerate(("q_raw", "k_raw", "v_raw")):
        want = inp[key][-K1:].double().reshape(K1, -1).numpy()
        assert np.array_equal(np64(res["conv_cache"])[0, X], want), f"conv cache stream {X}"
    print(f"T=65536 {path}: sampled max |err| y {e1:.2e} S {e2:.2e}")
    # 128 decode tokens continuing the long context.  Both sides start from
    # the same state: on the sampled heads the oracle's final state rounded
    # to fp32, the conv cache the sequence's last raw rows (equal, bit for
    # bit, to what this path wrote: checked above); the GPU's other heads
    # keep this path's own final state and are not compared.
    H, d = inp["H"], inp["d"]
    state = res["final_state"].cpu()
    state[:, heads] = torch.from_numpy(ref["final_state"]).float()
    cache = torch.stack([inp[key][-K1:].float().reshape(K1, H * d) for key in ("q_raw", "k_raw", "v_raw")])[None]
    del res
    torch.cuda.empty_cache()
    gst, gca, cw = state.cuda(), cache.cuda(), inp["conv_w"].cuda()
    ch = torch.cat([torch.arange(h * d, (h + 1) * d) for h in heads])
    st = state[:, heads].double().numpy().copy()
    ca = cache[..., ch].double().numpy().copy()
    cw_o = inp["conv_w"][:, ch]
    worst = 0.0
    for t, step in enumerate(inp["tail"]):
        sdev = _step_dev(step)
        got = kda.decode_step(sdev["q_raw"], sdev["k_raw"], sdev["v_raw"], cw, gca, gst, sdev["log_alpha"],
                              sdev["beta_logit"], sdev["gate_logit"])
        want = ORC.decode_step(st, ca, cw_o, {k: v[:, heads] for k, v in step.items()})
        worst = max(worst, assert_fp32_close(got[:, heads], want, f"tail y step {t}"))
    torch.cuda.synchronize()
    assert_fp32_close(gst[:, heads], st, "tail state")
    report(f"T=65536 {path} decode tail y (last step)", got[:, heads], want, bar="fp32")
    print(f"decode tail after {path} prefill, 128 steps: worst |y err| {worst:.2e}")
