"""GPU parity of the MLA decode token (kda_mla_decode_step, through the C
ABI) against the CPU oracle on the same seeded bf16 inputs.

Bar, per element of out [b, h, :]:
  |gpu - oracle| <= 2^-8 |oracle| + (1 + 2^-8) (2 d_qk 2^-24 S + 4e-6) max_j |v_j|,
where S = scale * max_j sum_c |q_c k_jc| over the (b, h) pair's keys.  The
first term and the factor (1 + 2^-8) are the bf16 rounding of the fp32
output; inside the bracket, 2 d_qk 2^-24 S bounds the relative change fp32
score rounding makes in any softmax weight
(a score moves by at most d_qk 2^-24 S, a weight by twice that relative to
the rest), and 4e-6 covers the fp32 exponentials and the at most 8-term
sequential plus tree-ordered sums of the weights and weighted values.
The cache writes are compared bit for bit: slot cache_len of each sequence
holds k_new / v_new, every other slot is unchanged.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import kimi_delta_attention_07_amd as kda
import oracle
from kda_testlib import np64

pytestmark = pytest.mark.gpu
ORC = oracle.get()
U = 2.0 ** -24


def run_gpu(inp, gate=True):
    dev = torch.device("cuda")
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    kc, vc = g["k_cache"].clone(), g["v_cache"].clone()
    out = kda.mla_decode_step(g["q"], g["k_new"], g["v_new"], kc, vc, g["cache_len"],
                              g["gate_logit"] if gate else None)
    torch.cuda.synchronize()
    return out, kc, vc


def oracle_step(inp, gate=True, batches=None):
    """The oracle on fp64 copies of the inputs (optionally a subset of the
    sequences); returns out and the updated caches."""
    sel = slice(None) if batches is None else batches
    kc, vc = np64(inp["k_cache"][sel]).copy(), np64(inp["v_cache"][sel]).copy()
    out = ORC.mla_decode_step(np64(inp["q"][sel]), np64(inp["k_new"][sel]), np64(inp["v_new"][sel]), kc, vc,
                              inp["cache_len"][sel].numpy(),
                              np64(inp["gate_logit"][sel]) if gate and inp["gate_logit"] is not None else None)
    return out, kc, vc


def bar(inp, kc64, vc64, batches=None):
    """Per-(b, h) error allowance (see the module docstring), broadcast over d_v."""
    sel = slice(None) if batches is None else batches
    q = np64(inp["q"][sel])
    B, H, dqk = q.shape
    G = H // inp["H_kv"]
    lens = inp["cache_len"][sel].numpy()
    scale = dqk ** -0.5
    out = np.zeros((B, H, 1))
    for b in range(B):
        n = int(lens[b]) + 1
        if not 0 <= lens[b] < inp["max_len"]:
            continue
        for h in range(H):
            K = kc64[b, h // G, :n]
            S = scale * (np.abs(K) @ np.abs(q[b, h])).max()
            out[b, h, 0] = (1 + 2.0 ** -8) * (2 * dqk * U * S + 4e-6) * np.abs(vc64[b, h // G, :n]).max()
    return out


def check(inp, what, gate=True):
    out, kc, vc = run_gpu(inp, gate)
    want, kc64, vc64 = oracle_step(inp, gate)
    got = np64(out)
    err = np.abs(got - want)
    allow = 2.0 ** -8 * np.abs(want) + bar(inp, kc64, vc64)
    bad = err > allow
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the bar (max abs {err.max():.3e})"
    print(f"PARITY {what}: max_abs {err.max():.3e} max_ref {np.abs(want).max():.3e} "
          f"bar_frac {(err / np.maximum(allow, 1e-300)).max():.3f}", flush=True)
    # caches: bit-exact append, nothing else touched
    assert torch.equal(kc.cpu(), torch.from_numpy(kc64).to(torch.bfloat16))
    assert torch.equal(vc.cpu(), torch.from_numpy(vc64).to(torch.bfloat16))
    return got


def test_mla_tiny_k3config():
    """The tiny K3Config's MLA widths (the k3 README, Tutorial 3: 2 heads,
    2 kv heads, nope 4 + rope 4 = 8 q/k channels, 4 value channels): the
    element-wise path (4 channels is not a whole 16-byte chunk)."""
    inp = ki.mla_inputs(40, 3, 2, 2, 8, 4, 16, lens=[0, 7, 15])
    check(inp, "mla tiny gated")
    check(inp, "mla tiny ungated", gate=False)


def test_mla_production_like_split_edges():
    """192 q/k channels (128 nope + 64 rope), 128 value channels, 16 heads,
    lengths on and around the 256-slot split edges and at the last slot."""
    inp = ki.mla_inputs(41, 6, 16, 16, 192, 128, 1100, lens=[0, 1, 255, 256, 511, 1099])
    check(inp, "mla 192/128 split edges")


@pytest.mark.parametrize("i", range(6))
def test_mla_random_configs(i):
    """Six seeded random batches: sequences, kv heads and group size, q/k and
    value widths anywhere in 1..256 (whole 16-byte chunks or not), cache
    size, lengths (the last slot and 0 among them), gate on or off."""
    rng = np.random.default_rng(9000 + i)
    B, Hkv, G = int(rng.integers(1, 9)), int(rng.choice([1, 2, 3, 4, 8])), int(rng.choice([1, 2, 4, 8]))
    vec = rng.random() < 0.5
    dqk = int(rng.integers(1, 33)) * 8 if vec else int(rng.integers(1, 257))
    dv = int(rng.integers(1, 33)) * 8 if vec else int(rng.integers(1, 257))
    L = int(rng.integers(1, 1201))
    lens = [int(x) for x in rng.integers(0, L, B)]
    lens[0] = L - 1
    if B > 1:
        lens[1] = 0
    gate = bool(rng.random() < 0.7)
    inp = ki.mla_inputs(9000 + i, B, Hkv * G, Hkv, dqk, dv, L, lens=lens, gate=gate)
    check(inp, f"mla random {i} (B={B}, H={Hkv * G}, H_kv={Hkv}, {dqk}/{dv}, L={L}, gate {gate})", gate=gate)


@pytest.mark.parametrize("H,H_kv,dqk,dv", [(8, 2, 128, 128), (6, 3, 64, 64), (4, 1, 256, 256), (4, 4, 100, 72),
                                           (2, 2, 16, 8), (16, 2, 192, 128), (24, 3, 64, 64), (32, 2, 64, 64)])
def test_mla_shapes(H, H_kv, dqk, dv):
    """Grouped heads (groups of 2 to 16; 16, 24 and 32 heads take the
    launch's XCD head order, H a multiple of 8), the other vector instances,
    widths that are not whole chunks (the element-wise path at 100 / 72
    channels)."""
    inp = ki.mla_inputs(42 + dqk, 3, H, H_kv, dqk, dv, 700, len_range=(0, 699))
    check(inp, f"mla H={H} H_kv={H_kv} {dqk}/{dv}")


def test_mla_out_of_range_lengths():
    """cache_len outside [0, max_len): the sequence is left alone (caches
    untouched, output 0); the others are unaffected."""
    inp = ki.mla_inputs(43, 4, 4, 2, 128, 128, 300, lens=[-1, 300, 17, 299])
    got = check(inp, "mla out-of-range lengths")
    assert not got[0].any() and not got[1].any() and got[2].any() and got[3].any()


def test_mla_decode_sequence():
    """24 tokens decoded one by one from an empty cache, the GPU's own caches
    carried from step to step, the oracle's likewise: every step within the
    bar, the caches equal at the end."""
    dev = torch.device("cuda")
    T, H, Hkv, dqk, dv, L = 24, 4, 2, 192, 128, 32
    seq = ki.mla_inputs(44, T, H, Hkv, dqk, dv, 1, lens=[0] * T)   # row t: the token of step t
    kc = torch.zeros(1, Hkv, L, dqk, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros(1, Hkv, L, dv, dtype=torch.bfloat16, device=dev)
    kc64, vc64 = np.zeros((1, Hkv, L, dqk)), np.zeros((1, Hkv, L, dv))
    worst = 0.0
    for t in range(T):
        lens = torch.tensor([t], dtype=torch.int32)
        step = {k: seq[k][t:t + 1] for k in ("q", "k_new", "v_new", "gate_logit")}
        out = kda.mla_decode_step(step["q"].to(dev), step["k_new"].to(dev), step["v_new"].to(dev), kc, vc,
                                  lens.to(dev), step["gate_logit"].to(dev))
        want = ORC.mla_decode_step(np64(step["q"]), np64(step["k_new"]), np64(step["v_new"]), kc64, vc64,
                                   lens.numpy(), np64(step["gate_logit"]))
        inp = dict(q=step["q"], cache_len=lens, H_kv=Hkv, max_len=L)
        allow = 2.0 ** -8 * np.abs(want) + bar(inp, kc64, vc64)
        err = np.abs(np64(out) - want)
        assert (err <= allow).all(), f"step {t}: max abs {err.max():.3e}"
        worst = max(worst, float((err / allow).max()))
    assert torch.equal(kc.cpu(), torch.from_numpy(kc64).to(torch.bfloat16))
    assert torch.equal(vc.cpu(), torch.from_numpy(vc64).to(torch.bfloat16))
    print(f"PARITY mla decode sequence of {T}: bar_frac {worst:.3f}", flush=True)


def test_mla_bench_workload_sampled():
    """The benchmark's workload (16 sequences, 64 heads, 192/128 channels,
    4096 cache slots, lengths U[1024, 4095]) in the launch the benchmark
    times; the oracle checks sequences 0, 7 and 15 in full (every head), the
    caches are checked bit for bit on the same sequences."""
    inp = ki.mla_inputs(45, 16, 64, 64, 192, 128, 4096, len_range=(1024, 4095))
    out, kc, vc = run_gpu(inp)
    sel = [0, 7, 15]
    want, kc64, vc64 = oracle_step(inp, batches=sel)
    got = np64(out)[sel]
    err = np.abs(got - want)
    allow = 2.0 ** -8 * np.abs(want) + bar(inp, kc64, vc64, batches=sel)
    assert (err <= allow).all(), f"{int((err > allow).sum())} elements beyond the bar (max abs {err.max():.3e})"
    print(f"PARITY mla bench workload (sequences {sel}): max_abs {err.max():.3e} "
          f"bar_frac {(err / allow).max():.3f}", flush=True)
    assert torch.equal(kc[sel].cpu(), torch.from_numpy(kc64).to(torch.bfloat16))
    assert torch.equal(vc[sel].cpu(), torch.from_numpy(vc64).to(torch.bfloat16))
