"""Pins for the CPU oracle (CPU only, no GPU).

The public pages print no KDA worked example, so every pin comes from the
mathematics of the method or from an independent library routine:

* brute force: the recurrence written as explicit dense matrix products
  S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T (numpy matmuls),
  against the oracle's factored token step;
* the chunked WY/UT form of the same recurrence (independent algebra:
  cumulative log-decay, unit-lower-triangular inverse) for chunk sizes
  1, 4, 16, 64 and a ragged tail;
* closed forms and invariants (alpha=1 & beta=0 keeps S; a zero state plus
  one token gives beta k v^T; beta=1 with q=k stores v exactly; beta=0 gives
  pure per-channel decay; linearity in (S0, v); column equivariance; a norm
  bound);
* numpy.convolve / scipy.special.expit / numpy.linalg.norm for conv, sigmoid
  and L2 normalisation, plus causality and no leak across sequences;
* composition: split prefill == whole prefill, token-by-token decode == prefill,
  packed varlen == separate sequences, slot remapping;
* mutation: plausible one-token mistakes planted in a copy of the oracle
  source must each fail at least one of these pins.
"""
import json
import os
import subprocess

import numpy as np
import pytest
from scipy.special import expit

import kda_inputs as ki
import oracle as O

ORC = O.get()
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers (numpy, written from the definitions, independent of kda_oracle.c)
# ----------------------------------------------------------------------------
def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_prepared(rng, lengths, H, dk, dv, la_lo=-5.0, la_hi=0.0, gate=True, s0=True):
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = len(lengths)
    return dict(
        q=_unit(rng, (T, H, dk)), k=_unit(rng, (T, H, dk)), v=rng.standard_normal((T, H, dv)),
        la=-np.exp(rng.uniform(la_lo, la_hi, (T, H, dk))), beta=expit(rng.standard_normal((T, H))),
        gate=expit(rng.standard_normal((T, H, dv))) if gate else None, cu=cu,
        s0=rng.standard_normal((N, H, dk, dv)) * 0.1 if s0 else None,
    )


def brute_force(p, scale=1.0):
    """Dense matrices, literally the defining recurrence."""
    q, k, v, la, beta, gate, cu = p["q"], p["k"], p["v"], p["la"], p["beta"], p["gate"], p["cu"]
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    y = np.zeros((T, H, dv))
    S_out = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = p["s0"][n, h].copy() if p["s0"] is not None else np.zeros((dk, dv))
            for t in range(cu[n], cu[n + 1]):
                M = (np.eye(dk) - beta[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(la[t, h]))
                S = M @ S + beta[t, h] * np.outer(k[t, h], v[t, h])
                o = scale * (S.T @ q[t, h])
                y[t, h] = o * (gate[t, h] if gate is not None else 1.0)
            S_out[n, h] = S
    return y, S_out


def chunked_wy(p, C, scale=1.0):
    """Chunked WY/UT form: per chunk with entry state S,
    G = cumsum(log alpha), A = tril(beta_i * sum_c k_i k_j e^{G_i-G_j}, -1),
    T = (I + A)^-1, W = T beta (K e^G), U~ = T beta V, U = U~ - W S,
    P = tril(sum_c q_i k_j e^{G_i-G_j}), O = (Q e^G) S + P U,
    S <- Diag(e^{G_last}) S + (K e^{G_last - G})^T U."""
    q, k, v, la, beta, gate, cu = p["q"], p["k"], p["v"], p["la"], p["beta"], p["gate"], p["cu"]
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    y = np.zeros((T, H, dv))
    S_out = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = p["s0"][n, h].copy() if p["s0"] is not None else np.zeros((dk, dv))
            for c0 in range(cu[n], cu[n + 1], C):
                sl = slice(c0, min(c0 + C, cu[n + 1]))
                L = sl.stop - sl.start
                G = np.cumsum(la[sl, h], axis=0)
                Kd, Ki, Qg = k[sl, h] * np.exp(G), k[sl, h] * np.exp(-G), q[sl, h] * np.exp(G)
                b = beta[sl, h][:, None]
                A = np.tril(Kd @ Ki.T, -1) * b
                Tm = np.linalg.inv(np.eye(L) + A)
                W = Tm @ (b * Kd)
                U = Tm @ (b * v[sl, h]) - W @ S
                P = np.tril(Qg @ Ki.T)
                Ob = Qg @ S + P @ U
                S = np.exp(G[-1])[:, None] * S + (k[sl, h] * np.exp(G[-1] - G)).T @ U
                g = gate[sl, h] if gate is not None else 1.0
                y[sl, h] = scale * Ob * g
            S_out[n, h] = S
    return y, S_out


def run_oracle(orc, p, scale=1.0):
    return orc.recurrence(p["q"], p["k"], p["v"], p["la"], p["beta"], p["gate"], p["cu"], scale, p["s0"])


def close(a, b, rtol=1e-10, atol=1e-12):
    return np.allclose(a, b, rtol=rtol, atol=atol)


# ----------------------------------------------------------------------------
# the pin suite (also run against planted mutants below)
# ----------------------------------------------------------------------------
def pin_brute_force(orc):
    rng = np.random.default_rng(10)
    ok = True
    for lengths, H, dk, dv in [([16], 2, 4, 4), ([5, 0, 11, 7], 2, 4, 5), ([9], 3, 6, 3)]:
        p = rand_prepared(rng, lengths, H, dk, dv)
        for scale in (1.0, 0.5):
            y, S = run_oracle(orc, p, scale)
            yb, Sb = brute_force(p, scale)
            ok &= close(y, yb) and close(S, Sb)
    return ok


def pin_brute_force_strong_decay(orc):
    """The same dense matrices at strong decays: log alpha = -exp(U(-1, 1.5))
    (per token down to -4.5) and constant -5, where a chunk's cumulative decay
    runs far past what e^{+G} can hold; the token loop never forms e^{+G}."""
    rng = np.random.default_rng(14)
    ok = True
    for lengths, H, dk, dv in [([70], 2, 4, 4), ([30, 0, 41], 1, 5, 3)]:
        p = rand_prepared(rng, lengths, H, dk, dv, la_lo=-1.0, la_hi=1.5)
        ok &= all(close(a, b) for a, b in zip(run_oracle(orc, p), brute_force(p)))
        p["la"] = np.full_like(p["la"], -5.0)
        ok &= all(close(a, b) for a, b in zip(run_oracle(orc, p), brute_force(p)))
    return ok


def pin_chunked(orc):
    rng = np.random.default_rng(11)
    p = rand_prepared(rng, [37, 150, 64, 1], 2, 5, 4)
    y, S = run_oracle(orc, p)
    ok = True
    for C in (1, 4, 16, 64):
        yc, Sc = chunked_wy(p, C)
        ok &= close(y, yc, 1e-9, 1e-11) and close(S, Sc, 1e-9, 1e-11)
    return ok


def _conv_ref(x, w, cu, act, cache):
    """numpy.convolve per channel on [cache history, sequence]."""
    T, C = x.shape
    K = w.shape[1]
    y = np.zeros_like(x)
    for n in range(len(cu) - 1):
        s, e = cu[n], cu[n + 1]
        if e == s:
            continue
        hist = cache[n] if cache is not None else np.zeros((K - 1, C))
        xp = np.concatenate([hist, x[s:e]], axis=0)
        for c in range(C):
            y[s:e, c] = np.convolve(xp[:, c], w[c, ::-1], mode="valid")[: e - s]
    return y * expit(y) if act == O.ACT_SILU else y


def pin_conv(orc):
    rng = np.random.default_rng(12)
    ok = True
    for K in (1, 2, 4):
        lengths = [7, 1, 2, 0, 12]
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        x = rng.standard_normal((sum(lengths), 6))
        w = rng.standard_normal((6, K))
        cache = rng.standard_normal((len(lengths), K - 1, 6))
        for act in (O.ACT_NONE, O.ACT_SILU):
            y, cout = orc.conv(x, w, cu, act, cache if K > 1 else None)
            ok &= close(y, _conv_ref(x, w, cu, act, cache if K > 1 else None), 1e-12, 1e-13)
            if K > 1:  # cache out = the last K-1 raw inputs (reaching into the old cache)
                for n in range(len(lengths)):
                    hist = np.concatenate([cache[n], x[cu[n]:cu[n + 1]]], axis=0)
                    ok &= np.array_equal(cout[n], hist[-(K - 1):])
    return ok


def pin_gates(orc):
    rng = np.random.default_rng(13)
    x = rng.standard_normal(1000) * 8
    ok = close(orc.sigmoid(x), expit(x), 1e-14, 1e-300)
    xs = rng.standard_normal((50, 2, 8)) * 3
    xn = orc.l2norm(xs)
    nrm = np.linalg.norm(xs, axis=-1, keepdims=True)
    ok &= close(xn / np.linalg.norm(xn, axis=-1, keepdims=True), xs / nrm, 1e-13, 1e-15)
    ok &= close(np.linalg.norm(xn, axis=-1) ** 2, (nrm[..., 0] ** 2) / (nrm[..., 0] ** 2 + O.L2_EPS), 1e-13)
    return ok


def pin_decode_equals_prefill(orc):
    """Token-by-token decode from (S0, cache) == one prefill of those tokens."""
    inp = ki.prefill_inputs(5, [9], H=2, d=4, K=3, dtype=__import__("torch").float32,
                            state_std=0.3, cache_std=1.0)
    ref = orc.prefill(inp)
    state = inp["initial_state"].double().numpy().copy()
    cache = inp["conv_cache"].double().numpy().copy()
    ys = [orc.decode_step(state, cache, inp["conv_w"], st)[0] for st in ki.tokens_as_steps(inp)]
    return (close(np.stack(ys), ref["y"], 1e-12, 1e-13) and close(state, ref["final_state"], 1e-12, 1e-13)
            and close(cache, ref["conv_cache"], 0, 0))


PINS = [pin_brute_force, pin_brute_force_strong_decay, pin_chunked, pin_conv, pin_gates, pin_decode_equals_prefill]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin(ORC)


# ----------------------------------------------------------------------------
# closed forms and invariants
# ----------------------------------------------------------------------------
def test_identity_step_keeps_state():
    rng = np.random.default_rng(20)
    p = rand_prepared(rng, [6], 2, 4, 5)
    p["la"][:] = 0.0
    p["beta"][:] = 0.0
    y, S = run_oracle(ORC, p, 0.7)
    assert np.array_equal(S, p["s0"])  # exact
    want = 0.7 * np.einsum("hkv,thk->thv", p["s0"][0], p["q"]) * p["gate"]
    assert close(y, want, 1e-14, 1e-15)


def test_zero_state_one_token():
    rng = np.random.default_rng(21)
    p = rand_prepared(rng, [1], 3, 4, 6, s0=False)
    y, S = run_oracle(ORC, p)
    b = p["beta"][0][:, None, None]
    assert close(S[0], b * np.einsum("hk,hv->hkv", p["k"][0], p["v"][0]), 1e-15, 0)
    kq = np.einsum("hk,hk->h", p["k"][0], p["q"][0])
    assert close(y[0], p["beta"][0][:, None] * kq[:, None] * p["v"][0] * p["gate"][0], 1e-14, 1e-16)


def test_delta_rule_stores_value():
    """beta=1, alpha=1, q=k unit: o_t = v_t whatever the prior state."""
    rng = np.random.default_rng(22)
    p = rand_prepared(rng, [8], 2, 6, 3, gate=False)
    p["la"][:] = 0.0
    p["beta"][:] = 1.0
    p["q"] = p["k"].copy()
    y, _ = run_oracle(ORC, p)
    assert close(y, p["v"], 1e-12, 1e-13)


def test_pure_decay_closed_form():
    rng = np.random.default_rng(23)
    p = rand_prepared(rng, [12, 5], 2, 4, 4)
    p["beta"][:] = 0.0
    y, S = run_oracle(ORC, p)
    cu = p["cu"]
    for n in range(2):
        G = np.cumsum(p["la"][cu[n]:cu[n + 1]], axis=0)  # [L, H, dk]
        assert close(S[n], np.exp(G[-1])[:, :, None] * p["s0"][n], 1e-13, 1e-15)
        St = np.exp(G)[..., None] * p["s0"][n][None]
        assert close(y[cu[n]:cu[n + 1]], np.einsum("thkv,thk->thv", St, p["q"][cu[n]:cu[n + 1]])
                     * p["gate"][cu[n]:cu[n + 1]], 1e-12, 1e-14)


def test_linear_in_state_and_values():
    rng = np.random.default_rng(24)
    p1 = rand_prepared(rng, [10, 7], 2, 4, 3)
    p2 = dict(p1, v=rng.standard_normal(p1["v"].shape), s0=rng.standard_normal(p1["s0"].shape))
    a, b = 0.7, -1.3
    p3 = dict(p1, v=a * p1["v"] + b * p2["v"], s0=a * p1["s0"] + b * p2["s0"])
    (y1, S1), (y2, S2), (y3, S3) = run_oracle(ORC, p1), run_oracle(ORC, p2), run_oracle(ORC, p3)
    assert close(y3, a * y1 + b * y2, 1e-10, 1e-12) and close(S3, a * S1 + b * S2, 1e-10, 1e-12)


def test_value_columns_independent():
    rng = np.random.default_rng(25)
    p = rand_prepared(rng, [11], 2, 4, 6)
    perm = rng.permutation(6)
    pp = dict(p, v=p["v"][..., perm], gate=p["gate"][..., perm], s0=p["s0"][..., perm])
    (y, S), (yp, Sp) = run_oracle(ORC, p), run_oracle(ORC, pp)
    assert close(yp, y[..., perm], 1e-14, 1e-15) and close(Sp, S[..., perm], 1e-14, 1e-15)


def test_state_norm_bound():
    rng = np.random.default_rng(26)
    p = rand_prepared(rng, [1], 2, 8, 8)
    S = p["s0"].copy()
    for t in range(40):
        q = dict(p, q=_unit(rng, (1, 2, 8)), k=_unit(rng, (1, 2, 8)), v=rng.standard_normal((1, 2, 8)),
                 la=-np.exp(rng.uniform(-5, 0, (1, 2, 8))), beta=expit(rng.standard_normal((1, 2))), s0=S)
        _, Sn = run_oracle(ORC, q)
        bound = np.linalg.norm(S, axis=(2, 3)) + q["beta"][0] * np.linalg.norm(q["v"][0], axis=-1)
        assert np.all(np.linalg.norm(Sn, axis=(2, 3)) <= bound * (1 + 1e-12))
        S = Sn


# ----------------------------------------------------------------------------
# conv / gate properties and compositions on raw inputs
# ----------------------------------------------------------------------------
def test_conv_identity_taps_and_causality():
    rng = np.random.default_rng(30)
    x = rng.standard_normal((20, 5))
    cu = np.array([0, 20], np.int32)
    w = np.zeros((5, 4))
    w[:, 3] = 1.0
    y, _ = ORC.conv(x, w, cu, O.ACT_NONE)
    assert np.array_equal(y, x)
    w = rng.standard_normal((5, 4))
    y0, _ = ORC.conv(x, w, cu, O.ACT_SILU)
    x2 = x.copy()
    x2[8, 2] += 1.0
    y2, _ = ORC.conv(x2, w, cu, O.ACT_SILU)
    changed = np.argwhere(y2 != y0)
    assert set(changed[:, 0]) <= {8, 9, 10, 11} and set(changed[:, 1]) == {2}


def test_conv_no_leak_across_sequences():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((30, 4))
    cu = np.array([0, 13, 30], np.int32)
    w = rng.standard_normal((4, 4))
    y0, _ = ORC.conv(x, w, cu)
    x2 = x.copy()
    x2[:13] = rng.standard_normal((13, 4))
    y2, _ = ORC.conv(x2, w, cu)
    assert np.array_equal(y0[13:], y2[13:])


def _slice_seq(inp, lo, hi):
    out = dict(inp)
    for key in ("q_raw", "k_raw", "v_raw", "beta_logit", "log_alpha", "gate_logit"):
        out[key] = inp[key][lo:hi]
    out["T"] = hi - lo
    out["lengths"] = [hi - lo]
    out["cu_seqlens"] = np.array([0, hi - lo], np.int32)
    return out


def test_split_prefill_equals_whole():
    import torch
    inp = ki.prefill_inputs(32, [45], H=2, d=8, K=4, dtype=torch.bfloat16, cache_std=1.0)
    whole = ORC.prefill(inp)
    for t1 in (1, 2, 20, 44):
        a = ORC.prefill(_slice_seq(inp, 0, t1))
        b = ORC.prefill(_slice_seq(inp, t1, 45), s0=a["final_state"], cache_in=a["conv_cache"])
        assert close(np.concatenate([a["y"], b["y"]]), whole["y"], 1e-11, 1e-13)
        assert close(b["final_state"], whole["final_state"], 1e-11, 1e-13)
        assert np.array_equal(b["conv_cache"], whole["conv_cache"])


def test_packed_equals_separate():
    import torch
    inp = ki.prefill_inputs(33, [17, 0, 3, 40], H=2, d=8, K=4, dtype=torch.bfloat16, cache_std=1.0)
    whole = ORC.prefill(inp)
    cu = inp["cu_seqlens"].numpy()
    for n in range(4):
        part = _slice_seq(inp, cu[n], cu[n + 1])
        part["initial_state"] = inp["initial_state"][n:n + 1]
        part["conv_cache"] = inp["conv_cache"][n:n + 1]
        part["N"] = 1
        r = ORC.prefill(part)
        assert close(r["y"], whole["y"][cu[n]:cu[n + 1]], 1e-13, 1e-15)
        assert close(r["final_state"][0], whole["final_state"][n], 1e-13, 1e-15)
        assert np.array_equal(r["conv_cache"][0], whole["conv_cache"][n])
    # an empty sequence passes its state and cache through
    assert np.array_equal(whole["final_state"][1], inp["initial_state"][1].double().numpy())
    assert np.array_equal(whole["conv_cache"][1], inp["conv_cache"][1].double().numpy())


def test_thread_count_does_not_change_results():
    """Heads run in parallel; the per-head arithmetic is the same on any
    number of threads, so one thread and several give identical bits."""
    import torch
    inp = ki.prefill_inputs(34, [30, 9], H=4, d=8, K=3, dtype=torch.bfloat16)
    threads = ORC.num_threads()
    try:
        ORC.set_num_threads(1)
        one = ORC.prefill(inp)
        ORC.set_num_threads(4)
        many = ORC.prefill(inp)
    finally:
        ORC.set_num_threads(threads)
    for key in ("y", "final_state", "conv_cache"):
        assert np.array_equal(one[key], many[key]), key


def test_decode_slot_remap():
    import torch
    dec = ki.decode_inputs(34, 3, H=2, d=8, K=4, steps=2, dtype=torch.bfloat16, n_slots=5,
                           slot_perm=True, state_std=0.1)
    si = dec["slot_idx"].numpy()
    st_a = dec["state"].double().numpy().copy()
    ca_a = dec["conv_cache"].double().numpy().copy()
    st_b = np.ascontiguousarray(st_a[si])
    ca_b = np.ascontiguousarray(ca_a[si])
    for step in dec["steps"]:
        ya = ORC.decode_step(st_a, ca_a, dec["conv_w"], step, slot_idx=si)
        yb = ORC.decode_step(st_b, ca_b, dec["conv_w"], step)
        assert np.array_equal(ya, yb)
    assert np.array_equal(st_a[si], st_b) and np.array_equal(ca_a[si], ca_b)
    untouched = np.setdiff1d(np.arange(5), si)
    assert np.array_equal(st_a[untouched], dec["state"].double().numpy()[untouched])


def test_golden_tiny_workload():
    """Regression fixture for the tiny fp32 workload, written by
    tests/golden/make_golden.py (which calls only the oracle)."""
    with open(os.path.join(GOLDEN, "tiny_fp32_oracle.json")) as f:
        g = json.load(f)
    r = ORC.prefill(ki.config_prefill(0))
    assert close(r["y"], np.array(g["y"]), 1e-13, 1e-15)
    assert close(r["final_state"], np.array(g["final_state"]), 1e-13, 1e-15)


# ----------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ----------------------------------------------------------------------------
MUTANTS = {
    "decay_sign": ("const double a = exp(la[i]);", "const double a = exp(-la[i]);"),
    "decay_col_index": ("for (int j = 0; j < dv; ++j) S[(long)i * dv + j] *= a;",
                        "for (int j = 0; j < dv; ++j) S[(long)i * dv + j] *= exp(la[j % dk]);"),
    "dropped_delta": ("(v[j] - kTD[j])", "(v[j])"),
    "update_sign": ("S[(long)i * dv + j] += beta * k[i]", "S[(long)i * dv + j] -= beta * k[i]"),
    "beta_twice": ("+= beta * k[i] * (v[j]", "+= beta * beta * k[i] * (v[j]"),
    "output_reads_k": ("acc += S[(long)i * dv + j] * q[i];", "acc += S[(long)i * dv + j] * k[i];"),
    "transposed_readout": ("acc += S[(long)i * dv + j] * q[i];",
                           "acc += S[(long)(j % dk) * dv + (i % dv)] * q[i];"),
    "gate_dropped": ("(g ? g[j] : 1.0)", "(1.0)"),
    "conv_tap_shift": ("XS(t - K + 1 + j, c)", "XS(t - K + j, c)"),
    "cache_order": ("cin[(long)((K - 1) - (start - (tau))) * C + (c)]", "cin[(long)((start - (tau)) - 1) * C + (c)]"),
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    "l2_no_sqrt": ("1.0 / sqrt(ss + eps)", "1.0 / (ss + eps)"),
}


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    src = open(O.SRC).read()
    d = tmp_path_factory.mktemp("mutants")
    libs = {}
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        ms = d / f"{name}.c"
        ms.write_text(src.replace(old, new))
        libs[name] = O.build(str(ms), str(d / f"lib{name}.so"))
    return libs


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(mutant_libs, name):
    orc = O.Oracle(mutant_libs[name])
    results = {p.__name__: bool(p(orc)) for p in PINS}
    assert not all(results.values()), f"mutant {name} passed every pin: {results}"
