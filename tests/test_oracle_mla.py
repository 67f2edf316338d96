"""Pins for the oracle's MLA decode token (CPU only).

The oracle appends the new token's k and v to the per-sequence cache, then
runs softmax attention of each head's q over every cached token and applies
the optional sigmoid output gate (kimi_k3 API docs, Functions:
mla_decode_token, gated_mla_attend; NoPE).  It is pinned here against
things other than itself:
  - torch's own CPU scaled_dot_product_attention in fp64 (an independent
    library implementation of SDPA, with its grouped-query mode and its
    causal mask for a whole sequence decoded token by token);
  - closed forms: one cached token gives v; identical keys give the mean of
    the values; two tokens give v0 + sigmoid(d) (v1 - v0), d the scaled score
    difference; scale 0 gives the plain mean;
  - invariants: permuting the cached tokens changes nothing; scores near
    1000 stay finite and pick the top key's value;
  - the cache write itself, and the out-of-range lengths it must skip.
Planted mistakes in the oracle's source must each fail one of the pins.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle as O

ORC = O.get()


def close(a, b, rtol=1e-12, atol=1e-12):
    return np.allclose(a, b, rtol=rtol, atol=atol)


def make(rng, B, H, Hkv, dqk, dv, L, lens, gate=True, kscale=1.0):
    q = rng.standard_normal((B, H, dqk))
    kn = rng.standard_normal((B, Hkv, dqk)) * kscale
    vn = rng.standard_normal((B, Hkv, dv))
    kc = rng.standard_normal((B, Hkv, L, dqk)) * kscale
    vc = rng.standard_normal((B, Hkv, L, dv))
    g = rng.standard_normal((B, H, dv)) if gate else None
    return q, kn, vn, kc, vc, np.array(lens, dtype=np.int32), g


def torch_sdpa(q, kc, vc, lens, g, scale):
    """Reference: torch's CPU SDPA (fp64) per sequence on the caches that
    already hold the new token, grouped-query mode, then the gate."""
    B, H, dqk = q.shape
    out = np.zeros((B, H, vc.shape[3]))
    for b in range(B):
        n = int(lens[b]) + 1
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b][None, :, None, :]), torch.from_numpy(np.ascontiguousarray(kc[b][None, :, :n])),
            torch.from_numpy(np.ascontiguousarray(vc[b][None, :, :n])), scale=scale,
            enable_gqa=True)[0, :, 0].numpy()
        out[b] = o * (expit(g[b]) if g is not None else 1.0)
    return out


def run(orc, q, kn, vn, kc, vc, lens, g, scale=None):
    kc, vc = kc.copy(), vc.copy()
    out = orc.mla_decode_step(q, kn, vn, kc, vc, lens, g, scale)
    return out, kc, vc


def pin_torch_sdpa(orc):
    """Random shapes, grouped heads (4 q heads on 2 kv heads), assorted
    cache lengths; the tiny K3Config MLA widths (2 heads, nope 4 + rope 4,
    v 4; the k3 README's Tutorial 3) and a production-like 192/128."""
    ok = True
    rng = np.random.default_rng(30)
    for B, H, Hkv, dqk, dv, L, lens in ((3, 4, 2, 16, 8, 40, [0, 17, 39]), (2, 2, 2, 8, 4, 16, [5, 15]),
                                        (2, 8, 1, 24, 12, 9, [8, 3]), (1, 4, 4, 192, 128, 70, [69])):
        q, kn, vn, kc, vc, lens, g = make(rng, B, H, Hkv, dqk, dv, L, lens)
        for gate in (g, None):
            for scale in (None, 0.3):
                out, kc2, vc2 = run(orc, q, kn, vn, kc, vc, lens, gate, scale)
                want = torch_sdpa(q, kc2, vc2, lens, gate, 1.0 / np.sqrt(dqk) if scale is None else scale)
                ok &= close(out, want)
    return ok


def pin_causal_sequence(orc):
    """Decoding a whole sequence token by token from an empty cache equals
    causal SDPA over the sequence (torch, is_causal), row by row."""
    rng = np.random.default_rng(31)
    T, H, Hkv, dqk, dv = 12, 4, 2, 8, 6
    Q = rng.standard_normal((T, H, dqk))
    Kx = rng.standard_normal((T, Hkv, dqk))
    Vx = rng.standard_normal((T, Hkv, dv))
    kc = np.full((1, Hkv, T, dqk), np.nan)   # never-written slots must never be read
    vc = np.full((1, Hkv, T, dv), np.nan)
    outs = []
    for t in range(T):
        outs.append(orc.mla_decode_step(Q[t][None], Kx[t][None], Vx[t][None], kc, vc, np.array([t], np.int32))[0])
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q.transpose(1, 0, 2).copy())[None], torch.from_numpy(Kx.transpose(1, 0, 2).copy())[None],
        torch.from_numpy(Vx.transpose(1, 0, 2).copy())[None], is_causal=True, enable_gqa=True)[0].numpy()
    return close(np.stack(outs), want.transpose(1, 0, 2)) and close(kc[0].transpose(1, 0, 2), Kx)


def pin_closed_forms(orc):
    rng = np.random.default_rng(32)
    ok = True
    # one cached token (the new one): softmax weight 1, out = v_new (gated)
    q, kn, vn, kc, vc, _, g = make(rng, 2, 4, 2, 8, 5, 6, [0, 0])
    out, _, _ = run(orc, q, kn, vn, kc, vc, np.array([0, 0], np.int32), g)
    ok &= close(out, np.repeat(vn, 2, axis=1) * expit(g))
    # identical keys: uniform weights, out = mean of the pos + 1 values
    q, kn, vn, kc, vc, _, _ = make(rng, 1, 2, 1, 8, 5, 10, [6], gate=False)
    kc[:] = kn[:, :, None, :]
    out, _, vc2 = run(orc, q, kn, vn, kc, vc, np.array([6], np.int32), None)
    ok &= close(out[0], np.repeat(vc2[0, :, :7].mean(axis=1), 2, axis=0))
    # two tokens: out = v0 + sigmoid(d) (v1 - v0), d = scale q.(k1 - k0)
    q, kn, vn, kc, vc, _, _ = make(rng, 1, 1, 1, 8, 5, 4, [1], gate=False)
    out, kc2, vc2 = run(orc, q, kn, vn, kc, vc, np.array([1], np.int32), None, 0.7)
    d = 0.7 * q[0, 0] @ (kc2[0, 0, 1] - kc2[0, 0, 0])
    ok &= close(out[0, 0], vc2[0, 0, 0] + expit(d) * (vc2[0, 0, 1] - vc2[0, 0, 0]))
    # scale 0: the plain mean
    q, kn, vn, kc, vc, _, _ = make(rng, 1, 3, 3, 8, 5, 9, [8], gate=False)
    out, _, vc2 = run(orc, q, kn, vn, kc, vc, np.array([8], np.int32), None, 0.0)
    ok &= close(out[0], vc2[0].mean(axis=1))
    # gate logit 0 halves the output
    q, kn, vn, kc, vc, _, _ = make(rng, 1, 2, 2, 8, 5, 9, [4], gate=False)
    a, _, _ = run(orc, q, kn, vn, kc, vc, np.array([4], np.int32), None)
    b, _, _ = run(orc, q, kn, vn, kc, vc, np.array([4], np.int32), np.zeros((1, 2, 5)))
    ok &= close(b, 0.5 * a)
    return ok


def pin_invariants(orc):
    rng = np.random.default_rng(33)
    ok = True
    # permuting the cached tokens (keys with their values) changes nothing
    q, kn, vn, kc, vc, lens, g = make(rng, 1, 2, 2, 8, 5, 12, [9])
    out, _, _ = run(orc, q, kn, vn, kc, vc, lens, g)
    perm = rng.permutation(9)
    kp, vp = kc.copy(), vc.copy()
    kp[:, :, :9], vp[:, :, :9] = kc[:, :, perm], vc[:, :, perm]
    outp, _, _ = run(orc, q, kn, vn, kp, vp, lens, g)
    ok &= close(out, outp)
    # scores near 1000 stay finite; one key far ahead of the others takes
    # all the weight
    q, kn, vn, kc, vc, lens, _ = make(rng, 1, 1, 1, 4, 3, 5, [4], gate=False)
    q[:] = 0.0
    q[0, 0, 0] = 1.0
    kc[0, 0, :, 0] = [900.0, 1000.0, 880.0, 950.0, 0.0]   # others at least e^-50 behind
    kn[0, 0, 0] = 920.0
    out, _, vc2 = run(orc, q, kn, vn, kc, vc, lens, None, 1.0)
    ok &= bool(np.isfinite(out).all()) and close(out[0, 0], vc2[0, 0, 1], 1e-8, 1e-8)
    return ok


def pin_cache_and_range(orc):
    rng = np.random.default_rng(34)
    q, kn, vn, kc, vc, _, g = make(rng, 4, 2, 2, 8, 5, 6, [0, 0, 0, 0])
    lens = np.array([3, 6, -1, 5], np.int32)   # 6 and -1 are outside [0, max_len)
    out, kc2, vc2 = run(orc, q, kn, vn, kc, vc, lens, g)
    ok = True
    for b, n in enumerate(lens):
        if 0 <= n < 6:
            ek, ev = kc.copy()[b], vc.copy()[b]
            ek[:, n], ev[:, n] = kn[b], vn[b]
            ok &= np.array_equal(kc2[b], ek) and np.array_equal(vc2[b], ev)
            ok &= bool(np.abs(out[b]).max() > 0)
        else:
            ok &= np.array_equal(kc2[b], kc[b]) and np.array_equal(vc2[b], vc[b]) and not out[b].any()
    return ok


PINS = [pin_torch_sdpa, pin_causal_sequence, pin_closed_forms, pin_invariants, pin_cache_and_range]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin(ORC)


MUTANTS = {
    "kv_head_modulo": ("const int hk = h / G;", "const int hk = h % H_kv;"),
    "no_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "new_token_excluded": ("for (int j = 0; j <= pos; ++j) {\n                double dot", "for (int j = 0; j < pos; ++j) {\n                double dot"),
    "no_max_shift": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "no_normalisation": ("o[c] = acc / den;", "o[c] = acc;"),
    "gate_sign": ("o[c] *= sigmoid(gate_logit[", "o[c] *= sigmoid(-gate_logit["),
    "append_one_late": ("+ hk) * max_len + pos) * d_qk;", "+ hk) * max_len + pos + 1) * d_qk;"),
    "value_stride": ("acc += s[j] * V[(long)j * d_v + c];", "acc += s[j] * V[(long)j * d_qk + c];"),
    "range_check_off_by_one": ("if (pos < 0 || pos >= max_len) {", "if (pos < 0 || pos > max_len) {"),
}


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    src = open(O.SRC).read()
    d = tmp_path_factory.mktemp("mla_mutants")
    libs = {}
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        ms = d / f"{name}.c"
        ms.write_text(src.replace(old, new))
        libs[name] = O.build(str(ms), str(d / f"lib{name}.so"))
    return libs


_CHILD = """
import sys, numpy as np
sys.path[:0] = [{root!r}, {tests!r}]
import oracle as O
import test_oracle_mla as T
orc = O.Oracle({lib!r})
res = []
for p in T.PINS:
    with np.errstate(all="ignore"):
        try:
            res.append(bool(p(orc)))
        except Exception:
            res.append(False)
print("PINS", int(all(res)))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(mutant_libs, name):
    """Each mutant runs the pins in a child process: a mutant that writes past
    a cache may crash it, which counts as caught."""
    import os
    import subprocess
    import sys
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _CHILD.format(root=os.path.dirname(tests), tests=tests, lib=str(mutant_libs[name]))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "OMP_NUM_THREADS": "1"})
    passed_all = r.returncode == 0 and "PINS 1" in r.stdout
    assert not passed_all, f"mutant {name} passed every pin"


def test_child_runner_passes_the_oracle():
    """Control for the mutant runner: the unmodified oracle passes every pin
    in the same child process, so a mutant's failure is the mutant's."""
    import os
    import subprocess
    import sys
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _CHILD.format(root=os.path.dirname(tests), tests=tests, lib=str(O.LIB))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "OMP_NUM_THREADS": "1"})
    assert r.returncode == 0 and "PINS 1" in r.stdout, r.stdout + r.stderr
