"""Pins of the oracle's prologue gradient (conv + activation, L2 norm,
sigmoids, back to the raw projections, the conv taps and the incoming conv
cache).  The pages print no gradient values, so the pin is the definition of
a gradient: central finite differences of the oracle's own forward prologue,
checked for every input element on tiny packed batches (an empty sequence,
one shorter than the conv window, K = 1, 2 and 4, SiLU and no activation,
with and without a gate).  Planted mistakes in the gradient's source must
each fail it.  CPU only."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle as O

ORC = O.get()
H, D = 2, 4


def make(seed, lengths, K, gate=True):
    inp = ki.prefill_inputs(seed, lengths, H=H, d=D, K=K, dtype=torch.float32, cache_std=1.0)
    inp = {k: (v.double() if torch.is_tensor(v) and v.is_floating_point() else v) for k, v in inp.items()}
    if not gate:
        inp["gate_logit"] = None
    g = torch.Generator().manual_seed(seed + 1000)
    T = inp["T"]
    grads = dict(dq=torch.randn(T, H, D, generator=g).double(), dk=torch.randn(T, H, D, generator=g).double(),
                 dv=torch.randn(T, H, D, generator=g).double(), dbeta=torch.randn(T, H, generator=g).double(),
                 dgate=torch.randn(T, H, D, generator=g).double() if gate else None)
    return inp, grads


def loss(orc, inp, grads, act):
    """sum over the prologue's outputs of output * upstream gradient."""
    p = orc.prologue(inp, act=act)
    tot = sum(float((p[k] * grads["d" + k].numpy()).sum()) for k in ("q", "k", "v", "beta"))
    if grads["dgate"] is not None:
        tot += float((p["gate"] * grads["dgate"].numpy()).sum())
    return tot


# input key -> gradient key
PAIRS = dict(q_raw="dq_raw", k_raw="dk_raw", v_raw="dv_raw", beta_logit="dbeta_logit", gate_logit="dgate_logit",
             conv_w="dconv_w", conv_cache="dconv_cache")


def fd_check(orc, inp, grads, act, h=1e-6):
    """Largest relative mismatch between the analytic gradient and central
    differences, over every element of every input."""
    g = orc.prologue_backward(inp, grads, act=act)
    worst = 0.0
    for key, gkey in PAIRS.items():
        if inp.get(key) is None or (key == "conv_cache" and inp["K"] == 1):
            continue
        base = inp[key]
        ana = np.asarray(g[gkey]).reshape(-1)
        num = np.zeros(base.numel())
        for i in range(base.numel()):
            plus, minus = base.clone(), base.clone()
            plus.view(-1)[i] += h
            minus.view(-1)[i] -= h
            num[i] = (loss(orc, {**inp, key: plus}, grads, act) - loss(orc, {**inp, key: minus}, grads, act)) / (2 * h)
        scale = max(1.0, float(np.abs(num).max()))
        worst = max(worst, float(np.abs(ana - num).max()) / scale)
    return worst


CASES = [
    (11, [3, 0, 5], 4, O.ACT_SILU, True),
    (12, [1, 6], 2, O.ACT_SILU, False),
    (13, [4, 2], 1, O.ACT_SILU, True),
    (14, [5, 0, 2], 4, 0, True),
]


@pytest.mark.parametrize("seed,lengths,K,act,gate", CASES)
def test_prologue_gradient_matches_finite_differences(seed, lengths, K, act, gate):
    inp, grads = make(seed, lengths, K, gate)
    assert fd_check(ORC, inp, grads, act) < 1e-6


def test_no_gradient_reaches_an_unused_cache_slot():
    """A sequence with no history rows used by the conv (K = 1) has none; with
    K = 4 every slot of a non-empty sequence's incoming cache is used, and an
    empty sequence's cache gets none."""
    inp, grads = make(15, [0, 4], 4)
    g = ORC.prologue_backward(inp, grads)
    assert np.array_equal(g["dconv_cache"][0], np.zeros_like(g["dconv_cache"][0]))
    assert np.abs(g["dconv_cache"][1]).min() > 0


# planted mistakes in the gradient's source: each must fail the pin
MUTANTS = {
    "silu_derivative": ("g *= sg * (1.0 + pre * (1.0 - sg));", "g *= sg;"),
    "tap_index": ("dx[tau * C + c] += w[(long)c * K + j] * g;", "dx[tau * C + c] += w[(long)c * K + (K - 1 - j)] * g;"),
    "cache_slot": ("if (dcin) dcin[slot * C + c] += w[(long)c * K + j] * g;",
                   "if (dcin) dcin[(K - 2 - slot) * C + c] += w[(long)c * K + j] * g;"),
    "l2_cube": ("x[r * d + c] * xd / (nrm * nrm * nrm)", "x[r * d + c] * xd / (nrm * nrm)"),
    "sigmoid_slope": ("dz[i] = dy[i] * y * (1.0 - y);", "dz[i] = dy[i] * y;"),
}


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    src = open(O.SRC).read()
    d = tmp_path_factory.mktemp("prologue_bwd_mutants")
    libs = {}
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        ms = d / f"{name}.c"
        ms.write_text(src.replace(old, new))
        libs[name] = O.build(str(ms), str(d / f"lib{name}.so"))
    return libs


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prologue_gradient_mutant_is_caught(mutant_libs, name):
    orc = O.Oracle(mutant_libs[name])
    inp, grads = make(11, [3, 0, 5], 4)
    assert fd_check(orc, inp, grads, O.ACT_SILU) > 1e-3
