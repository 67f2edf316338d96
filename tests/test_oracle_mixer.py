"""Pins for the oracle's mixer maps (CPU only): the dense linear map, the
log-decay activation and the input projection's column layout.

The pages fix none of the values: the linear map is pinned by numpy's matmul
(an independent routine), the activation by numpy's logaddexp (softplus
written another way) and by closed forms, and the projection's layout by
weights built to copy chosen input channels into each output.  Planted
mistakes in the oracle's source must each fail one of these pins.
"""
import numpy as np
import pytest

import oracle as O

ORC = O.get()


def close(a, b, rtol=1e-12, atol=1e-13):
    return np.allclose(a, b, rtol=rtol, atol=atol)


def pin_linear(orc):
    rng = np.random.default_rng(20)
    ok = True
    # the tiny K3Config's widths (hidden 16, 2 heads of 4: 5*8+2 = 42 outputs),
    # an odd shape and a wider one
    for rows, inn, out in ((4, 16, 42), (7, 5, 3), (33, 96, 70)):
        x = rng.standard_normal((rows, inn))
        w = rng.standard_normal((out, inn))
        ok &= close(orc.linear(x, w), x @ w.T)
    x = rng.standard_normal((2, 3, 8))   # leading dims are rows
    w = rng.standard_normal((5, 8))
    ok &= close(orc.linear(x, w), x @ w.T)
    return ok


def pin_log_decay(orc):
    rng = np.random.default_rng(21)
    z = rng.standard_normal((6, 3, 4)) * 4
    a = rng.standard_normal(3)
    b = rng.standard_normal(12)
    want = -np.exp(a)[None, :, None] * np.logaddexp(0.0, z + b.reshape(3, 4)[None])
    ok = close(orc.log_decay(z, a, b), want)
    # no a_log, no bias: -softplus(z); z = 0 gives -log 2; very negative z a
    # decay near 1 (log alpha -> 0-), very positive z about -z
    ok &= close(orc.log_decay(np.zeros((1, 1, 1))), -np.log(2.0))
    zz = np.array([-60.0, -30.0, 0.5, 30.0, 60.0]).reshape(1, 1, 5)
    ok &= close(orc.log_decay(zz), -np.logaddexp(0.0, zz), 1e-14, 1e-300)
    la = orc.log_decay(rng.standard_normal((50, 2, 8)) * 10, rng.standard_normal(2), rng.standard_normal(16))
    ok &= bool((la <= 0).all())
    return ok


def pin_in_projection_layout(orc):
    """Weights that copy input channel j into output column j: every segment
    must then hold exactly its slice of x (q, k, v, gate, decay, beta)."""
    rng = np.random.default_rng(22)
    H, d, T = 2, 4, 5
    N = 5 * H * d + H
    x = rng.standard_normal((T, N))
    r = orc.in_projection(x, np.eye(N), H, d)
    C = H * d
    ok = True
    for i, key in enumerate(("q_raw", "k_raw", "v_raw", "gate_logit")):
        ok &= close(r[key], x[:, i * C:(i + 1) * C].reshape(T, H, d))
    ok &= close(r["log_alpha"], -np.logaddexp(0.0, x[:, 4 * C:5 * C].reshape(T, H, d)))
    ok &= close(r["beta_logit"], x[:, 5 * C:5 * C + H])
    return ok


PINS = [pin_linear, pin_log_decay, pin_in_projection_layout]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin(ORC)


MUTANTS = {
    "linear_transposed_weight": ("x[r * in + i] * w[(long)o * in + i]", "x[r * in + i] * w[(long)i * out + o]"),
    "linear_dropped_term": ("for (int i = 0; i < in; ++i) acc", "for (int i = 1; i < in; ++i) acc"),
    "softplus_sign": ("log1p(exp(-x)) : log1p(exp(x))", "log1p(exp(-x)) : log1p(exp(-x))"),
    "decay_scale_not_exp": ("a_log ? exp(a_log[h]) : 1.0", "a_log ? a_log[h] : 1.0"),
    "decay_bias_wrong_channel": ("(bias ? bias[h * d + c] : 0.0)", "(bias ? bias[c] : 0.0)"),
    "decay_sign": ("la[e] = -A * softplus(", "la[e] = A * softplus("),
}


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    src = open(O.SRC).read()
    d = tmp_path_factory.mktemp("mixer_mutants")
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
