"""Pins for the oracle's backward (reverse-mode gradient of the recurrence),
CPU only.

The pages print no gradient values, so the pins come from elsewhere:

* central finite differences of the oracle's own forward (which the forward
  pins already tie to the defining matrix recurrence), on tiny packed inputs
  with several sequences, a gate, an initial state and a final-state gradient;
* torch.autograd (fp64) through the recurrence written as dense matrices,
  S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T;
* a closed form: with beta = 0 and alpha = 1 the state never changes, so
  dq_t = scale S0 (dy_t g_t), dS0 = dS_T + scale sum_t q_t (dy_t g_t)^T,
  dv = dk = 0, dlog alpha_t = rowsum(dS_t (.) S0) and
  dbeta_t = (dS_t^T k_t) . (v_t - S0^T k_t), with
  dS_t = dS_T + scale sum_{s >= t} q_s (dy_s g_s)^T;
* planted mistakes in a copy of the backward each fail a pin.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle as O

ORC = O.get()
KEYS = ("q", "k", "v", "la", "beta", "gate", "s0")
GRAD = {"q": "dq", "k": "dk", "v": "dv", "la": "dla", "beta": "dbeta", "gate": "dgate", "s0": "ds0"}


def tiny(seed, lengths=(3, 0, 5), H=2, dk=3, dv=2, gate=True):
    rng = np.random.default_rng(seed)
    T, N = sum(lengths), len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    p = dict(q=rng.standard_normal((T, H, dk)), k=rng.standard_normal((T, H, dk)) * 0.7,
             v=rng.standard_normal((T, H, dv)), la=-np.exp(rng.uniform(-3, 0, (T, H, dk))),
             beta=expit(rng.standard_normal((T, H))), gate=expit(rng.standard_normal((T, H, dv))) if gate else None,
             s0=rng.standard_normal((N, H, dk, dv)) * 0.3, cu=cu)
    dy = rng.standard_normal((T, H, dv))
    dsf = rng.standard_normal((N, H, dk, dv))
    return p, dy, dsf


def loss(orc, p, dy, dsf, scale):
    y, S = orc.recurrence(p["q"], p["k"], p["v"], p["la"], p["beta"], p["gate"], p["cu"], scale, p["s0"])
    return float((y * dy).sum() + (S * dsf).sum())


def finite_difference_ok(orc, seed=0, scale=0.7, gate=True, tol=1e-6):
    p, dy, dsf = tiny(seed, gate=gate)
    g = orc.recurrence_backward(p["q"], p["k"], p["v"], p["la"], p["beta"], p["gate"], p["cu"], dy, dsf,
                                scale, p["s0"])
    h = 1e-6
    for key in KEYS:
        if p[key] is None:
            continue
        num = np.zeros_like(p[key])
        for idx in np.ndindex(p[key].shape):
            orig = p[key][idx]
            p[key][idx] = orig + h
            lp = loss(ORC, p, dy, dsf, scale)   # the forward is the default oracle's
            p[key][idx] = orig - h
            lm = loss(ORC, p, dy, dsf, scale)
            p[key][idx] = orig
            num[idx] = (lp - lm) / (2 * h)
        got = g[GRAD[key]]
        if not np.allclose(got, num, rtol=tol, atol=tol):
            return False
    return True


def autograd_ok(orc, seed=1, scale=1.3):
    p, dy, dsf = tiny(seed, lengths=(4, 2), H=1, dk=4, dv=3)
    t = {k_: torch.tensor(p[k_], dtype=torch.float64, requires_grad=True) for k_ in KEYS}
    cu = p["cu"]
    T, H, dk = p["q"].shape
    ys, Ss = [], []
    for n in range(len(cu) - 1):
        for hh in range(H):
            S = t["s0"][n, hh]
            for s in range(cu[n], cu[n + 1]):
                k = t["k"][s, hh]
                M = (torch.eye(dk, dtype=torch.float64) - t["beta"][s, hh] * torch.outer(k, k)) @ torch.diag(
                    torch.exp(t["la"][s, hh]))
                S = M @ S + t["beta"][s, hh] * torch.outer(k, t["v"][s, hh])
                ys.append((scale * (S.T @ t["q"][s, hh]) * t["gate"][s, hh] * torch.tensor(dy[s, hh])).sum())
            Ss.append((S * torch.tensor(dsf[n, hh])).sum())
    torch.stack(ys + Ss).sum().backward()
    g = orc.recurrence_backward(p["q"], p["k"], p["v"], p["la"], p["beta"], p["gate"], p["cu"], dy, dsf,
                                scale, p["s0"])
    return all(np.allclose(g[GRAD[k_]], t[k_].grad.numpy(), rtol=1e-10, atol=1e-12) for k_ in KEYS)


def closed_form_ok(orc, seed=2, scale=0.9):
    p, dy, dsf = tiny(seed, lengths=(6,), H=1, dk=3, dv=4)
    p["beta"][:] = 0.0
    p["la"][:] = 0.0
    g = orc.recurrence_backward(p["q"], p["k"], p["v"], p["la"], p["beta"], p["gate"], p["cu"], dy, dsf,
                                scale, p["s0"])
    S0, q, k, v, gt = p["s0"][0, 0], p["q"][:, 0], p["k"][:, 0], p["v"][:, 0], p["gate"][:, 0]
    do = dy[:, 0] * gt
    dS = dsf[0, 0] + scale * q.T @ do
    ok = np.allclose(g["ds0"][0, 0], dS, atol=1e-12)
    ok &= np.allclose(g["dq"][:, 0], scale * do @ S0.T, atol=1e-12)
    ok &= np.allclose(g["dv"], 0.0) and np.allclose(g["dk"], 0.0)
    for s in range(6):
        dSs = dsf[0, 0] + scale * q[s:].T @ do[s:]
        ok &= np.isclose(g["dbeta"][s, 0], (dSs.T @ k[s]) @ (v[s] - S0.T @ k[s]), atol=1e-12)
        ok &= np.allclose(g["dla"][s, 0], (dSs * S0).sum(axis=1), atol=1e-12)
    return bool(ok)


PINS = [finite_difference_ok, autograd_ok, closed_form_ok]


def test_finite_differences():
    assert finite_difference_ok(ORC)


def test_finite_differences_no_gate():
    assert finite_difference_ok(ORC, seed=5, gate=False)


def test_autograd():
    assert autograd_ok(ORC)


def test_closed_form_beta0_alpha1():
    assert closed_form_ok(ORC)


MUTANTS = {
    "dP_missing_rank1": ("dP[e] = dS[e] + kt[i] * dw[j];", "dP[e] = dS[e];"),
    "dw_sign": ("dw[j] = -bt * du[j];", "dw[j] = bt * du[j];"),
    "dS_not_decayed": ("dS[(long)i * dv + j] = a * dP[(long)i * dv + j];", "dS[(long)i * dv + j] = dP[(long)i * dv + j];"),
    "dla_wrong_state": ("accd += dP[e] * Sp[e];", "accd += dP[e] * Sc[e];"),
    "dq_unscaled": ("dq[th * dk + i] = scale * acc;", "dq[th * dk + i] = acc;"),
    "dbeta_uses_v": ("db += du[j] * (vt[j] - w[j]);", "db += du[j] * vt[j];"),
    "dk_drops_P_term": ("acc += dS[e] * u[j] + a * Sp[e] * dw[j];", "acc += dS[e] * u[j];"),
    "gate_grad_from_dy": ("if (gt) dgate[th * dv + j] = dyt[j] * o[j];", "if (gt) dgate[th * dv + j] = dyt[j];"),
}


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    src = open(O.SRC).read()
    d = tmp_path_factory.mktemp("bwd_mutants")
    libs = {}
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        ms = d / f"{name}.c"
        ms.write_text(src.replace(old, new))
        libs[name] = O.build(str(ms), str(d / f"lib{name}.so"))
    return libs


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(mutant_libs, name):
    orc = O.Oracle(mutant_libs[name])
    results = {p.__name__: bool(p(orc)) for p in PINS}
    assert not all(results.values()), f"mutant {name} passed every pin: {results}"
