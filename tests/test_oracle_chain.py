"""Pin of the composed gradient: the oracle's recurrence gradient followed by
its prologue gradient gives the gradient of the whole prefill layer (raw
projections, conv taps and cache, log alpha, beta and gate logits, initial
state) with respect to loss = sum(dy * y) + sum(dS * final_state).  Each stage
is pinned on its own elsewhere; this checks that they compose, i.e. that the
recurrence's dbeta and dgate are gradients with respect to the sigmoid
outputs the prologue backward expects.  Central finite differences of the
oracle's forward prefill, every element, on a tiny packed batch.  CPU only."""
import numpy as np
import torch

import kda_inputs as ki
import oracle as O

ORC = O.get()
H, D, K = 1, 4, 2


def chain_grad(inp, dy, dsf):
    pro = ORC.prologue(inp)
    g = ORC.recurrence_backward(pro["q"], pro["k"], pro["v"], inp["log_alpha"], pro["beta"], pro["gate"],
                                inp["cu_seqlens"], dy, dsf, 1.0, inp["initial_state"])
    up = {k: torch.from_numpy(g[k]) for k in ("dq", "dk", "dv", "dbeta", "dgate")}
    raw = ORC.prologue_backward(inp, up)
    return dict(q_raw=raw["dq_raw"], k_raw=raw["dk_raw"], v_raw=raw["dv_raw"], conv_w=raw["dconv_w"],
                conv_cache=raw["dconv_cache"], beta_logit=raw["dbeta_logit"], gate_logit=raw["dgate_logit"],
                log_alpha=g["dla"], initial_state=g["ds0"])


def loss(inp, dy, dsf):
    r = ORC.prefill(inp)
    return float((r["y"] * dy.numpy()).sum() + (r["final_state"] * dsf.numpy()).sum())


def test_chained_gradient_matches_finite_differences():
    inp = ki.prefill_inputs(21, [4, 0, 3], H=H, d=D, K=K, dtype=torch.float32, cache_std=1.0)
    inp = {k: (v.double() if torch.is_tensor(v) and v.is_floating_point() else v) for k, v in inp.items()}
    g = torch.Generator().manual_seed(22)
    dy = torch.randn(inp["T"], H, D, generator=g).double()
    dsf = torch.randn(inp["N"], H, D, D, generator=g).double()
    ana = chain_grad(inp, dy, dsf)
    h = 1e-6
    for key, grad in ana.items():
        base = inp[key]
        num = np.zeros(base.numel())
        for i in range(base.numel()):
            plus, minus = base.clone(), base.clone()
            plus.view(-1)[i] += h
            minus.view(-1)[i] -= h
            num[i] = (loss({**inp, key: plus}, dy, dsf) - loss({**inp, key: minus}, dy, dsf)) / (2 * h)
        a = np.asarray(grad).reshape(-1)
        assert a.shape == num.shape, key
        err = float(np.abs(a - num).max()) / max(1.0, float(np.abs(num).max()))
        assert err < 1e-6, (key, err)
