"""The library's entry points inside HIP graphs (captured with torch's graph
API on its capture stream): the fused prefill, a 4-step KDA decode loop, an
MLA decode token and the whole KDA mixer.  Each graph is replayed three times with eager work and
synchronizations between the replays, and every replay must reproduce the
eager result bit for bit (same kernels, same inputs: deterministic).  The
library records no memset, allocation, copy or synchronization, so every
launch it makes can be captured.
"""
import pytest
import torch

import kda_inputs as ki
import kimi_delta_attention_07_amd as kda

pytestmark = pytest.mark.gpu


def _eager_noise(dev):
    """Unrelated eager work between replays (allocations, kernels, a sync)."""
    a = torch.randn(1 << 20, device=dev)
    b = (a * 3.0).sum()
    torch.cuda.synchronize()
    return float(b)


def test_prefill_graph_replays_match_eager():
    dev = torch.device("cuda")
    inp = ki.prefill_inputs(61, [300, 0, 129, 64], H=4, d=128, K=4, cache_std=1.0)
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    cu_h = inp["cu_seqlens"]
    ws = kda.chunk_workspace(4, 128, cu_h, dev)

    def call(y, S, cc):
        return kda.prefill(g["q_raw"], g["k_raw"], g["v_raw"], g["conv_w"], g["log_alpha"], g["beta_logit"],
                           g["gate_logit"], g["cu_seqlens"], g["initial_state"], g["conv_cache"], cc,
                           cu_seqlens_host=cu_h, workspace=ws, out=y, final_state=S)

    y0 = torch.empty(inp["T"], 4, 128, dtype=torch.bfloat16, device=dev)
    S0 = torch.empty(inp["N"], 4, 128, 128, dtype=torch.float32, device=dev)
    c0 = torch.empty_like(g["conv_cache"])
    call(y0, S0, c0)
    torch.cuda.synchronize()
    y1, S1, c1 = torch.full_like(y0, 7.0), torch.full_like(S0, 7.0), torch.full_like(c0, 7.0)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(y1, S1, c1)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        call(y1, S1, c1)
    for r in range(3):
        y1.fill_(7.0), S1.fill_(7.0), c1.fill_(7.0)
        _eager_noise(dev)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1, y0) and torch.equal(S1, S0) and torch.equal(c1, c0), f"replay {r}"


def test_decode_loop_graph_replays_match_eager():
    """Four consecutive kda_decode_step calls (state and conv cache updated in
    place) captured as one graph; before each replay the state and cache are
    reset eagerly."""
    dev = torch.device("cuda")
    dec = ki.decode_inputs(62, 16, H=4, d=128, K=4, steps=4)
    steps = [{k: v.to(dev) for k, v in st.items()} for st in dec["steps"]]
    cw = dec["conv_w"].to(dev)
    st0, ca0 = dec["state"].to(dev), dec["conv_cache"].to(dev)
    ys = [torch.empty(16, 4, 128, dtype=torch.float32, device=dev) for _ in steps]

    def loop(st, ca, outs):
        for s, o in zip(steps, outs):
            kda.decode_step(s["q_raw"], s["k_raw"], s["v_raw"], cw, ca, st, s["log_alpha"], s["beta_logit"],
                            s["gate_logit"], out=o)

    st_e, ca_e = st0.clone(), ca0.clone()
    loop(st_e, ca_e, ys)
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    st_g, ca_g = st0.clone(), ca0.clone()
    outs = [torch.empty_like(y) for y in ys]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        loop(st_g, ca_g, outs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop(st_g, ca_g, outs)
    for r in range(3):
        st_g.copy_(st0), ca_g.copy_(ca0)
        for o in outs:
            o.fill_(7.0)
        _eager_noise(dev)
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), f"replay {r}: outputs"
        assert torch.equal(st_g, st_e) and torch.equal(ca_g, ca_e), f"replay {r}: state, cache"


def test_mla_decode_graph_replays_match_eager():
    dev = torch.device("cuda")
    inp = ki.mla_inputs(63, 4, 8, 8, 192, 128, 600, len_range=(0, 599))
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    ws = torch.empty(kda.mla_decode_workspace_bytes(8, 8, 192, 128, 4, 600), dtype=torch.uint8, device=dev)
    kc_e, vc_e = g["k_cache"].clone(), g["v_cache"].clone()
    ref = kda.mla_decode_step(g["q"], g["k_new"], g["v_new"], kc_e, vc_e, g["cache_len"], g["gate_logit"],
                              workspace=ws)
    torch.cuda.synchronize()
    kc, vc = g["k_cache"].clone(), g["v_cache"].clone()
    out = torch.empty_like(ref)

    def call():
        kda.mla_decode_step(g["q"], g["k_new"], g["v_new"], kc, vc, g["cache_len"], g["gate_logit"], out=out,
                            workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        kc.copy_(g["k_cache"]), vc.copy_(g["v_cache"]), out.fill_(7.0)
        _eager_noise(dev)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(kc, kc_e) and torch.equal(vc, vc_e), f"replay {r}"


def test_mixer_prefill_graph_replays_match_eager():
    """The whole KDA mixer (input projection with its narrow beta-column
    kernel, the fused prefill, the output projection, whose tile width the
    launcher picks from the device's CU count) captured as one graph."""
    dev = torch.device("cuda")
    inp = ki.mixer_inputs(64, [300, 0, 77], 512, 4, 128, 4)
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    cu_h = inp["cu_seqlens"]
    ws = torch.empty(kda.mixer_workspace_bytes(4, 128, len(cu_h) - 1, inp["T"]), dtype=torch.uint8, device=dev)

    def call(out, S, cc):
        return kda.mixer_prefill(g["x"], g["w_in"], g["w_out"], g["conv_w"], g["cu_seqlens"], g["a_log"],
                                 g["dt_bias"], g["initial_state"], g["conv_cache"], cc, H=4, d=128,
                                 cu_seqlens_host=cu_h, workspace=ws, out=out, final_state=S)

    o0 = torch.empty(inp["T"], 512, dtype=torch.bfloat16, device=dev)
    S0 = torch.empty(inp["N"], 4, 128, 128, dtype=torch.float32, device=dev)
    c0 = torch.empty_like(g["conv_cache"])
    call(o0, S0, c0)
    torch.cuda.synchronize()
    o1, S1, c1 = torch.full_like(o0, 7.0), torch.full_like(S0, 7.0), torch.full_like(c0, 7.0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(o1, S1, c1)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o1, S1, c1)
    for r in range(3):
        o1.fill_(7.0), S1.fill_(7.0), c1.fill_(7.0)
        _eager_noise(dev)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o1, o0) and torch.equal(S1, S0) and torch.equal(c1, c0), f"replay {r}"
