"""ctypes binding of libkda.so (declared in include/kda.h).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch provides device memory and the current stream.  If the library is
not built this module raises on first use; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
ACT = {"none": 0, "silu": 1}
CHUNK = 64
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE", 4: "KDA_ERR_UNSUPPORTED",
          5: "KDA_ERR_SEQLENS", 6: "KDA_ERR_WORKSPACE", 7: "KDA_ERR_ALIGN", 8: "KDA_ERR_HIP"}
EXPORTS = ("kda_prologue", "kda_chunk_workspace_bytes", "kda_chunk_forward", "kda_chunk_prepare",
           "kda_chunk_scan", "kda_prefill", "kda_prefill_prepare", "kda_prefill_scan", "kda_decode_step",
           "kda_chunk_backward_workspace_bytes", "kda_chunk_backward", "kda_prologue_backward_workspace_bytes",
           "kda_prologue_backward", "kda_prefill_noalloc", "kda_in_projection", "kda_out_projection",
           "kda_mixer_workspace_bytes", "kda_mixer_prefill", "kda_mla_decode_workspace_bytes",
           "kda_mla_decode_step", "kda_status_str", "kda_last_error_detail")


class KdaError(RuntimeError):
    def __init__(self, code, detail):
        super().__init__(f"{STATUS.get(code, code)}: {detail}")
        self.code = code
        self.detail = detail


class Geom(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("d", ctypes.c_int32), ("conv_k", ctypes.c_int32),
                ("act", ctypes.c_int32), ("l2_eps", ctypes.c_float), ("scale", ctypes.c_float)]


class MlaGeom(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("d_qk", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("scale", ctypes.c_float)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_lib = None


def load(path=LIB_PATH):
    """Load libkda.so and declare its prototypes (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m kimi_delta_attention_07_amd.build`")
    L = ctypes.CDLL(path)
    G = ctypes.POINTER(Geom)
    L.kda_prologue.argtypes = [G, _I, _I, _P, _P, _I] + [_P] * 13 + [_P]
    L.kda_prologue.restype = _I
    L.kda_chunk_workspace_bytes.argtypes = [G, _I, _I]
    L.kda_chunk_workspace_bytes.restype = ctypes.c_size_t
    L.kda_chunk_forward.argtypes = [G, _I, _I, _P, _P, _I, _I] + [_P] * 10 + [ctypes.c_size_t, _P]
    L.kda_chunk_forward.restype = _I
    L.kda_chunk_backward_workspace_bytes.argtypes = [G, _I, _I]
    L.kda_chunk_backward_workspace_bytes.restype = ctypes.c_size_t
    L.kda_chunk_backward.argtypes = [G, _I, _I, _P, _P, _I] + [_P] * 17 + [ctypes.c_size_t, _P]
    L.kda_chunk_backward.restype = _I
    L.kda_prologue_backward_workspace_bytes.argtypes = [G, _I]
    L.kda_prologue_backward_workspace_bytes.restype = ctypes.c_size_t
    L.kda_prologue_backward.argtypes = [G, _I, _I, _P, _P, _I] + [_P] * 20 + [ctypes.c_size_t, _P]
    L.kda_prologue_backward.restype = _I
    L.kda_chunk_prepare.argtypes = [G, _I, _I, _P, _P, _I] + [_P] * 6 + [ctypes.c_size_t, _P]
    L.kda_chunk_prepare.restype = _I
    L.kda_chunk_scan.argtypes = [G, _I, _I, _P, _P, _I] + [_P] * 5 + [ctypes.c_size_t, _P]
    L.kda_chunk_scan.restype = _I
    L.kda_prefill.argtypes = [G, _I, _I, _P, _P, _I, _I] + [_P] * 13 + [ctypes.c_size_t, _P]
    L.kda_prefill.restype = _I
    L.kda_prefill_prepare.argtypes = [G, _I, _I, _P, _P, _I] + [_P] * 9 + [ctypes.c_size_t, _P]
    L.kda_prefill_prepare.restype = _I
    L.kda_prefill_scan.argtypes = [G, _I, _I, _P, _P, _I] + [_P] * 5 + [ctypes.c_size_t, _P]
    L.kda_prefill_scan.restype = _I
    L.kda_prefill_noalloc.argtypes = [G, _I, _I, _P, _P, _I, _I] + [_P] * 12 + [_P]
    L.kda_prefill_noalloc.restype = _I
    L.kda_in_projection.argtypes = [G, _I, _I] + [_P] * 10 + [_P]
    L.kda_in_projection.restype = _I
    L.kda_out_projection.argtypes = [G, _I, _I, _P, _P, _P, _P]
    L.kda_out_projection.restype = _I
    L.kda_mixer_workspace_bytes.argtypes = [G, _I, _I]
    L.kda_mixer_workspace_bytes.restype = ctypes.c_size_t
    L.kda_mixer_prefill.argtypes = [G, _I, _I, _P, _P, _I] + [_P] * 12 + [ctypes.c_size_t, _P]
    L.kda_mixer_prefill.restype = _I
    L.kda_decode_step.argtypes = [G, _I, _P, _I, _I] + [_P] * 9 + [_I, _P, _P]
    L.kda_decode_step.restype = _I
    L.kda_status_str.argtypes = [_I]
    MG = ctypes.POINTER(MlaGeom)
    L.kda_mla_decode_workspace_bytes.argtypes = [MG, _I, _I]
    L.kda_mla_decode_workspace_bytes.restype = ctypes.c_size_t
    L.kda_mla_decode_step.argtypes = [MG, _I, _I] + [_P] * 9 + [ctypes.c_size_t, _P]
    L.kda_mla_decode_step.restype = _I
    L.kda_status_str.restype = ctypes.c_char_p
    L.kda_last_error_detail.argtypes = []
    L.kda_last_error_detail.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(code):
    if code != 0:
        raise KdaError(code, load().kda_last_error_detail().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libkda must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dtype(t):
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def geom(H, d, conv_k, act="silu", eps=1e-6, scale=1.0):
    return Geom(H, d, conv_k, ACT[act] if isinstance(act, str) else int(act), float(eps), float(scale))


def _host_cu(cu_seqlens, cu_seqlens_host):
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.to("cpu")
    h = cu_seqlens_host.to(torch.int32).contiguous()
    return h, ctypes.cast(h.data_ptr(), ctypes.c_void_p)


def prologue(q_raw, k_raw, v_raw, conv_w, cu_seqlens, beta_logit, gate_logit=None, conv_cache_in=None,
             conv_cache_out=None, *, act="silu", eps=1e-6, cu_seqlens_host=None, outs=None):
    """Short conv + activation + L2(q, k) + sigmoid gates.  Returns
    dict(q, k, v, beta, gate) (allocated unless ``outs`` supplies them)."""
    T, H, d = q_raw.shape
    K = conv_w.shape[2]
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    if outs is None:
        outs = dict(q=torch.empty_like(q_raw), k=torch.empty_like(k_raw), v=torch.empty_like(v_raw),
                    beta=torch.empty((T, H), dtype=torch.float32, device=q_raw.device),
                    gate=torch.empty_like(gate_logit) if gate_logit is not None else None)
    g = geom(H, d, K, act, eps)
    _check(load().kda_prologue(ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(q_raw), _ptr(q_raw),
                               _ptr(k_raw), _ptr(v_raw), _ptr(conv_w), _ptr(conv_cache_in), _ptr(conv_cache_out),
                               _ptr(beta_logit), _ptr(gate_logit), _ptr(outs["q"]), _ptr(outs["k"]),
                               _ptr(outs["v"]), _ptr(outs["beta"]), _ptr(outs["gate"]), _stream(q_raw)))
    return outs


def prologue_backward(q_raw, k_raw, v_raw, conv_w, cu_seqlens, beta_logit, gate_logit, conv_cache_in, dq, dk, dv,
                      dbeta, dgate=None, *, act="silu", eps=1e-6, cu_seqlens_host=None, want_dconv_cache=True,
                      workspace=None):
    """Gradients of prologue() with respect to its inputs, given fp32
    gradients dq, dk, dv, dbeta, dgate reaching its outputs.  Returns a dict
    with dq_raw, dk_raw, dv_raw, dconv_w, dconv_cache (None when not wanted or
    conv_k = 1), dbeta_logit and dgate_logit (None without a gate); fp32."""
    T, H, d = q_raw.shape
    K = conv_w.shape[2]
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    g = geom(H, d, K, act, eps)
    if workspace is None:
        nbytes = int(load().kda_prologue_backward_workspace_bytes(ctypes.byref(g), T))
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q_raw.device)
    f32 = dict(dtype=torch.float32, device=q_raw.device)
    out = dict(dq_raw=torch.empty((T, H, d), **f32), dk_raw=torch.empty((T, H, d), **f32),
               dv_raw=torch.empty((T, H, d), **f32), dconv_w=torch.empty(tuple(conv_w.shape), **f32),
               dconv_cache=torch.empty((n, 3, K - 1, H * d), **f32) if want_dconv_cache and K > 1 else None,
               dbeta_logit=torch.empty((T, H), **f32),
               dgate_logit=torch.empty((T, H, d), **f32) if gate_logit is not None else None)
    _check(load().kda_prologue_backward(
        ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(q_raw), _ptr(q_raw), _ptr(k_raw), _ptr(v_raw),
        _ptr(conv_w), _ptr(conv_cache_in), _ptr(beta_logit), _ptr(gate_logit), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dbeta), _ptr(dgate), _ptr(out["dq_raw"]), _ptr(out["dk_raw"]), _ptr(out["dv_raw"]),
        _ptr(out["dconv_w"]), _ptr(out["dconv_cache"]), _ptr(out["dbeta_logit"]), _ptr(out["dgate_logit"]),
        _ptr(workspace), workspace.numel(), _stream(q_raw)))
    return out


def chunk_workspace_bytes(H, d, cu_seqlens_host):
    """Workspace bytes for a batch shaped like ``cu_seqlens_host`` (the ABI
    sizes it from the sequence count and the token total only)."""
    h = cu_seqlens_host.to("cpu", torch.int32)
    g = geom(H, d, 4)
    return int(load().kda_chunk_workspace_bytes(ctypes.byref(g), h.numel() - 1, int(h[-1])))


def chunk_workspace(H, d, cu_seqlens_host, device):
    return torch.empty(chunk_workspace_bytes(H, d, cu_seqlens_host), dtype=torch.uint8, device=device)


def chunk_forward(q, k, v, log_alpha, beta, gate, cu_seqlens, initial_state=None, *, final_state=None,
                  out=None, scale=1.0, workspace=None, cu_seqlens_host=None, want_final_state=True):
    """Chunked prefill (d = 128, bf16).  Returns (out, final_state)."""
    T, H, d = q.shape
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    if workspace is None:
        workspace = chunk_workspace(H, d, hcu, q.device)
    if out is None:
        out = torch.empty_like(v)
    if final_state is None and want_final_state:
        final_state = torch.empty((n, H, d, d), dtype=torch.float32, device=q.device)
    g = geom(H, d, 4, scale=scale)
    _check(load().kda_chunk_forward(ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(q), CHUNK, _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(gate), _ptr(initial_state),
                                    _ptr(final_state), _ptr(out), _ptr(workspace), workspace.numel(), _stream(q)))
    return out, final_state


def chunk_backward_workspace_bytes(H, d, cu_seqlens_host):
    h = cu_seqlens_host.to("cpu", torch.int32)
    g = geom(H, d, 4)
    return int(load().kda_chunk_backward_workspace_bytes(ctypes.byref(g), h.numel() - 1, int(h[-1])))


def chunk_backward(q, k, v, log_alpha, beta, gate, cu_seqlens, dy, initial_state=None, d_final_state=None, *,
                   scale=1.0, workspace=None, cu_seqlens_host=None, want_d_initial_state=True):
    """Gradients of chunk_forward (d = 128, bf16 inputs; fp32 gradients).
    Returns a dict with dq, dk, dv, dlog_alpha, dbeta, dgate (None without a
    gate) and d_initial_state (None when not wanted)."""
    T, H, d = q.shape
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    if workspace is None:
        workspace = torch.empty(chunk_backward_workspace_bytes(H, d, hcu), dtype=torch.uint8, device=q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    g_out = dict(dq=torch.empty((T, H, d), **f32), dk=torch.empty((T, H, d), **f32),
                 dv=torch.empty((T, H, d), **f32), dlog_alpha=torch.empty((T, H, d), **f32),
                 dbeta=torch.empty((T, H), **f32), dgate=torch.empty((T, H, d), **f32) if gate is not None else None,
                 d_initial_state=torch.empty((n, H, d, d), **f32) if want_d_initial_state else None)
    g = geom(H, d, 4, scale=scale)
    _check(load().kda_chunk_backward(
        ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(q), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
        _ptr(beta), _ptr(gate), _ptr(initial_state), _ptr(dy), _ptr(d_final_state), _ptr(g_out["dq"]),
        _ptr(g_out["dk"]), _ptr(g_out["dv"]), _ptr(g_out["dlog_alpha"]), _ptr(g_out["dbeta"]), _ptr(g_out["dgate"]),
        _ptr(g_out["d_initial_state"]), _ptr(workspace), workspace.numel(), _stream(q)))
    return g_out


def chunk_prepare(q, k, v, log_alpha, beta, cu_seqlens, workspace, *, cu_seqlens_host=None):
    T, H, d = q.shape
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    g = geom(H, d, 4)
    _check(load().kda_chunk_prepare(ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(q), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(workspace), workspace.numel(),
                                    _stream(q)))


def chunk_scan(gate, cu_seqlens, workspace, out, initial_state=None, final_state=None, *, H, d=128, scale=1.0,
               cu_seqlens_host=None):
    T = out.shape[0]
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    g = geom(H, d, 4, scale=scale)
    _check(load().kda_chunk_scan(ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(out), _ptr(gate),
                                 _ptr(initial_state), _ptr(final_state), _ptr(out), _ptr(workspace),
                                 workspace.numel(), _stream(out)))


def prefill(q_raw, k_raw, v_raw, conv_w, log_alpha, beta_logit, gate_logit, cu_seqlens, initial_state=None,
            conv_cache_in=None, conv_cache_out=None, *, final_state=None, out=None, act="silu", eps=1e-6,
            scale=1.0, workspace=None, cu_seqlens_host=None, want_final_state=True):
    """Fused prefill from raw inputs (d = 128, bf16).  Returns (out, final_state)."""
    T, H, d = q_raw.shape
    K = conv_w.shape[2]
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    if workspace is None:
        workspace = chunk_workspace(H, d, hcu, q_raw.device)
    if out is None:
        out = torch.empty_like(v_raw)
    if final_state is None and want_final_state:
        final_state = torch.empty((n, H, d, d), dtype=torch.float32, device=q_raw.device)
    g = geom(H, d, K, act, eps, scale)
    _check(load().kda_prefill(ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(q_raw), CHUNK, _ptr(q_raw),
                              _ptr(k_raw), _ptr(v_raw), _ptr(conv_w), _ptr(conv_cache_in), _ptr(conv_cache_out),
                              _ptr(log_alpha), _ptr(beta_logit), _ptr(gate_logit), _ptr(initial_state),
                              _ptr(final_state), _ptr(out), _ptr(workspace), workspace.numel(), _stream(q_raw)))
    return out, final_state


def prefill_noalloc(q_raw, k_raw, v_raw, conv_w, log_alpha, beta_logit, gate_logit, cu_seqlens, initial_state=None,
                    conv_cache_in=None, conv_cache_out=None, *, final_state=None, out=None, act="silu", eps=1e-6,
                    scale=1.0, cu_seqlens_host=None, want_final_state=True):
    """prefill() through kda_prefill_noalloc: no workspace argument, the
    library's fixed per-GPU scratch instead (output tensors are still
    allocated here unless passed in).  Returns (out, final_state)."""
    T, H, d = q_raw.shape
    K = conv_w.shape[2]
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    if out is None:
        out = torch.empty_like(v_raw)
    if final_state is None and want_final_state:
        final_state = torch.empty((n, H, d, d), dtype=torch.float32, device=q_raw.device)
    g = geom(H, d, K, act, eps, scale)
    _check(load().kda_prefill_noalloc(ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(q_raw), CHUNK,
                                      _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(conv_w), _ptr(conv_cache_in),
                                      _ptr(conv_cache_out), _ptr(log_alpha), _ptr(beta_logit), _ptr(gate_logit),
                                      _ptr(initial_state), _ptr(final_state), _ptr(out), _stream(q_raw)))
    return out, final_state


def in_projection(x, w_in, H, d, a_log=None, dt_bias=None, *, outs=None):
    """The mixer's input projection of x [T, hidden] (bf16) with w_in
    [5 H d + H, hidden]: returns dict(q_raw, k_raw, v_raw, gate_logit,
    log_alpha [T, H, d], beta_logit [T, H]), bf16."""
    T, hidden = x.shape
    if outs is None:
        mk = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device=x.device)
        outs = dict(q_raw=mk(T, H, d), k_raw=mk(T, H, d), v_raw=mk(T, H, d), gate_logit=mk(T, H, d),
                    log_alpha=mk(T, H, d), beta_logit=mk(T, H))
    g = geom(H, d, 1)
    _check(load().kda_in_projection(ctypes.byref(g), T, hidden, _ptr(x), _ptr(w_in), _ptr(a_log), _ptr(dt_bias),
                                    _ptr(outs["q_raw"]), _ptr(outs["k_raw"]), _ptr(outs["v_raw"]),
                                    _ptr(outs["gate_logit"]), _ptr(outs["log_alpha"]), _ptr(outs["beta_logit"]),
                                    _stream(x)))
    return outs


def out_projection(y, w_out, *, out=None):
    """out [T, hidden] = y [T, H, d] (or [T, H d]) @ w_out^T, w_out [hidden, H d]; bf16."""
    T = y.shape[0]
    hidden, C = w_out.shape
    if out is None:
        out = torch.empty((T, hidden), dtype=torch.bfloat16, device=y.device)
    g = geom(1, C, 1)
    _check(load().kda_out_projection(ctypes.byref(g), T, hidden, _ptr(y), _ptr(w_out), _ptr(out), _stream(y)))
    return out


def mixer_workspace_bytes(H, d, n_seqs, total_tokens):
    g = geom(H, d, 4)
    return int(load().kda_mixer_workspace_bytes(ctypes.byref(g), n_seqs, total_tokens))


def mixer_prefill(x, w_in, w_out, conv_w, cu_seqlens, a_log=None, dt_bias=None, initial_state=None,
                  conv_cache_in=None, conv_cache_out=None, *, H, d=128, final_state=None, out=None, act="silu",
                  eps=1e-6, scale=1.0, workspace=None, cu_seqlens_host=None, want_final_state=True):
    """The KDA mixer on hidden states x [T, hidden]: input projection, the
    fused chunked prefill, output projection.  Returns (out [T, hidden] bf16,
    final_state)."""
    T, hidden = x.shape
    K = conv_w.shape[2]
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    if workspace is None:
        workspace = torch.empty(max(mixer_workspace_bytes(H, d, n, T), 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, hidden), dtype=torch.bfloat16, device=x.device)
    if final_state is None and want_final_state:
        final_state = torch.empty((n, H, d, d), dtype=torch.float32, device=x.device)
    g = geom(H, d, K, act, eps, scale)
    _check(load().kda_mixer_prefill(ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, hidden, _ptr(x), _ptr(w_in),
                                    _ptr(a_log), _ptr(dt_bias), _ptr(conv_w), _ptr(conv_cache_in),
                                    _ptr(conv_cache_out), _ptr(initial_state), _ptr(final_state), _ptr(w_out),
                                    _ptr(out), _ptr(workspace), workspace.numel(), _stream(x)))
    return out, final_state


def prefill_prepare(q_raw, k_raw, v_raw, conv_w, log_alpha, beta_logit, cu_seqlens, workspace, conv_cache_in=None,
                    conv_cache_out=None, *, act="silu", eps=1e-6, cu_seqlens_host=None):
    T, H, d = q_raw.shape
    K = conv_w.shape[2]
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    g = geom(H, d, K, act, eps)
    _check(load().kda_prefill_prepare(ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(q_raw), _ptr(q_raw),
                                      _ptr(k_raw), _ptr(v_raw), _ptr(conv_w), _ptr(conv_cache_in),
                                      _ptr(conv_cache_out), _ptr(log_alpha), _ptr(beta_logit), _ptr(workspace),
                                      workspace.numel(), _stream(q_raw)))


def prefill_scan(gate_logit, cu_seqlens, workspace, out, initial_state=None, final_state=None, *, H, d=128,
                 K=4, scale=1.0, cu_seqlens_host=None):
    T = out.shape[0]
    n = cu_seqlens.numel() - 1
    hcu, hptr = _host_cu(cu_seqlens, cu_seqlens_host)
    g = geom(H, d, K, scale=scale)
    _check(load().kda_prefill_scan(ctypes.byref(g), n, T, _ptr(cu_seqlens), hptr, _dtype(out), _ptr(gate_logit),
                                   _ptr(initial_state), _ptr(final_state), _ptr(out), _ptr(workspace),
                                   workspace.numel(), _stream(out)))


def decode_step(q_raw, k_raw, v_raw, conv_w, conv_cache, state, log_alpha, beta_logit, gate_logit=None,
                slot_idx=None, *, act="silu", eps=1e-6, scale=1.0, out=None, out_dtype=torch.float32):
    """One decode token per row; state and conv_cache updated in place.  Returns out [B, H, d]."""
    B, H, d = q_raw.shape
    K = conv_w.shape[2]
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype, device=q_raw.device)
    g = geom(H, d, K, act, eps, scale)
    _check(load().kda_decode_step(ctypes.byref(g), B, _ptr(slot_idx), state.shape[0], _dtype(q_raw), _ptr(q_raw),
                                  _ptr(k_raw), _ptr(v_raw), _ptr(conv_w), _ptr(conv_cache), _ptr(state),
                                  _ptr(log_alpha), _ptr(beta_logit), _ptr(gate_logit), _dtype(out), _ptr(out),
                                  _stream(q_raw)))
    return out


def mla_geom(H, H_kv, d_qk, d_v, scale=None):
    return MlaGeom(H, H_kv, d_qk, d_v, float(d_qk ** -0.5 if scale is None else scale))


def mla_decode_workspace_bytes(H, H_kv, d_qk, d_v, batch, max_len):
    g = mla_geom(H, H_kv, d_qk, d_v)
    return int(load().kda_mla_decode_workspace_bytes(ctypes.byref(g), batch, max_len))


def mla_decode_step(q, k_new, v_new, k_cache, v_cache, cache_len, gate_logit=None, *, scale=None, out=None,
                    workspace=None):
    """One MLA decode token (NoPE) for a batch: q [B, H, d_qk], k_new
    [B, H_kv, d_qk], v_new [B, H_kv, d_v], gate_logit [B, H, d_v] or None,
    caches [B, H_kv, max_len, d_qk / d_v], all bf16 on the device;
    cache_len [B] int32 on the device (tokens already cached; not advanced).
    Writes the new token into the caches and returns out [B, H, d_v] bf16."""
    B, H, dqk = q.shape
    Hkv, L, dv = v_cache.shape[1], v_cache.shape[2], v_cache.shape[3]
    g = mla_geom(H, Hkv, dqk, dv, scale)
    if workspace is None:
        workspace = torch.empty(max(mla_decode_workspace_bytes(H, Hkv, dqk, dv, B, L), 16), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.bfloat16, device=q.device)
    _check(load().kda_mla_decode_step(ctypes.byref(g), B, L, _ptr(cache_len), _ptr(q), _ptr(k_new), _ptr(v_new),
                                      _ptr(gate_logit), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(workspace),
                                      workspace.numel(), _stream(q)))
    return out
