"""CPU oracle for the KDA hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or executes anything here, and this
package never imports the product.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, token by token,
compiled with gcc); this module only compiles it, marshals numpy arrays and
composes its steps in the method's order:

    prefill:  conv+act (q, k, v)  ->  L2(q), L2(k)  ->  beta = sigmoid,
              gate = sigmoid  ->  recurrence  ->  y, final state, conv cache
    decode:   one more prefill token per row, state and conv cache in place
    backward: gradients of the recurrence with respect to q, k, v, log alpha,
              beta, gate and the initial state

Function citations are in ``kda_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")

ACT_NONE, ACT_SILU = 0, 1
L2_EPS = 1e-6  # KDA_L2_EPS reading (value not printed on the pages; 1e-6 as the tiny fp32 workload states)

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int32)


def build(src=SRC, out=LIB, extra=()):
    """Compile the oracle with gcc (OpenMP over independent heads)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor -> exact fp64 copy
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a, t=_D):
    return None if a is None else a.ctypes.data_as(t)


class Oracle:
    """Handle on one compiled oracle library (the default one, or a test build)."""

    def __init__(self, path=LIB):
        if not os.path.exists(path):
            if path != LIB:
                raise FileNotFoundError(path)
            build()
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.kda_oracle_num_threads.restype = ctypes.c_int
        L.kda_oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.kda_oracle_conv.argtypes = [ctypes.c_int, _I, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _D, _D, _D, _D, ctypes.c_long, _D]
        L.kda_oracle_l2norm.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_double, _D]
        L.kda_oracle_sigmoid.argtypes = [ctypes.c_long, _D, _D]
        L.kda_oracle_conv_backward.argtypes = [ctypes.c_int, _I, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               _D, _D, _D, ctypes.c_long, _D, _D, _D, _D]
        L.kda_oracle_l2norm_backward.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_double, _D, _D, _D]
        L.kda_oracle_sigmoid_backward.argtypes = [ctypes.c_long, _D, _D, _D]
        L.kda_oracle_recurrence.argtypes = [ctypes.c_int, _I, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            _D, _D, _D, _D, _D, _D, ctypes.c_double, _D, _D, _D]
        L.kda_oracle_recurrence_backward.argtypes = [ctypes.c_int, _I, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                     _D, _D, _D, _D, _D, _D, ctypes.c_double, _D, _D, _D,
                                                     _D, _D, _D, _D, _D, _D, _D]
        L.kda_oracle_decode_step.argtypes = [ctypes.c_int, _I, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                             _D, _D, _D, _D, _D, _D, _D, _D, _D, _D]
        L.kda_oracle_linear.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, _D, _D, _D]
        L.kda_oracle_log_decay.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, _D, _D, _D, _D]
        L.kda_oracle_mla_decode_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_double, _I, _D, _D, _D, _D,
                                                 _D, _D, _D]

    def num_threads(self):
        return int(self.lib.kda_oracle_num_threads())

    def set_num_threads(self, n):
        """Threads for later calls (timing only; the results do not depend on it)."""
        self.lib.kda_oracle_set_num_threads(int(n))

    # ---- single steps --------------------------------------------------
    def conv(self, x, w, cu, act=ACT_SILU, cache_in=None):
        """x [T, C], w [C, K], cu [N+1], cache_in None or [N, K-1, C].
        Returns (y [T, C], cache_out [N, K-1, C])."""
        x, w, cu, cache_in = _f64(x), _f64(w), _i32(cu), _f64(cache_in)
        T, C = x.shape
        K = w.shape[1]
        N = cu.shape[0] - 1
        y = np.zeros((T, C))
        cache_out = np.zeros((N, max(K - 1, 0), C))
        self.lib.kda_oracle_conv(N, _p(cu, _I), C, K, act, _p(x), _p(w), _p(cache_in),
                                 _p(cache_out) if K > 1 else None, (K - 1) * C, _p(y))
        return y, cache_out

    def l2norm(self, x, eps=L2_EPS):
        x = _f64(x).copy()
        d = x.shape[-1]
        self.lib.kda_oracle_l2norm(x.size // d, d, eps, _p(x))
        return x

    def sigmoid(self, x):
        x = _f64(x)
        y = np.empty_like(x)
        self.lib.kda_oracle_sigmoid(x.size, _p(x), _p(y))
        return y

    def recurrence(self, q, k, v, la, beta, gate, cu, scale=1.0, s0=None):
        """Prepared operands (normalised q, k; post-sigmoid beta and gate).
        q, k, la [T, H, dk]; v [T, H, dv]; beta [T, H]; gate None or [T, H, dv];
        s0 None or [N, H, dk, dv].  Returns (y [T, H, dv], S [N, H, dk, dv])."""
        q, k, v, la, beta, gate, s0 = map(_f64, (q, k, v, la, beta, gate, s0))
        cu = _i32(cu)
        T, H, dk = q.shape
        dv = v.shape[2]
        N = cu.shape[0] - 1
        y = np.zeros((T, H, dv))
        S = np.zeros((N, H, dk, dv))
        self.lib.kda_oracle_recurrence(N, _p(cu, _I), H, dk, dv, _p(q), _p(k), _p(v), _p(la),
                                       _p(beta), _p(gate), float(scale), _p(s0), _p(y), _p(S))
        return y, S

    def recurrence_backward(self, q, k, v, la, beta, gate, cu, dy, ds_final=None, scale=1.0, s0=None):
        """Gradients of recurrence(): dy [T, H, dv] on the outputs and ds_final
        None or [N, H, dk, dv] on the final states.  Returns a dict with dq, dk,
        dv, dla, dbeta, dgate (None without a gate) and ds0, shaped like the
        matching inputs."""
        q, k, v, la, beta, gate, s0, dy, ds_final = map(_f64, (q, k, v, la, beta, gate, s0, dy, ds_final))
        cu = _i32(cu)
        T, H, dk = q.shape
        dv = v.shape[2]
        N = cu.shape[0] - 1
        out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
                   dla=np.zeros((T, H, dk)), dbeta=np.zeros((T, H)),
                   dgate=np.zeros((T, H, dv)) if gate is not None else None, ds0=np.zeros((N, H, dk, dv)))
        self.lib.kda_oracle_recurrence_backward(
            N, _p(cu, _I), H, dk, dv, _p(q), _p(k), _p(v), _p(la), _p(beta), _p(gate), float(scale), _p(s0),
            _p(dy), _p(ds_final), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dla"]), _p(out["dbeta"]),
            _p(out["dgate"]), _p(out["ds0"]))
        return out

    def linear(self, x, w):
        """x [..., in] @ w[out, in]^T -> [..., out] (fp64 triple loop)."""
        x, w = _f64(x), _f64(w)
        lead = x.shape[:-1]
        rows = int(np.prod(lead)) if lead else 1
        out, inn = w.shape
        y = np.zeros((rows, out))
        self.lib.kda_oracle_linear(rows, inn, out, _p(np.ascontiguousarray(x.reshape(rows, inn))), _p(w), _p(y))
        return y.reshape(*lead, out)

    def log_decay(self, z, a_log=None, bias=None):
        """log alpha = -exp(a_log[h]) softplus(z + bias[h, c]); z [rows, H, d]."""
        z, a_log, bias = _f64(z), _f64(a_log), _f64(bias)
        rows, H, d = z.shape
        la = np.zeros_like(z)
        self.lib.kda_oracle_log_decay(rows, H, d, _p(z), _p(a_log), _p(bias), _p(la))
        return la

    def in_projection(self, x, w_in, H, d, a_log=None, bias=None):
        """The mixer's input projection of hidden states x [T, hidden] with
        w_in [5 H d + H, hidden], rows in the order q, k, v, gate, decay (each
        H d, head-major) and beta (H).  Returns q_raw, k_raw, v_raw,
        gate_logit [T, H, d], log_alpha [T, H, d] and beta_logit [T, H]."""
        y = self.linear(x, w_in)
        T = y.shape[0]
        C = H * d
        seg = lambda i: y[:, i * C:(i + 1) * C].reshape(T, H, d)
        return dict(q_raw=seg(0), k_raw=seg(1), v_raw=seg(2), gate_logit=seg(3),
                    log_alpha=self.log_decay(np.ascontiguousarray(seg(4)), a_log, bias),
                    beta_logit=y[:, 5 * C:5 * C + H])

    def mla_decode_step(self, q, k_new, v_new, k_cache, v_cache, cache_len, gate_logit=None, scale=None):
        """One MLA decode token (NoPE).  q [B, H, d_qk], k_new [B, H_kv, d_qk],
        v_new [B, H_kv, d_v], gate_logit [B, H, d_v] or None; k_cache
        [B, H_kv, max_len, d_qk] and v_cache [B, H_kv, max_len, d_v] must be
        float64 numpy arrays and are updated in place (the new token is written
        at cache_len[b]).  scale None = 1 / sqrt(d_qk).  Returns out
        [B, H, d_v]."""
        for c in (k_cache, v_cache):
            assert c.dtype == np.float64 and c.flags.c_contiguous
        q, kn, vn, gl = _f64(q), _f64(k_new), _f64(v_new), _f64(gate_logit)
        B, H, dqk = q.shape
        Hkv, L, dv = v_cache.shape[1], v_cache.shape[2], v_cache.shape[3]
        assert H % Hkv == 0 and k_cache.shape == (B, Hkv, L, dqk) and v_cache.shape[0] == B
        if scale is None:
            scale = 1.0 / np.sqrt(dqk)
        out = np.zeros((B, H, dv))
        self.lib.kda_oracle_mla_decode_step(B, H, Hkv, dqk, dv, L, float(scale), _p(_i32(cache_len), _I), _p(q),
                                            _p(kn), _p(vn), _p(gl), _p(k_cache), _p(v_cache), _p(out))
        return out

    # ---- composed paths ----------------------------------------------------
    def prologue(self, inp, act=ACT_SILU, eps=L2_EPS, cache_in=None):
        """Conv + act + L2 + gates on raw prefill inputs (dict from kda_inputs).
        cache_in: None = the dict's conv_cache, or an explicit [N, 3, K-1, H*d]."""
        H, d, K = inp["H"], inp["d"], inp["K"]
        T = inp["T"]
        cu = inp["cu_seqlens"]
        w = _f64(inp["conv_w"])
        cache = _f64(inp["conv_cache"] if cache_in is None else cache_in)
        outs, caches = [], []
        for X, key in enumerate(("q_raw", "k_raw", "v_raw")):
            y, c = self.conv(_f64(inp[key]).reshape(T, H * d), w[X], cu, act,
                             cache[:, X] if K > 1 else None)
            outs.append(y.reshape(T, H, d))
            caches.append(c)
        q = self.l2norm(outs[0], eps)
        k = self.l2norm(outs[1], eps)
        v = outs[2]
        beta = self.sigmoid(inp["beta_logit"])
        gate = self.sigmoid(inp["gate_logit"]) if inp.get("gate_logit") is not None else None
        cache_out = np.stack(caches, axis=1) if K > 1 else np.zeros((inp["N"], 3, 0, H * d))
        return dict(q=q, k=k, v=v, beta=beta, gate=gate, conv_cache=cache_out)

    def prologue_backward(self, inp, grads, act=ACT_SILU, eps=L2_EPS, cache_in=None):
        """Gradient of prologue() with respect to the raw inputs.  ``grads``
        holds dq, dk, dv [T, H, d], dbeta [T, H] and dgate [T, H, d] (or None):
        the gradients reaching the prologue's outputs.  Returns dq_raw, dk_raw,
        dv_raw [T, H, d], dconv_w [3, H*d, K], dconv_cache [N, 3, K-1, H*d] and
        dbeta_logit [T, H], dgate_logit [T, H, d] (None without a gate)."""
        H, d, K, T, N = inp["H"], inp["d"], inp["K"], inp["T"], inp["N"]
        C = H * d
        cu = _i32(inp["cu_seqlens"])
        w = _f64(inp["conv_w"])
        cache = _f64(inp["conv_cache"] if cache_in is None else cache_in)
        has_cache = K > 1
        out = dict(dconv_w=np.zeros((3, C, K)), dconv_cache=np.zeros((N, 3, max(K - 1, 0), C)))
        for X, (key, gkey) in enumerate((("q_raw", "dq"), ("k_raw", "dk"), ("v_raw", "dv"))):
            x = _f64(inp[key]).reshape(T, C)
            cin = np.ascontiguousarray(cache[:, X]) if has_cache else None
            dy = _f64(grads[gkey]).reshape(T, C)
            if X < 2:   # q and k were L2-normalised after the conv
                pre, _ = self.conv(x, w[X], inp["cu_seqlens"], act, cin)
                pre = np.ascontiguousarray(pre.reshape(T * H, d))
                dyn = np.empty_like(pre)
                self.lib.kda_oracle_l2norm_backward(T * H, d, eps, _p(pre), _p(np.ascontiguousarray(dy.reshape(T * H, d))),
                                                  _p(dyn))
                dy = dyn.reshape(T, C)
            dx = np.zeros((T, C))
            dw = np.zeros((C, K))
            dc = np.zeros((N, max(K - 1, 0), C)) if has_cache else None
            self.lib.kda_oracle_conv_backward(N, _p(cu, _I), C, K, act, _p(x), _p(np.ascontiguousarray(w[X])),
                                            _p(cin) if has_cache else None, (K - 1) * C, _p(np.ascontiguousarray(dy)),
                                            _p(dx), _p(dw), _p(dc) if has_cache else None)
            out["d" + key] = dx.reshape(T, H, d)
            out["dconv_w"][X] = dw
            if has_cache:
                out["dconv_cache"][:, X] = dc
        zb = _f64(inp["beta_logit"])
        dzb = np.empty_like(zb)
        self.lib.kda_oracle_sigmoid_backward(zb.size, _p(zb), _p(_f64(grads["dbeta"])), _p(dzb))
        out["dbeta_logit"] = dzb
        out["dgate_logit"] = None
        if inp.get("gate_logit") is not None and grads.get("dgate") is not None:
            zg = _f64(inp["gate_logit"])
            dzg = np.empty_like(zg)
            self.lib.kda_oracle_sigmoid_backward(zg.size, _p(zg), _p(_f64(grads["dgate"])), _p(dzg))
            out["dgate_logit"] = dzg
        return out

    def prefill(self, inp, act=ACT_SILU, eps=L2_EPS, scale=1.0, s0=None, cache_in=None):
        """Full prefill on raw inputs.  Returns dict with y, final_state,
        conv_cache and the prologue intermediates q, k, v, beta, gate."""
        pro = self.prologue(inp, act, eps, cache_in)
        y, S = self.recurrence(pro["q"], pro["k"], pro["v"], inp["log_alpha"], pro["beta"],
                               pro["gate"], inp["cu_seqlens"], scale,
                               inp["initial_state"] if s0 is None else s0)
        pro.update(y=y, final_state=S)
        return pro

    def decode_step(self, state, conv_cache, conv_w, step, slot_idx=None, act=ACT_SILU,
                    eps=L2_EPS, scale=1.0):
        """One decode step.  ``state`` [n_slots, H, d, d] and ``conv_cache``
        [n_slots, 3, K-1, H*d] must be float64 numpy arrays; both are
        updated in place.  ``step`` holds q_raw, k_raw, v_raw, log_alpha,
        beta_logit, gate_logit for [batch, H, d].  Returns y [batch, H, d]."""
        assert state.dtype == np.float64 and state.flags.c_contiguous
        assert conv_cache.dtype == np.float64 and conv_cache.flags.c_contiguous
        q, k, v = _f64(step["q_raw"]), _f64(step["k_raw"]), _f64(step["v_raw"])
        la, bl = _f64(step["log_alpha"]), _f64(step["beta_logit"])
        gl = _f64(step.get("gate_logit"))
        w = _f64(conv_w)
        B, H, d = q.shape
        K = w.shape[2]
        si = _i32(slot_idx)
        y = np.zeros((B, H, d))
        self.lib.kda_oracle_decode_step(B, _p(si, _I), H, d, K, act, eps, float(scale),
                                        _p(q), _p(k), _p(v), _p(w), _p(conv_cache), _p(state),
                                        _p(la), _p(bl), _p(gl), _p(y))
        return y


_default = None


def get():
    """The default oracle (compiled on first use if no build is present)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
