/*
 * KDA CPU oracle -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * Only the test suite, the package's smoke check and the benchmark's CPU
 * baseline leg may load this library.  It shares no code, header or constant
 * with the HIP implementation; the two meet only through seeded inputs.
 *
 * What it computes, in fp64, token by token, exactly as the method is defined
 * (page names below are the titles of the public pages this follows):
 *
 *  - Kimi Delta Attention per head, the gated delta rule with per-channel
 *    decay ("recurrent KDA state" in the implementation list of the forum post
 *    "Experimental Native Vulkan Backend for Kimi K3"; the fp32 recurrent KDA
 *    step of the "metrale_model_arch::kimi_k3" API docs, Constants):
 *        S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *        o_t = scale * S_t^T q_t,          y_t = o_t (.) gate_t
 *    S is dk x dv (row index = key channel), alpha_t = exp(log_alpha_t).
 *  - the independent short causal depthwise convolutions on q, k and v
 *    (forum post, implementation list), each followed by an activation
 *    (SiLU by default, or none);
 *  - L2 normalisation of q and k over the key channels with the epsilon the
 *    kimi_k3 API docs call KDA_L2_EPS (Constants), as x / sqrt(sum x^2 + eps);
 *  - beta = sigmoid(beta_logit) per (token, head) and the output gate
 *    sigmoid(gate_logit) per (token, head, value channel) ("KDA output
 *    gating", forum post, implementation list);
 *  - the gradient of the recurrence with respect to q, k, v, log alpha,
 *    beta, the gate and the initial state (reverse mode, token by token; the
 *    k3 README's functional proxy checks gradients of a KDA layer), and of
 *    the prologue (conv + activation, L2 norm, sigmoids) back to the raw
 *    projections, the conv taps and the incoming conv cache;
 *  - the decode step as conv update, then recurrent step (kimi_k3 API docs,
 *    Functions: kda_decode_token): one more prefill token that reads and
 *    rewrites the per-sequence conv cache and recurrent state in place (the
 *    docs' struct KdaState keeps both as fp32 read-modify-write buffers; fp64
 *    here).
 *
 *  - the KDA mixer's linear maps around the operator (the k3 README, "Use
 *    this repository as a template", puts the projections and the output gate
 *    in the KDA module): one projection of the hidden states to the raw q, k, v, the
 *    gate logits, the decay pre-activations and the beta logits, the decay
 *    log alpha = -exp(a_log[h]) * softplus(z + bias[channel]) (a reading: the
 *    pages do not say how log alpha comes from the projection; with a_log and
 *    bias absent it is -softplus(z), which maps any real onto log alpha <= 0),
 *    and the output projection back to the hidden size.
 *  - the MLA decode token (kimi_k3 API docs, Functions: mla_decode_token and
 *    gated_mla_attend): append the new token's k and v to the per-sequence
 *    cache, softmax attention of each head's q over every cached token, then
 *    the optional sigmoid output gate (NoPE: no rotary step).
 *
 * Readings taken where the pages are silent: conv tap K-1 multiplies the
 * current token, no conv bias, zero history at a sequence start unless a
 * cache is given, and the conv never crosses sequences; the output scale is
 * an explicit argument; nothing (no RMSNorm) follows the output gate.
 *
 * Layouts are row-major, last index fastest.  The ctypes prototypes live in
 * oracle/__init__.py, the only caller.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int kda_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of later parallel regions (heads run in parallel); n <= 0
 * leaves it unchanged.  Timing control only: results do not depend on it. */
void kda_oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static double activation(int act, double x) {
    /* act 1 = SiLU x*sigmoid(x); act 0 = identity */
    return act == 1 ? x * sigmoid(x) : x;
}

/*
 * Causal depthwise convolution of one stream over a packed batch.
 *   x        [T][C] raw inputs, sequences packed by cu_seqlens [n_seqs+1]
 *   w        [C][K] taps; y_t[c] = act( sum_j w[c][j] * x_{t-K+1+j}[c] )
 *   cache_in NULL or [n_seqs] x (K-1) x C at stride cache_stride between
 *            sequences: the K-1 raw inputs that precede each sequence,
 *            oldest first; NULL means zeros
 *   cache_out NULL or same layout: the last K-1 raw inputs of each sequence
 *            (reaching back into cache_in when the sequence is shorter)
 * cache_out may alias cache_in.
 */
void kda_oracle_conv(int n_seqs, const int32_t *cu, int C, int K, int act,
                     const double *x, const double *w,
                     const double *cache_in, double *cache_out, long cache_stride,
                     double *y) {
    for (int n = 0; n < n_seqs; ++n) {
        const long start = cu[n], end = cu[n + 1];
        const double *cin = cache_in ? cache_in + (long)n * cache_stride : NULL;
        /* history value of channel c at absolute token position tau */
#define XS(tau, c)                                                          \
    ((tau) >= start ? x[(long)(tau) * C + (c)]                              \
     : (cin && (start - (tau)) <= K - 1 ? cin[(long)((K - 1) - (start - (tau))) * C + (c)] \
        : 0.0))
#pragma omp parallel for schedule(static)
        for (int c = 0; c < C; ++c) {
            for (long t = start; t < end; ++t) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) acc += w[(long)c * K + j] * XS(t - K + 1 + j, c);
                y[t * C + c] = activation(act, acc);
            }
        }
        if (cache_out && K > 1) {
            double *tmp = (double *)malloc(sizeof(double) * (size_t)(K - 1) * (size_t)C);
            for (int j = 0; j < K - 1; ++j)
                for (int c = 0; c < C; ++c) tmp[(long)j * C + c] = XS(end - (K - 1) + j, c);
            memcpy(cache_out + (long)n * cache_stride, tmp, sizeof(double) * (size_t)(K - 1) * (size_t)C);
            free(tmp);
        }
#undef XS
    }
}

/* x[r][0..d) <- x / sqrt(sum x^2 + eps), for each of `rows` rows (in place) */
void kda_oracle_l2norm(long rows, int d, double eps, double *x) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int c = 0; c < d; ++c) ss += x[r * d + c] * x[r * d + c];
        const double inv = 1.0 / sqrt(ss + eps);
        for (int c = 0; c < d; ++c) x[r * d + c] *= inv;
    }
}

/* y[i] = sigmoid(x[i]) */
void kda_oracle_sigmoid(long n, const double *x, double *y) {
    for (long i = 0; i < n; ++i) y[i] = sigmoid(x[i]);
}

/*
 * Gradients of the prologue's steps (reverse mode, same conventions as the
 * forward functions above; they are what a caller needs to carry the
 * recurrence's gradient back to the raw projections and the conv taps).
 *
 * Convolution + activation: with pre_t[c] = sum_j w[c][j] x_{t-K+1+j}[c] and
 * y_t = act(pre_t), given dy:
 *   dpre_t = dy_t * act'(pre_t)    (SiLU: s (1 + pre (1 - s)), s = sigmoid(pre))
 *   dx_tau[c]   += w[c][j] dpre_t[c]       for tau = t-K+1+j inside the sequence
 *   dcache[c]   += w[c][j] dpre_t[c]       for tau before it (history slot
 *                                          (K-1) - (start - tau)), when a cache is given
 *   dw[c][j]    += x_tau[c] dpre_t[c]      (x_tau from the sequence or the cache)
 * dx and dw are accumulated into (the caller zeroes them); dcache_in (NULL:
 * skipped) has cache_in's layout and is written.  The outgoing cache copies
 * raw inputs and is taken to receive no gradient.
 */
void kda_oracle_conv_backward(int n_seqs, const int32_t *cu, int C, int K, int act,
                              const double *x, const double *w,
                              const double *cache_in, long cache_stride,
                              const double *dy, double *dx, double *dw, double *dcache_in) {
    for (int n = 0; n < n_seqs; ++n) {
        const long start = cu[n], end = cu[n + 1];
        const double *cin = cache_in ? cache_in + (long)n * cache_stride : NULL;
        double *dcin = dcache_in ? dcache_in + (long)n * cache_stride : NULL;
        if (dcin)
            for (long e = 0; e < (long)(K - 1) * C; ++e) dcin[e] = 0.0;
#pragma omp parallel for schedule(static)
        for (int c = 0; c < C; ++c) {
            for (long t = start; t < end; ++t) {
                double pre = 0.0;
                for (int j = 0; j < K; ++j) {
                    const long tau = t - K + 1 + j;
                    const double xv = tau >= start ? x[tau * C + c]
                                    : (cin ? cin[(long)((K - 1) - (start - tau)) * C + c] : 0.0);
                    pre += w[(long)c * K + j] * xv;
                }
                double g = dy[t * C + c];
                if (act == 1) {
                    const double sg = sigmoid(pre);
                    g *= sg * (1.0 + pre * (1.0 - sg));
                }
                for (int j = 0; j < K; ++j) {
                    const long tau = t - K + 1 + j;
                    if (tau >= start) {
                        dx[tau * C + c] += w[(long)c * K + j] * g;
                        dw[(long)c * K + j] += x[tau * C + c] * g;
                    } else if (cin) {
                        const long slot = (K - 1) - (start - tau);
                        if (dcin) dcin[slot * C + c] += w[(long)c * K + j] * g;
                        dw[(long)c * K + j] += cin[slot * C + c] * g;
                    }
                }
            }
        }
    }
}

/* L2 norm: with n = sqrt(sum x^2 + eps) and y = x / n, given dy (x is the
 * un-normalised input): dx = dy / n - x (x . dy) / n^3, for each row */
void kda_oracle_l2norm_backward(long rows, int d, double eps, const double *x, const double *dy, double *dx) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        double ss = 0.0, xd = 0.0;
        for (int c = 0; c < d; ++c) {
            ss += x[r * d + c] * x[r * d + c];
            xd += x[r * d + c] * dy[r * d + c];
        }
        const double nrm = sqrt(ss + eps);
        for (int c = 0; c < d; ++c) dx[r * d + c] = dy[r * d + c] / nrm - x[r * d + c] * xd / (nrm * nrm * nrm);
    }
}

/* sigmoid: y = sigmoid(z), given dy: dz = dy y (1 - y) */
void kda_oracle_sigmoid_backward(long n, const double *z, const double *dy, double *dz) {
    for (long i = 0; i < n; ++i) {
        const double y = sigmoid(z[i]);
        dz[i] = dy[i] * y * (1.0 - y);
    }
}

/*
 * One token of the recurrence on a dk x dv state S (row-major, in place):
 *   D  = Diag(alpha) S                     (alpha = exp(la))
 *   S' = D - beta k (k^T D) + beta k v^T   = (I - beta k k^T) D + beta k v^T
 *   o  = scale S'^T q;  y = o (.) g  (g NULL: no gate)
 */
static void token_step(double *S, int dk, int dv, const double *q, const double *k,
                       const double *v, const double *la, double beta, const double *g,
                       double scale, double *kTD, double *y) {
    for (int i = 0; i < dk; ++i) {
        const double a = exp(la[i]);
        for (int j = 0; j < dv; ++j) S[(long)i * dv + j] *= a;
    }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += k[i] * S[(long)i * dv + j];
        kTD[j] = acc;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(long)i * dv + j] += beta * k[i] * (v[j] - kTD[j]);
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * q[i];
        y[j] = scale * acc * (g ? g[j] : 1.0);
    }
}

/*
 * The recurrence over a packed batch, on already-prepared operands:
 *   q, k [T][H][dk] (normalised), v [T][H][dv], la [T][H][dk] (log alpha),
 *   beta [T][H], gate NULL or [T][H][dv] (post-sigmoid),
 *   s0 NULL (zeros) or [n_seqs][H][dk][dv];  y [T][H][dv];
 *   s_final NULL or [n_seqs][H][dk][dv] (may alias s0).
 * Sequences and heads are independent and run in parallel; within one
 * (sequence, head) the tokens run strictly in order.
 */
void kda_oracle_recurrence(int n_seqs, const int32_t *cu, int H, int dk, int dv,
                           const double *q, const double *k, const double *v,
                           const double *la, const double *beta, const double *gate,
                           double scale, const double *s0, double *y, double *s_final) {
    const long SS = (long)dk * dv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < n_seqs; ++n) {
        for (int h = 0; h < H; ++h) {
            double *S = (double *)malloc(sizeof(double) * (size_t)SS);
            double *kTD = (double *)malloc(sizeof(double) * (size_t)dv);
            if (s0) memcpy(S, s0 + ((long)n * H + h) * SS, sizeof(double) * (size_t)SS);
            else memset(S, 0, sizeof(double) * (size_t)SS);
            for (long t = cu[n]; t < cu[n + 1]; ++t) {
                const long th = t * H + h;
                token_step(S, dk, dv, q + th * dk, k + th * dk, v + th * dv, la + th * dk,
                           beta[th], gate ? gate + th * dv : NULL, scale, kTD, y + th * dv);
            }
            if (s_final) memcpy(s_final + ((long)n * H + h) * SS, S, sizeof(double) * (size_t)SS);
            free(kTD);
            free(S);
        }
    }
}

/*
 * One decode step for `batch` rows (metrale kimi_k3 docs, kda_decode_token:
 * conv update, then recurrent step).  Row b works on slot s = slot_idx[b]
 * (identity when slot_idx is NULL; slots must be distinct):
 *   q_raw, k_raw, v_raw [batch][H][d] pre-conv inputs, la [batch][H][d],
 *   beta_logit [batch][H], gate_logit NULL or [batch][H][d];
 *   conv_w [3][H*d][K]; conv_cache [n_slots][3][K-1][H*d] and
 *   state [n_slots][H][d][d] are read and rewritten in place;  y [batch][H][d].
 * It is exactly one more prefill token for each row's sequence.
 */
void kda_oracle_decode_step(int batch, const int32_t *slot_idx, int H, int d, int K, int act,
                            double eps, double scale, const double *q_raw, const double *k_raw,
                            const double *v_raw, const double *conv_w, double *conv_cache,
                            double *state, const double *la, const double *beta_logit,
                            const double *gate_logit, double *y) {
    const int C = H * d;
    const long cstride = 3L * (K - 1) * C;
    const int32_t cu1[2] = {0, 1};
    double *xq = (double *)malloc(sizeof(double) * (size_t)C);
    double *xk = (double *)malloc(sizeof(double) * (size_t)C);
    double *xv = (double *)malloc(sizeof(double) * (size_t)C);
    for (int b = 0; b < batch; ++b) {
        const long s = slot_idx ? slot_idx[b] : b;
        double *cache = conv_cache + s * cstride;
        const double *raw[3] = {q_raw + (long)b * C, k_raw + (long)b * C, v_raw + (long)b * C};
        double *out[3] = {xq, xk, xv};
        for (int X = 0; X < 3; ++X)
            kda_oracle_conv(1, cu1, C, K, act, raw[X], conv_w + (long)X * C * K,
                            K > 1 ? cache + (long)X * (K - 1) * C : NULL,
                            K > 1 ? cache + (long)X * (K - 1) * C : NULL, cstride, out[X]);
        kda_oracle_l2norm(H, d, eps, xq);
        kda_oracle_l2norm(H, d, eps, xk);
#pragma omp parallel for schedule(static)
        for (int h = 0; h < H; ++h) {
            double *kTD = (double *)malloc(sizeof(double) * (size_t)d);
            double *g = (double *)malloc(sizeof(double) * (size_t)d);
            const long bh = (long)b * H + h;
            if (gate_logit)
                for (int j = 0; j < d; ++j) g[j] = sigmoid(gate_logit[bh * d + j]);
            token_step(state + (s * H + h) * (long)d * d, d, d, xq + (long)h * d, xk + (long)h * d,
                       xv + (long)h * d, la + bh * d, sigmoid(beta_logit[bh]),
                       gate_logit ? g : NULL, scale, kTD, y + bh * d);
            free(g);
            free(kTD);
        }
    }
    free(xv);
    free(xk);
    free(xq);
}

/*
 * Reverse-mode gradient of kda_oracle_recurrence (the chunked KDA backward
 * that the k3 README's training proxy exercises: gradients of a KDA layer,
 * "Functional tiny proxy"), taken token by token from the same definition:
 *   P = Diag(alpha) S_{t-1},  w = P^T k,  u = beta (v - w),  S_t = P + k u^T,
 *   o = scale S_t^T q,  y = o (.) g.
 * Given dy [T][H][dv] and ds_final NULL (zeros) or [n][H][dk][dv] (the
 * gradient arriving at each final state), walking each sequence backwards:
 *   do = dy (.) g,  dg = dy (.) o,  dq = scale S_t do,  dS += scale q do^T,
 *   du = dS^T k,  dk = dS u,  dbeta = du . (v - w),  dv = beta du,
 *   dw = -beta du,  dP = dS + k dw^T,  dk += P dw,
 *   dla_i = alpha_i sum_j dP_ij S_{t-1,ij},  dS_{t-1} = Diag(alpha) dP.
 * The forward states S_0 .. S_L of a (sequence, head) are all kept, so this
 * is for the small sizes the tests use.  Outputs: dq, dk_ [T][H][dk],
 * dv_ [T][H][dv], dla [T][H][dk], dbeta [T][H], dgate [T][H][dv] (only
 * when gate is given), ds0 [n][H][dk][dv] (the gradient of the initial state).
 */
void kda_oracle_recurrence_backward(int n_seqs, const int32_t *cu, int H, int dk, int dv,
                                    const double *q, const double *k, const double *v,
                                    const double *la, const double *beta, const double *gate,
                                    double scale, const double *s0, const double *dy,
                                    const double *ds_final, double *dq, double *dk_, double *dv_,
                                    double *dla, double *dbeta, double *dgate, double *ds0) {
    const long SS = (long)dk * dv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < n_seqs; ++n) {
        for (int h = 0; h < H; ++h) {
            const long L = cu[n + 1] - cu[n];
            double *St = (double *)malloc(sizeof(double) * (size_t)((L + 1) * SS));
            double *dS = (double *)malloc(sizeof(double) * (size_t)SS);
            double *dP = (double *)malloc(sizeof(double) * (size_t)SS);
            double *vec = (double *)malloc(sizeof(double) * (size_t)(6 * dv));
            double *o = vec, *dov = vec + dv, *w = vec + 2 * dv, *u = vec + 3 * dv, *du = vec + 4 * dv,
                   *dw = vec + 5 * dv;
            double *ytmp = (double *)malloc(sizeof(double) * (size_t)dv);
            double *kTD = (double *)malloc(sizeof(double) * (size_t)dv);
            if (s0) memcpy(St, s0 + ((long)n * H + h) * SS, sizeof(double) * (size_t)SS);
            else memset(St, 0, sizeof(double) * (size_t)SS);
            for (long s = 0; s < L; ++s) {   /* forward, keeping every state */
                const long th = (cu[n] + s) * H + h;
                memcpy(St + (s + 1) * SS, St + s * SS, sizeof(double) * (size_t)SS);
                token_step(St + (s + 1) * SS, dk, dv, q + th * dk, k + th * dk, v + th * dv, la + th * dk,
                           beta[th], gate ? gate + th * dv : NULL, scale, kTD, ytmp);
            }
            if (ds_final) memcpy(dS, ds_final + ((long)n * H + h) * SS, sizeof(double) * (size_t)SS);
            else memset(dS, 0, sizeof(double) * (size_t)SS);
            for (long s = L - 1; s >= 0; --s) {
                const long th = (cu[n] + s) * H + h;
                const double *Sp = St + s * SS, *Sc = St + (s + 1) * SS;
                const double *qt = q + th * dk, *kt = k + th * dk, *vt = v + th * dv, *lat = la + th * dk;
                const double *gt = gate ? gate + th * dv : NULL, *dyt = dy + th * dv;
                const double bt = beta[th];
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < dk; ++i) acc += Sc[(long)i * dv + j] * qt[i];
                    o[j] = scale * acc;
                    dov[j] = dyt[j] * (gt ? gt[j] : 1.0);
                    if (gt) dgate[th * dv + j] = dyt[j] * o[j];
                }
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += Sc[(long)i * dv + j] * dov[j];
                    dq[th * dk + i] = scale * acc;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) dS[(long)i * dv + j] += scale * qt[i] * dov[j];
                for (int j = 0; j < dv; ++j) {
                    double aw = 0.0, ad = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        aw += exp(lat[i]) * Sp[(long)i * dv + j] * kt[i];
                        ad += dS[(long)i * dv + j] * kt[i];
                    }
                    w[j] = aw;
                    u[j] = bt * (vt[j] - aw);
                    du[j] = ad;
                }
                double db = 0.0;
                for (int j = 0; j < dv; ++j) {
                    db += du[j] * (vt[j] - w[j]);
                    dv_[th * dv + j] = bt * du[j];
                    dw[j] = -bt * du[j];
                }
                dbeta[th] = db;
                for (int i = 0; i < dk; ++i) {
                    const double a = exp(lat[i]);
                    double acc = 0.0, accd = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        const long e = (long)i * dv + j;
                        acc += dS[e] * u[j] + a * Sp[e] * dw[j];
                        dP[e] = dS[e] + kt[i] * dw[j];
                        accd += dP[e] * Sp[e];
                    }
                    dk_[th * dk + i] = acc;
                    dla[th * dk + i] = a * accd;
                    for (int j = 0; j < dv; ++j) dS[(long)i * dv + j] = a * dP[(long)i * dv + j];
                }
            }
            memcpy(ds0 + ((long)n * H + h) * SS, dS, sizeof(double) * (size_t)SS);
            free(kTD);
            free(ytmp);
            free(vec);
            free(dP);
            free(dS);
            free(St);
        }
    }
}

/* ---------------------------------------------------------------------------
 * The mixer's linear maps (k3 README, "Use this repository as a template":
 * the KDA module owns the projections and the output gating).
 * ------------------------------------------------------------------------- */

/* y[r][o] = sum_i x[r][i] w[o][i]: x [rows][in], w [out][in] (one row of
 * weights per output feature), y [rows][out]; a plain triple loop. */
void kda_oracle_linear(long rows, int in, int out, const double *x, const double *w, double *y) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r)
        for (int o = 0; o < out; ++o) {
            double acc = 0.0;
            for (int i = 0; i < in; ++i) acc += x[r * in + i] * w[(long)o * in + i];
            y[r * out + o] = acc;
        }
}

static double softplus(double x) { return x > 0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/* log alpha from its projection, per (row, head, channel):
 * la = -exp(a_log[h]) * softplus(z + bias[h * d + c]); a_log, bias may be
 * NULL (read as 0). z, la [rows][H][d]. */
void kda_oracle_log_decay(long rows, int H, int d, const double *z, const double *a_log, const double *bias,
                          double *la) {
    for (long r = 0; r < rows; ++r)
        for (int h = 0; h < H; ++h) {
            const double A = a_log ? exp(a_log[h]) : 1.0;
            for (int c = 0; c < d; ++c) {
                const long e = (r * H + h) * d + c;
                la[e] = -A * softplus(z[e] + (bias ? bias[h * d + c] : 0.0));
            }
        }
}

/* ---------------------------------------------------------------------------
 * The MLA decode token (kimi_k3 API docs, Functions: mla_decode_token, whose
 * steps are optional RoPE, K/V append, SDPA and an optional output gate, and
 * gated_mla_attend, the gated NoPE form that skips RoPE).  The projections
 * stay outside, in the MLA mixer, so the step sees each head's q and the new
 * token's per-head k and v.  Readings where the docs stop: the cache holds
 * one k (d_qk = nope + rope channels) and one v (d_v channels) per token and
 * kv head; the new token goes to position cache_len[b] and then attends to
 * positions 0 .. cache_len[b] inclusive; q head h reads kv head
 * h / (H / H_kv); the attention is softmax(scale q k^T) v; the gate is
 * sigmoid(gate_logit) per (head, value channel), multiplied into the output.
 * NoPE: no rotary step.  A sequence whose cache_len is outside
 * [0, max_len) is left alone: its caches are not written and its output is 0.
 * ------------------------------------------------------------------------- */

/* q [batch][H][d_qk], k_new [batch][H_kv][d_qk], v_new [batch][H_kv][d_v],
 * gate_logit [batch][H][d_v] or NULL, k_cache [batch][H_kv][max_len][d_qk],
 * v_cache [batch][H_kv][max_len][d_v] (both updated), out [batch][H][d_v]. */
void kda_oracle_mla_decode_step(int batch, int H, int H_kv, int d_qk, int d_v, int max_len, double scale,
                                const int32_t *cache_len, const double *q, const double *k_new,
                                const double *v_new, const double *gate_logit, double *k_cache,
                                double *v_cache, double *out) {
    const int G = H / H_kv;
    for (int b = 0; b < batch; ++b) {
        const int pos = cache_len[b];
        if (pos < 0 || pos >= max_len) {
            for (int i = 0; i < H * d_v; ++i) out[(long)b * H * d_v + i] = 0.0;
            continue;
        }
        /* append */
        for (int hk = 0; hk < H_kv; ++hk) {
            double *kc = k_cache + (((long)b * H_kv + hk) * max_len + pos) * d_qk;
            double *vc = v_cache + (((long)b * H_kv + hk) * max_len + pos) * d_v;
            for (int c = 0; c < d_qk; ++c) kc[c] = k_new[((long)b * H_kv + hk) * d_qk + c];
            for (int c = 0; c < d_v; ++c) vc[c] = v_new[((long)b * H_kv + hk) * d_v + c];
        }
        /* SDPA per q head over the pos + 1 cached tokens */
        double *s = malloc(sizeof(double) * (pos + 1));
        for (int h = 0; h < H; ++h) {
            const int hk = h / G;
            const double *qh = q + ((long)b * H + h) * d_qk;
            const double *K = k_cache + ((long)b * H_kv + hk) * max_len * d_qk;
            const double *V = v_cache + ((long)b * H_kv + hk) * max_len * d_v;
            double m = -INFINITY;
            for (int j = 0; j <= pos; ++j) {
                double dot = 0.0;
                for (int c = 0; c < d_qk; ++c) dot += qh[c] * K[(long)j * d_qk + c];
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
            }
            double den = 0.0;
            for (int j = 0; j <= pos; ++j) {
                s[j] = exp(s[j] - m);
                den += s[j];
            }
            double *o = out + ((long)b * H + h) * d_v;
            for (int c = 0; c < d_v; ++c) {
                double acc = 0.0;
                for (int j = 0; j <= pos; ++j) acc += s[j] * V[(long)j * d_v + c];
                o[c] = acc / den;
                if (gate_logit) o[c] *= sigmoid(gate_logit[((long)b * H + h) * d_v + c]);
            }
        }
        free(s);
    }
}
