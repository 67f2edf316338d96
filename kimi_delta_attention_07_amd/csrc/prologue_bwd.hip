// Backward of the KDA prologue for gfx950: carries the gradients that reach
// the prologue's outputs (q^, k^, v, beta, gate; from kda_chunk_backward)
// back through the L2 normalisation of q and k (kimi_k3 API docs, Constants:
// KDA_L2_EPS), the activation, the short causal depthwise conv on q, k, v
// (implementation list of the forum post "Experimental Native Vulkan Backend
// for Kimi K3") and the two sigmoids, to the raw projections, the conv taps
// and the incoming conv cache.  Everything is fp32.
//
// With pre_t[c] = sum_j w[c][j] x_{t-K+1+j}[c], x~ = act(pre), and for q, k
// n = sqrt(sum_c x~^2 + eps), x^ = x~ / n:
//   dx~  = dx^ / n - x~ (x~ . dx^) / n^3          (v: dx~ = dv)
//   dpre = dx~ act'(pre)                          (SiLU: s (1 + pre (1 - s)))
//   dx_tau[c] = sum_j w[c][j] dpre_{tau+K-1-j}[c]  over tokens of tau's sequence
//   dw[c][j]  = sum_t x_{t-K+1+j}[c] dpre_t[c]     (history from the cache)
//   dz = dy s (1 - s) for both sigmoids.
// The device copy of cu_seqlens is trusted to match the host copy the entry
// point validated, but every index derived from it is clamped, so a mismatch
// cannot reach outside the buffers.  Memory-bound stages:
//   pre     (token, head) rows: recomputes the conv and activation, writes
//           dpre of the three streams to the workspace, and the two sigmoid
//           gradients;
//   dx      gathers dx from the K taps' dpre rows of the same sequence;
//   dw      partial tap sums over blocks of 64 tokens;
// at head dim 128 one streaming kernel does all three per (64 tokens, head),
// dpre never leaving registers.  Then a small kernel forms the incoming
// cache's gradient from the first K-1 dpre rows of each sequence, and one
// fixed-order sum adds the tap partials (deterministic, no atomics).
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kBwdTokBlock = 64;    // tokens per partial sum of the tap gradient

__device__ __forceinline__ int seq_of(const int32_t *cu, int n_seqs, long t) {
    // largest n with cu[n] <= t (empty sequences share their start with the next)
    int lo = 0, hi = n_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid;
    }
    return lo;
}

// raw input of stream X at token tau of sequence n (tau may precede the
// sequence start: then the incoming cache row, or 0), channels c0, c0 + 1
template <int DT>
__device__ __forceinline__ float2 raw2(const PrologueBwdParams &p, int X, int n, long start, long tau, long ch) {
    if (tau >= start && tau >= 0) {
        const void *raw = X == 0 ? p.q_raw : (X == 1 ? p.k_raw : p.v_raw);
        return load2<DT>(raw, tau * (long)p.H * p.d + ch);
    }
    const int Km1 = p.K - 1;
    if (!p.cache_in || start - tau > Km1) return make_float2(0.f, 0.f);
    const float *cp = p.cache_in + (((long)n * 3 + X) * Km1 + (Km1 - (start - tau))) * (long)p.H * p.d + ch;
    return *reinterpret_cast<const float2 *>(cp);
}

// The K taps of channels ch and ch + 1 of stream X (w[c][j] at (X C + c) K +
// j): with K = 4 each channel's taps are one 16-byte load.
template <int K>
__device__ __forceinline__ void load_taps(const float *conv_w, long C, int X, long ch, float2 (&w)[K]) {
    const float *a = conv_w + ((long)X * C + ch) * K, *b = a + K;
    if constexpr (K == 4) {
        const float4 ta = *reinterpret_cast<const float4 *>(a), tb = *reinterpret_cast<const float4 *>(b);
        w[0] = make_float2(ta.x, tb.x);
        w[1] = make_float2(ta.y, tb.y);
        w[2] = make_float2(ta.z, tb.z);
        w[3] = make_float2(ta.w, tb.w);
    } else {
#pragma unroll
        for (int j = 0; j < K; ++j) w[j] = make_float2(a[j], b[j]);
    }
}

__device__ __forceinline__ float act_grad(int act, float pre) {
    if (act != 1) return 1.0f;
    const float s = sigmoidf(pre);
    return s * (1.0f + pre * (1.0f - s));
}

// ---- stage 1: dpre of q, k, v; sigmoid gradients ------------------------------
// Lanes hold channel pairs of one token row (LPT = D / 2 lanes per token), as
// in the forward prologue; the two L2 sums are lane-group reductions.  Every
// load of the row (the K-row conv window, the taps, the upstream gradients,
// the logits) is issued before any of them is used.
template <int D, int DT, int K>
__global__ __launch_bounds__(256) void prologue_bwd_pre_kernel(PrologueBwdParams p) {
    constexpr int LPT = D / 2, TPB = 256 / LPT;   // lanes per token, tokens per block
    const int h = blockIdx.y;
    const int sub = threadIdx.x / LPT, c0 = 2 * (threadIdx.x % LPT);
    const long t = (long)blockIdx.x * TPB + sub;
    const bool valid = t < p.T;
    const long tc = valid ? t : p.T - 1;       // rows past the end redo the last row, unstored
    const long C = (long)p.H * D, ch = (long)h * D + c0;
    const long o = (tc * p.H + h) * D + c0;    // row-major [T][H][D] index
    const int n = seq_of(p.cu, p.n_seqs, tc);
    const long start = p.cu[n];
    float2 x[3][K], w[3][K];
    // rows whose conv window lies inside the sequence (all but its first K-1)
    // load without a branch per tap
    if (tc - (K - 1) >= start) {
#pragma unroll
        for (int X = 0; X < 3; ++X) {
            const void *raw = X == 0 ? p.q_raw : (X == 1 ? p.k_raw : p.v_raw);
#pragma unroll
            for (int j = 0; j < K; ++j) x[X][j] = load2<DT>(raw, (tc - (K - 1) + j) * C + ch);
        }
    } else {
#pragma unroll
        for (int X = 0; X < 3; ++X)
#pragma unroll
            for (int j = 0; j < K; ++j) x[X][j] = raw2<DT>(p, X, n, start, tc - (K - 1) + j, ch);
    }
#pragma unroll
    for (int X = 0; X < 3; ++X) load_taps<K>(p.conv_w, C, X, ch, w[X]);
    float2 dy[3];
    dy[0] = *reinterpret_cast<const float2 *>(p.dq + o);
    dy[1] = *reinterpret_cast<const float2 *>(p.dk + o);
    dy[2] = *reinterpret_cast<const float2 *>(p.dv + o);
    float2 zg = make_float2(0.f, 0.f), dg = zg;
    if (p.gate_logit) {
        zg = load2<DT>(p.gate_logit, o);
        dg = *reinterpret_cast<const float2 *>(p.dgate + o);
    }
    const long ob = tc * p.H + h;
    const float zb = load1<DT>(p.beta_logit, ob), db = p.dbeta[ob];
    float pre[3][2], xa[3][2];
#pragma unroll
    for (int X = 0; X < 3; ++X) {
        pre[X][0] = pre[X][1] = 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            pre[X][0] += w[X][j].x * x[X][j].x;
            pre[X][1] += w[X][j].y * x[X][j].y;
        }
        xa[X][0] = activate(p.act, pre[X][0]);
        xa[X][1] = activate(p.act, pre[X][1]);
    }
    // L2 backward of q and k: every lane takes part in the group sums
    float sums[2][2];   // [q, k][sum x~^2, sum x~ dx^]
#pragma unroll
    for (int X = 0; X < 2; ++X) {
        sums[X][0] = group_sum(xa[X][0] * xa[X][0] + xa[X][1] * xa[X][1], LPT);
        sums[X][1] = group_sum(xa[X][0] * dy[X].x + xa[X][1] * dy[X].y, LPT);
    }
    float dxt[3][2];
#pragma unroll
    for (int X = 0; X < 2; ++X) {
        const float ss = sums[X][0], xd = sums[X][1];
        const float inv = 1.0f / sqrtf(ss + p.eps);
        const float k3 = xd * inv * inv * inv;
        dxt[X][0] = dy[X].x * inv - xa[X][0] * k3;
        dxt[X][1] = dy[X].y * inv - xa[X][1] * k3;
    }
    dxt[2][0] = dy[2].x;
    dxt[2][1] = dy[2].y;
    if (!valid) return;
#pragma unroll
    for (int X = 0; X < 3; ++X) {
        const float2 g = make_float2(dxt[X][0] * act_grad(p.act, pre[X][0]), dxt[X][1] * act_grad(p.act, pre[X][1]));
        *reinterpret_cast<float2 *>(p.dpre + ((long)X * p.T + t) * C + ch) = g;
    }
    if (p.gate_logit) {
        const float s0 = sigmoidf(zg.x), s1 = sigmoidf(zg.y);
        *reinterpret_cast<float2 *>(p.dgate_logit + o) = make_float2(dg.x * s0 * (1.f - s0), dg.y * s1 * (1.f - s1));
    }
    if (c0 == 0) {
        const float sb = sigmoidf(zb);
        p.dbeta_logit[ob] = db * sb * (1.f - sb);
    }
}

// ---- stage 2: dx (raw inputs) and the incoming cache's gradient ----------------
// thread: a channel pair of one token row of one head, all three streams;
// taps of tokens past the sequence's end (or the batch's) read a clamped row
// and count as zero
template <int D, int K>
__global__ __launch_bounds__(256) void prologue_bwd_dx_kernel(PrologueBwdParams p) {
    constexpr int LPT = D / 2, TPB = 256 / LPT;
    const int h = blockIdx.y;
    const int sub = threadIdx.x / LPT, c0 = 2 * (threadIdx.x % LPT);
    const long tau = (long)blockIdx.x * TPB + sub;
    if (tau >= p.T) return;
    const long C = (long)p.H * D, ch = (long)h * D + c0;
    const int n = seq_of(p.cu, p.n_seqs, tau);
    const long end = min((long)p.cu[n + 1], (long)p.T);
    float2 g[3][K], w[3][K];
#pragma unroll
    for (int X = 0; X < 3; ++X)
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const long t = min(tau + (K - 1) - j, (long)p.T - 1);   // the token whose tap j reads tau
            g[X][j] = *reinterpret_cast<const float2 *>(p.dpre + ((long)X * p.T + t) * C + ch);
        }
#pragma unroll
    for (int X = 0; X < 3; ++X) load_taps<K>(p.conv_w, C, X, ch, w[X]);
    float *outs[3] = {p.dq_raw, p.dk_raw, p.dv_raw};
#pragma unroll
    for (int X = 0; X < 3; ++X) {
        float2 acc = make_float2(0.f, 0.f);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (tau + (K - 1) - j < end) {
                acc.x += w[X][j].x * g[X][j].x;
                acc.y += w[X][j].y * g[X][j].y;
            }
        }
        *reinterpret_cast<float2 *>(outs[X] + tau * C + ch) = acc;
    }
}

// ---- head dim 128: the three stages in one pass ---------------------------
// A wave streams the 64 token rows of one block for one head (lane l:
// channels 2l, 2l + 1), plus the K - 1 rows after them.  Each row's dpre (the
// pre stage's arithmetic) goes into a ring of the last K rows: the row K - 1
// earlier then has every dpre row its dx reads, and the row's own conv window
// gives its tap-gradient terms.  dpre reaches HBM only for the first K - 1
// rows of each sequence, which the incoming cache's gradient reads.  Each
// row's loads are issued a row ahead.
// One token row's inputs as loaded (bf16 pairs stay packed until used: a
// conversion right after the load would make the wave wait for it there).
template <int DT>
struct RowIn128 {
    using Pair = typename std::conditional<DT == 1, uint32_t, float2>::type;
    float2 dy[3], dg;   // dq, dk, dv reaching the outputs; dgate
    Pair zg, xr[3];     // gate logit; raw q, k, v
};
__device__ __forceinline__ float2 pair_f2(uint32_t u) { return make_float2(lo_bf(u), hi_bf(u)); }
__device__ __forceinline__ float2 pair_f2(float2 v) { return v; }
// The streaming kernel reads every row once: its loads carry the
// non-temporal bit.
typedef float ntf2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 nt2(const float *q) {
    const ntf2 v = __builtin_nontemporal_load(reinterpret_cast<const ntf2 *>(q));
    return make_float2(v[0], v[1]);
}
template <int DT>
__device__ __forceinline__ typename RowIn128<DT>::Pair load_pair(const void *base, long idx) {
    if constexpr (DT == 1) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(base) + idx));
    else return nt2(static_cast<const float *>(base) + idx);
}
// Rows past the end load the last row (unused).  Without a gate, the gate
// loads read dq instead (in bounds, unused), so no branch splits the loads.
template <int DT>
__device__ __forceinline__ void load_row128(const PrologueBwdParams &p, long t, long C, long ch, RowIn128<DT> &r) {
    t = min(t, (long)p.T - 1);
    const long o = t * C + ch;
    r.dy[0] = nt2(p.dq + o);
    r.dy[1] = nt2(p.dk + o);
    r.dy[2] = nt2(p.dv + o);
    r.zg = load_pair<DT>(p.gate_logit ? p.gate_logit : static_cast<const void *>(p.dq), o);
    r.dg = nt2((p.gate_logit ? p.dgate : p.dq) + o);
    r.xr[0] = load_pair<DT>(p.q_raw, o);
    r.xr[1] = load_pair<DT>(p.k_raw, o);
    r.xr[2] = load_pair<DT>(p.v_raw, o);
}

template <int DT, int K>
__global__ __launch_bounds__(256) void prologue_bwd_fused128_kernel(PrologueBwdParams p) {
    constexpr int D = 128, Km1 = K - 1;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int h = 4 * blockIdx.y + w;
    if (h >= p.H) return;   // wave-uniform; the kernel has no barrier
    const long C = (long)p.H * D, ch = (long)h * D + 2 * l;
    const long t0 = (long)blockIdx.x * kBwdTokBlock, t1 = min((long)p.T, t0 + kBwdTokBlock);
    const float2 z2 = make_float2(0.f, 0.f);
    float2 wt[3][K], acc[3][K], ring[3][K], xw[3][K];
#pragma unroll
    for (int X = 0; X < 3; ++X) {
        load_taps<K>(p.conv_w, C, X, ch, wt[X]);
#pragma unroll
        for (int j = 0; j < K; ++j) acc[X][j] = ring[X][j] = xw[X][j] = z2;
    }
    // sequence of row t (n, its start and end) and of row tau = t - (K - 1)
    // (nt, its end); the bounds are reloaded only when a sequence ends, since
    // any load waited for in the loop would also wait for the prefetched row
    int n = seq_of(p.cu, p.n_seqs, t0);
    int nt = n;
    long start = p.cu[n], end_n = p.cu[n + 1], end_nt = end_n;
    float *outs[3] = {p.dq_raw, p.dk_raw, p.dv_raw};
    // beta logit and dbeta of own row t0 + i in lane i: a per-row load of
    // them would be a scalar load, and waiting for it waits for every scalar
    // load issued, the prefetched rows' included
    static_assert(kBwdTokBlock == 64, "one lane per own row");
    const long tb = min(t0 + l, (long)p.T - 1);
    const float bz = load1<DT>(p.beta_logit, tb * p.H + h), bd = p.dbeta[tb * p.H + h];
    auto row = [&](long t, const RowIn128<DT> &cur) {
        float2 g[3] = {z2, z2, z2};
        if (t < p.T) {   // uniform
            while (t >= end_n && n + 1 < p.n_seqs) {
                ++n;
                start = end_n;
                end_n = p.cu[n + 1];
            }
            if (t == t0 || t - Km1 < start) {   // window rebuilt: block start, or history before the sequence
#pragma unroll
                for (int X = 0; X < 3; ++X)
#pragma unroll
                    for (int j = 0; j < K; ++j) xw[X][j] = raw2<DT>(p, X, n, start, t - Km1 + j, ch);
            } else {   // rows t - K + 1 .. t - 1 are the previous row's window
#pragma unroll
                for (int X = 0; X < 3; ++X) {
#pragma unroll
                    for (int j = 0; j < Km1; ++j) xw[X][j] = xw[X][j + 1];
                    xw[X][Km1] = pair_f2(cur.xr[X]);
                }
            }
            float pre[3][2], xa[3][2];
#pragma unroll
            for (int X = 0; X < 3; ++X) {
                pre[X][0] = pre[X][1] = 0.f;
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    pre[X][0] += wt[X][j].x * xw[X][j].x;
                    pre[X][1] += wt[X][j].y * xw[X][j].y;
                }
                xa[X][0] = activate(p.act, pre[X][0]);
                xa[X][1] = activate(p.act, pre[X][1]);
            }
            float dxt[3][2];
#pragma unroll
            for (int X = 0; X < 2; ++X) {
                const float v = wave_sum_pair(xa[X][0] * xa[X][0] + xa[X][1] * xa[X][1],
                                              xa[X][0] * cur.dy[X].x + xa[X][1] * cur.dy[X].y);
                const float inv = 1.0f / sqrtf(lane_value(v, 0) + p.eps);
                const float k3 = lane_value(v, 16) * inv * inv * inv;
                dxt[X][0] = cur.dy[X].x * inv - xa[X][0] * k3;
                dxt[X][1] = cur.dy[X].y * inv - xa[X][1] * k3;
            }
            dxt[2][0] = cur.dy[2].x;
            dxt[2][1] = cur.dy[2].y;
#pragma unroll
            for (int X = 0; X < 3; ++X)
                g[X] = make_float2(dxt[X][0] * act_grad(p.act, pre[X][0]), dxt[X][1] * act_grad(p.act, pre[X][1]));
            if (t < t1) {   // this block's own row
                const long o = t * C + ch;
                if (p.gate_logit) {
                    const float2 zg = pair_f2(cur.zg);
                    const float s0 = sigmoidf(zg.x), s1 = sigmoidf(zg.y);
                    *reinterpret_cast<float2 *>(p.dgate_logit + o) =
                        make_float2(cur.dg.x * s0 * (1.f - s0), cur.dg.y * s1 * (1.f - s1));
                }
                {
                    const int r = (int)(t - t0);   // < 64
                    const float zb = lane_value(bz, r), db = lane_value(bd, r);
                    const float sb = sigmoidf(zb);
                    if (l == 0) p.dbeta_logit[t * p.H + h] = db * sb * (1.f - sb);
                }
#pragma unroll
                for (int X = 0; X < 3; ++X)
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        acc[X][j].x += xw[X][j].x * g[X].x;
                        acc[X][j].y += xw[X][j].y * g[X].y;
                    }
                if (t - start < Km1)   // the incoming cache's gradient reads these rows
#pragma unroll
                    for (int X = 0; X < 3; ++X)
                        *reinterpret_cast<float2 *>(p.dpre + ((long)X * p.T + t) * C + ch) = g[X];
            }
        }
        // ring: dpre of rows t - K + 1 .. t (rows past the end are 0)
#pragma unroll
        for (int X = 0; X < 3; ++X) {
#pragma unroll
            for (int j = 0; j < Km1; ++j) ring[X][j] = ring[X][j + 1];
            ring[X][Km1] = g[X];
        }
        const long tau = t - Km1;   // every dpre row its dx reads is in the ring
        if (tau >= t0) {
            while (tau >= end_nt && nt + 1 < p.n_seqs) end_nt = p.cu[++nt + 1];
            const long end = min(end_nt, (long)p.T);
#pragma unroll
            for (int X = 0; X < 3; ++X) {
                float2 d = z2;
#pragma unroll
                for (int j = 0; j < K; ++j)
                    if (t - j < end) {   // tap j of token t - j reads tau
                        d.x += wt[X][j].x * ring[X][Km1 - j].x;
                        d.y += wt[X][j].y * ring[X][Km1 - j].y;
                    }
                *reinterpret_cast<float2 *>(outs[X] + tau * C + ch) = d;
            }
        }
    };
    // rows in pairs through two buffers, each refilled right after its row
    // (no copy of a buffer in flight)
    RowIn128<DT> A, B;
    const long tE = t1 + Km1;
    load_row128<DT>(p, t0, C, ch, A);
    long t = t0;
    for (; t + 1 < tE; t += 2) {
        load_row128<DT>(p, t + 1, C, ch, B);
        row(t, A);
        load_row128<DT>(p, t + 2, C, ch, A);
        row(t + 1, B);
    }
    if (t < tE) row(t, A);
    // tap partials of this block, [block][X][c][4 taps]
#pragma unroll
    for (int X = 0; X < 3; ++X) {
        float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < K; ++j) {
            a[j] = acc[X][j].x;
            b[j] = acc[X][j].y;
        }
        float *part = p.dw_part + (((long)blockIdx.x * 3 + X) * C + ch) * 4;
        *reinterpret_cast<float4 *>(part) = make_float4(a[0], a[1], a[2], a[3]);
        *reinterpret_cast<float4 *>(part + 4) = make_float4(b[0], b[1], b[2], b[3]);
    }
}

// grid (sequences, 3 streams x (K-1) history slots, channel blocks of 512),
// thread: one channel pair
__global__ __launch_bounds__(256) void prologue_bwd_dcache_kernel(PrologueBwdParams p) {
    const int n = blockIdx.x, Km1 = p.K - 1;
    const int X = blockIdx.y / Km1, s = blockIdx.y % Km1;
    const long C = (long)p.H * p.d;
    const long start = max(0L, (long)p.cu[n]), end = min((long)p.cu[n + 1], (long)p.T);
    const long tau = start - Km1 + s;   // the absolute position this slot stands for
    const long ch = ((long)blockIdx.z * 256 + threadIdx.x) * 2;
    if (ch < C) {
        float2 acc = make_float2(0.f, 0.f);
        for (int j = 0; j < p.K; ++j) {
            const long t = tau + Km1 - j;
            if (t >= start && t < end) {
                const float2 g = *reinterpret_cast<const float2 *>(p.dpre + ((long)X * p.T + t) * C + ch);
                acc.x += p.conv_w[((long)X * C + ch) * p.K + j] * g.x;
                acc.y += p.conv_w[((long)X * C + ch + 1) * p.K + j] * g.y;
            }
        }
        *reinterpret_cast<float2 *>(p.dcache_in + (((long)n * 3 + X) * Km1 + s) * C + ch) = acc;
    }
}

// ---- stage 3: tap gradient, partial sums over token blocks, then their sum ---
// grid (token blocks, channel blocks of 256, 3 streams); thread: one channel.
// Tokens go in batches of 8 whose loads are all issued first.
template <int DT, int K>
__global__ __launch_bounds__(256) void prologue_bwd_dw_partial_kernel(PrologueBwdParams p) {
    constexpr int B8 = 8;
    const long C = (long)p.H * p.d;
    const long c = (long)blockIdx.y * 256 + threadIdx.x;
    const int X = blockIdx.z;
    const long t0 = (long)blockIdx.x * kBwdTokBlock, t1 = min((long)p.T, t0 + kBwdTokBlock);
    if (c >= C) return;
    const void *raw = X == 0 ? p.q_raw : (X == 1 ? p.k_raw : p.v_raw);
    constexpr int Km1 = K - 1;
    float acc[K];
#pragma unroll
    for (int j = 0; j < K; ++j) acc[j] = 0.f;
    int n = seq_of(p.cu, p.n_seqs, t0);
    for (long tb = t0; tb < t1; tb += B8) {
        float gv[B8], xv[B8][K];
        while (tb >= p.cu[n + 1] && n + 1 < p.n_seqs) ++n;   // the batch's first token's sequence (uniform)
        if (tb - Km1 >= p.cu[n] && tb + B8 <= min(t1, (long)p.cu[n + 1])) {
            // the whole batch and its conv windows inside one sequence: no branch per tap
#pragma unroll
            for (int u = 0; u < B8; ++u) {
                gv[u] = p.dpre[((long)X * p.T + tb + u) * C + c];
#pragma unroll
                for (int j = 0; j < K; ++j) xv[u][j] = load1<DT>(raw, (tb + u - Km1 + j) * C + c);
            }
        } else {
#pragma unroll
            for (int u = 0; u < B8; ++u) {
                const long t = min(tb + u, t1 - 1);   // past t1: a repeated row, weighted 0 below
                while (t >= p.cu[n + 1] && n + 1 < p.n_seqs) ++n;   // the token's sequence (uniform)
                const long start = p.cu[n];
                gv[u] = tb + u < t1 ? p.dpre[((long)X * p.T + t) * C + c] : 0.f;
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const long tau = t - Km1 + j;
                    if (tau >= start && tau >= 0) xv[u][j] = load1<DT>(raw, tau * C + c);
                    else if (p.cache_in && start - tau <= Km1)
                        xv[u][j] = p.cache_in[(((long)n * 3 + X) * Km1 + (Km1 - (start - tau))) * C + c];
                    else xv[u][j] = 0.f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < B8; ++u)
#pragma unroll
            for (int j = 0; j < K; ++j) acc[j] += xv[u][j] * gv[u];
    }
    float out[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) out[j] = acc[j];
    float *part = p.dw_part + (((long)blockIdx.x * 3 + X) * C + c) * 4;
    *reinterpret_cast<float4 *>(part) = make_float4(out[0], out[1], out[2], out[3]);
}

// One fixed-order sum over the blocks per (stream, channel): 64-thread blocks
// spread it over the CUs, and the block loop is unrolled so its loads are in
// flight together.
__global__ __launch_bounds__(64) void prologue_bwd_dw_sum_kernel(PrologueBwdParams p, int n_blocks) {
    const long C = (long)p.H * p.d;
    const long e = (long)blockIdx.x * 64 + threadIdx.x;   // (X, c)
    if (e >= 3 * C) return;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int b = 0; b < n_blocks; ++b) {
        const float4 v = *reinterpret_cast<const float4 *>(p.dw_part + ((long)b * 3 * C + e) * 4);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    const float sv[4] = {s.x, s.y, s.z, s.w};
    for (int j = 0; j < p.K; ++j) p.dconv_w[e * p.K + j] = sv[j];
}

template <int D, int K>
void launch_stages(const PrologueBwdParams &p, int dtype, int nb, hipStream_t s) {
    if constexpr (D == 128) {
        const dim3 g((unsigned)nb, (unsigned)((p.H + 3) / 4));
        if (dtype == 1) hipLaunchKernelGGL((prologue_bwd_fused128_kernel<1, K>), g, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((prologue_bwd_fused128_kernel<0, K>), g, dim3(256), 0, s, p);
        return;
    }
    constexpr int TPB = 256 / (D / 2);
    const dim3 grid((unsigned)((p.T + TPB - 1) / TPB), (unsigned)p.H);
    if (dtype == 1) hipLaunchKernelGGL((prologue_bwd_pre_kernel<D, 1, K>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prologue_bwd_pre_kernel<D, 0, K>), grid, dim3(256), 0, s, p);
    hipLaunchKernelGGL((prologue_bwd_dx_kernel<D, K>), grid, dim3(256), 0, s, p);
    const long C = (long)p.H * D;
    const dim3 g3((unsigned)nb, (unsigned)((C + 255) / 256), 3);
    if (dtype == 1) hipLaunchKernelGGL((prologue_bwd_dw_partial_kernel<1, K>), g3, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prologue_bwd_dw_partial_kernel<0, K>), g3, dim3(256), 0, s, p);
}

template <int D>
void launch_d(const PrologueBwdParams &p, int dtype, int nb, hipStream_t s) {
    switch (p.K) {
        case 1: launch_stages<D, 1>(p, dtype, nb, s); break;
        case 2: launch_stages<D, 2>(p, dtype, nb, s); break;
        case 3: launch_stages<D, 3>(p, dtype, nb, s); break;
        default: launch_stages<D, 4>(p, dtype, nb, s); break;
    }
}

}  // namespace

size_t prologue_bwd_workspace_bytes(int H, int d, long T) {
    const long C = (long)H * d, nb = (T + kBwdTokBlock - 1) / kBwdTokBlock;
    return (size_t)(3 * T * C) * 4 + (size_t)(nb * 3 * C * 4) * 4;
}

hipError_t launch_prologue_backward(PrologueBwdParams p, int dtype, hipStream_t s) {
    const long C = (long)p.H * p.d;
    p.dpre = static_cast<float *>(p.workspace);
    p.dw_part = p.dpre + 3 * (long)p.T * C;
    const int nb = (int)((p.T + kBwdTokBlock - 1) / kBwdTokBlock);
    if (p.T > 0) {
        switch (p.d) {
            case 4: launch_d<4>(p, dtype, nb, s); break;
            case 8: launch_d<8>(p, dtype, nb, s); break;
            case 16: launch_d<16>(p, dtype, nb, s); break;
            case 32: launch_d<32>(p, dtype, nb, s); break;
            case 64: launch_d<64>(p, dtype, nb, s); break;
            default: launch_d<128>(p, dtype, nb, s); break;
        }
    }
    if (p.dcache_in && p.K > 1)
        hipLaunchKernelGGL(prologue_bwd_dcache_kernel,
                           dim3((unsigned)p.n_seqs, (unsigned)(3 * (p.K - 1)), (unsigned)((C + 511) / 512)), dim3(256),
                           0, s, p);
    hipLaunchKernelGGL(prologue_bwd_dw_sum_kernel, dim3((unsigned)((3 * C + 63) / 64)), dim3(64), 0, s, p, p.T > 0 ? nb : 0);
    return hipGetLastError();
}

}  // namespace kda
