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
// cannot reach outside the buffers.  Three memory-bound stages:
//   pre     (token, head) rows: recomputes the conv and activation, writes
//           dpre of the three streams to the workspace, and the two sigmoid
//           gradients;
//   dx      (token, head) rows: gathers dx from the K taps' dpre rows of the
//           same sequence; a small kernel does the same for the incoming
//           cache's K-1 history rows of each sequence;
//   dw      partial tap sums over blocks of 256 tokens, then one fixed-order
//           sum over the blocks (deterministic, no atomics).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kBwdTokBlock = 256;   // tokens per partial sum of the tap gradient

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

__device__ __forceinline__ float act_grad(int act, float pre) {
    if (act != 1) return 1.0f;
    const float s = sigmoidf(pre);
    return s * (1.0f + pre * (1.0f - s));
}

// ---- stage 1: dpre of q, k, v; sigmoid gradients ------------------------------
// Lanes hold channel pairs of one token row (LPT = D / 2 lanes per token), as
// in the forward prologue; the two L2 sums are lane-group reductions.
template <int D, int DT>
__global__ __launch_bounds__(256) void prologue_bwd_pre_kernel(PrologueBwdParams p) {
    constexpr int LPT = D / 2, TPB = 256 / LPT;   // lanes per token, tokens per block
    const int h = blockIdx.y;
    const int sub = threadIdx.x / LPT, c0 = 2 * (threadIdx.x % LPT);
    const long t = (long)blockIdx.x * TPB + sub;
    const bool valid = t < p.T;
    const long C = (long)p.H * D, ch = (long)h * D + c0;
    float pre[3][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
    if (valid) {
        const int n = seq_of(p.cu, p.n_seqs, t);
        const long start = p.cu[n];
        for (int j = 0; j < p.K; ++j) {
            const long tau = t - (p.K - 1) + j;
#pragma unroll
            for (int X = 0; X < 3; ++X) {
                const float2 x = raw2<DT>(p, X, n, start, tau, ch);
                const float2 w = make_float2(p.conv_w[((long)X * C + ch) * p.K + j],
                                             p.conv_w[((long)X * C + ch + 1) * p.K + j]);
                pre[X][0] += w.x * x.x;
                pre[X][1] += w.y * x.y;
            }
        }
    }
    const long o = (t * p.H + h) * D + c0;   // row-major [T][H][D] index
    float2 dy[3] = {make_float2(0.f, 0.f), make_float2(0.f, 0.f), make_float2(0.f, 0.f)};
    if (valid) {
        dy[0] = *reinterpret_cast<const float2 *>(p.dq + o);
        dy[1] = *reinterpret_cast<const float2 *>(p.dk + o);
        dy[2] = *reinterpret_cast<const float2 *>(p.dv + o);
    }
    float xa[3][2];
#pragma unroll
    for (int X = 0; X < 3; ++X) {
        xa[X][0] = activate(p.act, pre[X][0]);
        xa[X][1] = activate(p.act, pre[X][1]);
    }
    // L2 backward of q and k: every lane takes part in the group sums
    float dxt[3][2];
#pragma unroll
    for (int X = 0; X < 2; ++X) {
        const float ss = group_sum(xa[X][0] * xa[X][0] + xa[X][1] * xa[X][1], LPT);
        const float xd = group_sum(xa[X][0] * dy[X].x + xa[X][1] * dy[X].y, LPT);
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
        const float2 z = load2<DT>(p.gate_logit, o);
        const float2 d = *reinterpret_cast<const float2 *>(p.dgate + o);
        const float s0 = sigmoidf(z.x), s1 = sigmoidf(z.y);
        *reinterpret_cast<float2 *>(p.dgate_logit + o) = make_float2(d.x * s0 * (1.f - s0), d.y * s1 * (1.f - s1));
    }
    if (c0 == 0) {
        const long ob = t * p.H + h;
        const float s = sigmoidf(load1<DT>(p.beta_logit, ob));
        p.dbeta_logit[ob] = p.dbeta[ob] * s * (1.f - s);
    }
}

// ---- stage 2: dx (raw inputs) and the incoming cache's gradient ----------------
// thread: a channel pair of one token row of one head, all three streams
template <int D>
__global__ __launch_bounds__(256) void prologue_bwd_dx_kernel(PrologueBwdParams p) {
    constexpr int LPT = D / 2, TPB = 256 / LPT;
    const int h = blockIdx.y;
    const int sub = threadIdx.x / LPT, c0 = 2 * (threadIdx.x % LPT);
    const long tau = (long)blockIdx.x * TPB + sub;
    if (tau >= p.T) return;
    const long C = (long)p.H * D, ch = (long)h * D + c0;
    const int n = seq_of(p.cu, p.n_seqs, tau);
    const long end = min((long)p.cu[n + 1], (long)p.T);
    float *outs[3] = {p.dq_raw, p.dk_raw, p.dv_raw};
#pragma unroll
    for (int X = 0; X < 3; ++X) {
        float2 acc = make_float2(0.f, 0.f);
        for (int j = 0; j < p.K; ++j) {
            const long t = tau + (p.K - 1) - j;   // the token whose tap j reads tau
            if (t < end) {
                const float2 g = *reinterpret_cast<const float2 *>(p.dpre + ((long)X * p.T + t) * C + ch);
                acc.x += p.conv_w[((long)X * C + ch) * p.K + j] * g.x;
                acc.y += p.conv_w[((long)X * C + ch + 1) * p.K + j] * g.y;
            }
        }
        *reinterpret_cast<float2 *>(outs[X] + tau * C + ch) = acc;
    }
}

// grid (sequences, 3 streams x (K-1) history slots), threads over channel pairs
__global__ __launch_bounds__(256) void prologue_bwd_dcache_kernel(PrologueBwdParams p) {
    const int n = blockIdx.x, Km1 = p.K - 1;
    const int X = blockIdx.y / Km1, s = blockIdx.y % Km1;
    const long C = (long)p.H * p.d;
    const long start = max(0L, (long)p.cu[n]), end = min((long)p.cu[n + 1], (long)p.T);
    const long tau = start - Km1 + s;   // the absolute position this slot stands for
    for (long ch = 2 * (long)threadIdx.x; ch < C; ch += 2 * 256) {
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
// grid (token blocks, channel blocks of 256, 3 streams); thread: one channel
template <int DT>
__global__ __launch_bounds__(256) void prologue_bwd_dw_partial_kernel(PrologueBwdParams p) {
    const long C = (long)p.H * p.d;
    const long c = (long)blockIdx.y * 256 + threadIdx.x;
    const int X = blockIdx.z;
    const long t0 = (long)blockIdx.x * kBwdTokBlock, t1 = min((long)p.T, t0 + kBwdTokBlock);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (c < C) {
        const void *raw = X == 0 ? p.q_raw : (X == 1 ? p.k_raw : p.v_raw);
        const int Km1 = p.K - 1;
        int n = seq_of(p.cu, p.n_seqs, t0);
        long start = p.cu[n], end = p.cu[n + 1];
        for (long t = t0; t < t1; ++t) {
            while (t >= end && n + 1 < p.n_seqs) {   // next non-empty sequence (uniform across the block)
                ++n;
                start = p.cu[n];
                end = p.cu[n + 1];
            }
            const float g = p.dpre[((long)X * p.T + t) * C + c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < p.K) {
                    const long tau = t - Km1 + j;
                    float x = 0.f;
                    if (tau >= start && tau >= 0) x = load1<DT>(raw, tau * C + c);
                    else if (p.cache_in && start - tau <= Km1)
                        x = p.cache_in[(((long)n * 3 + X) * Km1 + (Km1 - (start - tau))) * C + c];
                    acc[j] += x * g;
                }
            }
        }
        float *part = p.dw_part + (((long)blockIdx.x * 3 + X) * C + c) * 4;
        *reinterpret_cast<float4 *>(part) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
}

__global__ __launch_bounds__(256) void prologue_bwd_dw_sum_kernel(PrologueBwdParams p, int n_blocks) {
    const long C = (long)p.H * p.d;
    const long e = (long)blockIdx.x * 256 + threadIdx.x;   // (X, c)
    if (e >= 3 * C) return;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
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

template <int D>
void launch_pre_dx(const PrologueBwdParams &p, int dtype, hipStream_t s) {
    constexpr int TPB = 256 / (D / 2);
    const dim3 grid((unsigned)((p.T + TPB - 1) / TPB), (unsigned)p.H);
    if (dtype == 1) hipLaunchKernelGGL((prologue_bwd_pre_kernel<D, 1>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prologue_bwd_pre_kernel<D, 0>), grid, dim3(256), 0, s, p);
    hipLaunchKernelGGL(prologue_bwd_dx_kernel<D>, grid, dim3(256), 0, s, p);
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
            case 4: launch_pre_dx<4>(p, dtype, s); break;
            case 8: launch_pre_dx<8>(p, dtype, s); break;
            case 16: launch_pre_dx<16>(p, dtype, s); break;
            case 32: launch_pre_dx<32>(p, dtype, s); break;
            case 64: launch_pre_dx<64>(p, dtype, s); break;
            default: launch_pre_dx<128>(p, dtype, s); break;
        }
        const dim3 g3((unsigned)nb, (unsigned)((C + 255) / 256), 3);
        if (dtype == 1) hipLaunchKernelGGL(prologue_bwd_dw_partial_kernel<1>, g3, dim3(256), 0, s, p);
        else hipLaunchKernelGGL(prologue_bwd_dw_partial_kernel<0>, g3, dim3(256), 0, s, p);
    }
    if (p.dcache_in && p.K > 1)
        hipLaunchKernelGGL(prologue_bwd_dcache_kernel, dim3((unsigned)p.n_seqs, (unsigned)(3 * (p.K - 1))), dim3(256), 0,
                           s, p);
    hipLaunchKernelGGL(prologue_bwd_dw_sum_kernel, dim3((unsigned)((3 * C + 255) / 256)), dim3(256), 0, s, p, p.T > 0 ? nb : 0);
    return hipGetLastError();
}

}  // namespace kda
