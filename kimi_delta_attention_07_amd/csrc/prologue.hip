// KDA prologue for gfx950: short causal depthwise conv + activation on q, k,
// v (independently, as the implementation list of the forum post
// "Experimental Native Vulkan Backend for Kimi K3" has it), L2 normalisation
// of q and k with KDA_L2_EPS (kimi_k3 API docs, Constants), beta =
// sigmoid(beta_logit) and gate = sigmoid(gate_logit).
//
// Memory-bound.  Lanes hold channel pairs of one token row (256 contiguous
// bytes per bf16 row of head dim 128), so every load and store of a wave is
// one coalesced row; the L2 norm is a lane-group reduction with no barrier.
// Head dim 128 (the production shape) has its own kernel that streams a
// register window of rows; smaller head dims use a simple kernel where a wave
// step covers 128/d tokens and the K-1 history rows are re-read (L1/L2 hits).
// Before a sequence start the conv reads the incoming conv cache; a second
// small kernel writes each sequence's outgoing conv cache after the main
// kernel has read the incoming one, so the two may alias.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kSteps = 16;  // wave steps per workgroup

__device__ __forceinline__ int find_seq(const int32_t *cu, int n_seqs, long t) {
    // largest n with cu[n] <= t  (then cu[n+1] > t; empty sequences skipped)
    int lo = 0, hi = n_seqs;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid;
    }
    return lo;
}

template <int D, int DT>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueParams p) {
    constexpr int LPT = D / 2;                  // lanes per token
    constexpr int TPW = 64 / LPT;               // tokens per wave step
    const int h = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPT;
    const int c0 = 2 * (lane % LPT);
    const int C = p.H * D;
    const int Km1 = p.K - 1;

    // this lane's conv taps: [stream][channel pair][tap]
    float w[3][2][4];
#pragma unroll
    for (int X = 0; X < 3; ++X)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[X][e][j] = j < p.K ? p.conv_w[((long)X * C + h * D + c0 + e) * p.K + j] : 0.0f;

    const long tok_base = (long)blockIdx.x * (4 * TPW * kSteps);
    for (int step = 0; step < kSteps; ++step) {
        const long t = tok_base + (long)(step * 4 + wave) * TPW + sub;
        const bool valid = t < p.T;
        float x[3][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
        if (valid) {
            const int n = find_seq(p.cu, p.n_seqs, t);
            const long start = p.cu[n];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < p.K) {
                    const long tau = t - Km1 + j;
#pragma unroll
                    for (int X = 0; X < 3; ++X) {
                        const void *raw = X == 0 ? p.q_raw : (X == 1 ? p.k_raw : p.v_raw);
                        float2 v;
                        if (tau >= start) {
                            v = load2<DT>(raw, (tau * p.H + h) * D + c0);
                        } else if (p.cache_in) {
                            const float *cp = p.cache_in +
                                (((long)n * 3 + X) * Km1 + (Km1 - (start - tau))) * C + h * D + c0;
                            v = *reinterpret_cast<const float2 *>(cp);
                        } else {
                            v = make_float2(0.f, 0.f);
                        }
                        x[X][0] += w[X][0][j] * v.x;
                        x[X][1] += w[X][1][j] * v.y;
                    }
                }
            }
#pragma unroll
            for (int X = 0; X < 3; ++X) {
                x[X][0] = activate(p.act, x[X][0]);
                x[X][1] = activate(p.act, x[X][1]);
            }
        }
        // L2 over the token's D channels (LPT lanes); every lane takes part
        const float sq = group_sum(x[0][0] * x[0][0] + x[0][1] * x[0][1], LPT);
        const float sk = group_sum(x[1][0] * x[1][0] + x[1][1] * x[1][1], LPT);
        if (valid) {
            const float rq = 1.0f / sqrtf(sq + p.eps), rk = 1.0f / sqrtf(sk + p.eps);
            const long o = (t * p.H + h) * D + c0;
            store2<DT>(p.q_out, o, x[0][0] * rq, x[0][1] * rq);
            store2<DT>(p.k_out, o, x[1][0] * rk, x[1][1] * rk);
            store2<DT>(p.v_out, o, x[2][0], x[2][1]);
            if (p.gate_logit) {
                const float2 gl = load2<DT>(p.gate_logit, o);
                store2<DT>(p.gate_out, o, sigmoidf(gl.x), sigmoidf(gl.y));
            }
            if (c0 == 0) p.beta_out[t * p.H + h] = sigmoidf(load1<DT>(p.beta_logit, t * p.H + h));
        }
    }
}

// Head dim 128: a wave owns 16 consecutive token rows of one head (lane l has
// channels 2l, 2l+1).  A block takes 4 adjacent heads of the same 16 tokens.  It issues the loads of all 16 rows plus the K-1 rows
// before them at once, keeps them as a register window, and convolves from
// the window; taps that fall before the token's sequence start read the
// incoming conv cache instead (a wave-uniform branch).
template <int K, int DT>
__global__ __launch_bounds__(256) void prologue128_kernel(PrologueParams p) {
    constexpr int D = 128, R = 16, Km1 = K - 1, NW = R + Km1;
    // block = 16 tokens x 4 adjacent heads (wave w: head 4 hg + w); head
    // groups vary fastest, so concurrent waves read whole contiguous token rows
    const int n_hg = (p.H + 3) / 4;
    const int hg = blockIdx.x % n_hg;
    const long tb = blockIdx.x / n_hg;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int h = hg * 4 + wave;
    const int c0 = 2 * lane;
    const int C = p.H * D;
    const long t0 = tb * R;
    if (h >= p.H || t0 >= p.T) return;

    float w[3][2][K];
#pragma unroll
    for (int X = 0; X < 3; ++X)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int j = 0; j < K; ++j) w[X][e][j] = p.conv_w[((long)X * C + h * D + c0 + e) * K + j];

    // window rows t0-Km1 .. t0+R-1, all loads issued before any use.  Row
    // indices are clamped into [0, T) so every load is unconditional; a
    // clamped row is never used (taps before a sequence start read the cache).
    uint2 win[3][NW];
#pragma unroll
    for (int r = 0; r < NW; ++r) {
        const long tau = t0 - Km1 + r;
        const long tc = tau < 0 ? 0 : (tau >= p.T ? p.T - 1 : tau);
#pragma unroll
        for (int X = 0; X < 3; ++X) {
            const void *raw = X == 0 ? p.q_raw : (X == 1 ? p.k_raw : p.v_raw);
            win[X][r] = load_raw2<DT>(raw, (tc * p.H + h) * D + c0);
        }
    }
    uint2 gl[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const long tc = t0 + i < p.T ? t0 + i : p.T - 1;
        gl[i] = p.gate_logit ? load_raw2<DT>(p.gate_logit, (tc * p.H + h) * D + c0) : make_uint2(0u, 0u);
    }
    const long tb_ = t0 + (lane & (R - 1));
    const float beta_l = load1<DT>(p.beta_logit, (tb_ < p.T ? tb_ : p.T - 1) * p.H + h);

    int n = find_seq(p.cu, p.n_seqs, t0);
    long start = p.cu[n], end = p.cu[n + 1];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const long t = t0 + i;
        if (t >= p.T) break;
        while (t >= end) {   // next non-empty sequence (tokens rise within the wave)
            ++n;
            start = p.cu[n];
            end = p.cu[n + 1];
        }
        float x[3][2];
        if (t - Km1 >= start) {
#pragma unroll
            for (int X = 0; X < 3; ++X) {
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const float2 v = unpack2<DT>(win[X][i + j]);
                    a0 += w[X][0][j] * v.x;
                    a1 += w[X][1][j] * v.y;
                }
                x[X][0] = a0;
                x[X][1] = a1;
            }
        } else {
#pragma unroll
            for (int X = 0; X < 3; ++X) {
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const long tau = t - Km1 + j;
                    float2 v;
                    if (tau >= start) {
                        v = unpack2<DT>(win[X][i + j]);
                    } else if (p.cache_in) {
                        v = *reinterpret_cast<const float2 *>(
                            p.cache_in + (((long)n * 3 + X) * Km1 + (Km1 - (start - tau))) * C + h * D + c0);
                    } else {
                        v = make_float2(0.f, 0.f);
                    }
                    a0 += w[X][0][j] * v.x;
                    a1 += w[X][1][j] * v.y;
                }
                x[X][0] = a0;
                x[X][1] = a1;
            }
        }
#pragma unroll
        for (int X = 0; X < 3; ++X) {
            x[X][0] = activate(p.act, x[X][0]);
            x[X][1] = activate(p.act, x[X][1]);
        }
        const float r = __builtin_amdgcn_rsqf(
            wave_sum_pair(x[0][0] * x[0][0] + x[0][1] * x[0][1], x[1][0] * x[1][0] + x[1][1] * x[1][1]) + p.eps);
        const float rq = lane_value(r, 0), rk = lane_value(r, 16);
        const long o = (t * p.H + h) * D + c0;
        store2<DT>(p.q_out, o, x[0][0] * rq, x[0][1] * rq);
        store2<DT>(p.k_out, o, x[1][0] * rk, x[1][1] * rk);
        store2<DT>(p.v_out, o, x[2][0], x[2][1]);
        if (p.gate_logit) {
            const float2 gv = unpack2<DT>(gl[i]);
            store2<DT>(p.gate_out, o, sigmoidf(gv.x), sigmoidf(gv.y));
        }
    }
    if (lane < R && tb_ < p.T) p.beta_out[tb_ * p.H + h] = sigmoidf(beta_l);
}

// Outgoing conv cache: the last K-1 raw inputs of each sequence, reaching
// into the incoming cache when the sequence is shorter than K-1.  Slot j takes
// raw token end-(K-1)+j, or incoming slot j+len; slots are visited in rising
// order so an aliased in/out buffer is read before it is overwritten.
template <int DT>
__global__ __launch_bounds__(256) void conv_cache_out_kernel(PrologueParams p, int nblk) {
    const int C = p.H * p.d;
    const int Km1 = p.K - 1;
    const int nx = blockIdx.x / nblk;          // n * 3 + X
    const int ch = (blockIdx.x - nx * nblk) * 256 + threadIdx.x;
    if (ch >= C) return;
    const int n = nx / 3, X = nx - n * 3;
    const long start = p.cu[n], end = p.cu[n + 1], len = end - start;
    const void *raw = X == 0 ? p.q_raw : (X == 1 ? p.k_raw : p.v_raw);
    for (int j = 0; j < Km1; ++j) {
        const long tau = end - Km1 + j;
        float v;
        if (tau >= start) v = load1<DT>(raw, tau * C + ch);
        else v = p.cache_in ? p.cache_in[((long)nx * Km1 + (j + len)) * C + ch] : 0.0f;
        p.cache_out[((long)nx * Km1 + j) * C + ch] = v;
    }
}

template <int D, int DT>
hipError_t launch_pd(const PrologueParams &p, hipStream_t s) {
    if (p.T > 0) {
        if constexpr (D == 128) {
            dim3 grid((unsigned)(((p.T + 15) / 16) * ((p.H + 3) / 4)));
            switch (p.K) {
                case 1: hipLaunchKernelGGL((prologue128_kernel<1, DT>), grid, dim3(256), 0, s, p); break;
                case 2: hipLaunchKernelGGL((prologue128_kernel<2, DT>), grid, dim3(256), 0, s, p); break;
                case 3: hipLaunchKernelGGL((prologue128_kernel<3, DT>), grid, dim3(256), 0, s, p); break;
                default: hipLaunchKernelGGL((prologue128_kernel<4, DT>), grid, dim3(256), 0, s, p); break;
            }
        } else {
            constexpr int TPW = 64 / (D / 2);
            const long per_block = 4L * TPW * kSteps;
            dim3 grid((unsigned)((p.T + per_block - 1) / per_block), p.H);
            hipLaunchKernelGGL((prologue_kernel<D, DT>), grid, dim3(256), 0, s, p);
        }
    }
    if (p.cache_out && p.K > 1) {
        const int nblk = (p.H * D + 255) / 256;
        hipLaunchKernelGGL((conv_cache_out_kernel<DT>), dim3((unsigned)(nblk * 3 * p.n_seqs)),
                           dim3(256), 0, s, p, nblk);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_p(const PrologueParams &p, hipStream_t s) {
    switch (p.d) {
        case 4: return launch_pd<4, DT>(p, s);
        case 8: return launch_pd<8, DT>(p, s);
        case 16: return launch_pd<16, DT>(p, s);
        case 32: return launch_pd<32, DT>(p, s);
        case 64: return launch_pd<64, DT>(p, s);
        case 128: return launch_pd<128, DT>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_conv_cache_out(const PrologueParams &p, int dtype, hipStream_t s) {
    if (p.cache_out && p.K > 1) {
        const int nblk = (p.H * p.d + 255) / 256;
        const dim3 grid((unsigned)(nblk * 3 * p.n_seqs));
        if (dtype == 1) hipLaunchKernelGGL((conv_cache_out_kernel<1>), grid, dim3(256), 0, s, p, nblk);
        else hipLaunchKernelGGL((conv_cache_out_kernel<0>), grid, dim3(256), 0, s, p, nblk);
    }
    return hipGetLastError();
}

hipError_t launch_prologue(const PrologueParams &p, int dtype, hipStream_t s) {
    return dtype == 1 ? launch_p<1>(p, s) : launch_p<0>(p, s);
}

}  // namespace kda
