// MLA decode token for gfx950 (kimi_k3 API docs, Functions: mla_decode_token,
// whose steps are optional RoPE, K/V append, SDPA and an optional output
// gate, with the projections left to the MLA mixer; gated_mla_attend, the
// gated NoPE form without the rotary step).  Per sequence b and query head h,
// with kv head h / (H / H_kv) and pos = cache_len[b]:
//   the new token's k and v are written to the cache at pos, then
//   o = softmax_j(scale q . k_j) v_j over j = 0 .. pos, out = o * sigmoid(gate).
//
// Decode attention is a stream over the cache with a few flops per byte, so
// the design is for HBM bandwidth, without MFMA:
//   attend: one block of four waves per (256-token split, q head, sequence),
//     the split index slowest in the grid: every sequence's first splits are
//     dispatched first and the last, partial or empty ones at the end, so the
//     launch does not end on a round of full splits.  The q heads of one kv
//     group run on one XCD and share its L2.
//     Eight lanes share one cached token: a k or v row is cut into chunks of
//     eight channels (16 bytes of bf16), chunk c held by lane c % 8 of the
//     token's lane group, so every load instruction reads whole 128-byte runs.
//     The next iteration's rows are requested before the current ones are
//     used.  The q . k partial sums meet across the eight lanes by xor
//     shuffles; each lane group keeps its own running max, sum and weighted
//     value sum over its tokens (no cross-group step inside the loop); the
//     groups, then the waves, merge at the end, and the block writes one
//     (max, sum, weighted sum) partial.  The block whose split holds pos
//     also takes the new token from k_new / v_new (so no block reads a slot
//     that another block is writing) and writes it into the cache.  When
//     every kv head serves one q head (H = H_kv), each cached row is read by
//     one block only, and its loads are marked non-temporal.
//   combine: per (q head, sequence), merges the split partials in one pass
//     (eight splits' loads at a time, rescaled to a running max), applies the
//     gate and writes bf16.
// Loads go through buffer resources: rows past the cache end read as zero.
#include <cmath>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kSplit = 256;      // cached tokens per attend block
constexpr int kThreads = 256;    // four waves, 64 tokens each, 8 per iteration

// 8 bf16 of one chunk of a row (row_elem0 = the row's first element), or
// zeros where the chunk lies past d; VEC: the chunk is whole and 16-byte
// aligned, one load; otherwise element by element.  NT: a row read once
// (the cache policy's non-temporal bit).
template <bool VEC, bool NT = false>
__device__ __forceinline__ u32x4 load_chunk(__amdgpu_buffer_rsrc_t r, long row_elem0, int d, int chunk,
                                            bool valid) {
    if constexpr (VEC) {
        const uint32_t off = (valid && chunk * 8 < d) ? (uint32_t)((row_elem0 + chunk * 8) * 2) : 0xffffffffu;
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0);
    } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = chunk * 8 + e;
            const uint32_t off = (valid && c < d) ? (uint32_t)((row_elem0 + c) * 2) : 0xffffffffu;
            h[e] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
        }
        return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
}

__device__ __forceinline__ void unpack8(const u32x4 &w, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = lo_bf(w[i]);
        x[2 * i + 1] = hi_bf(w[i]);
    }
}

// merge (m2, l2, a2) into (m, l, a): the softmax partials of two disjoint
// token sets
template <int N>
__device__ __forceinline__ void merge(float &m, float &l, float (&a)[N], float m2, float l2, const float (&a2)[N]) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;   // both empty
    const float s1 = __expf(m - M), s2 = __expf(m2 - M);
    l = l * s1 + l2 * s2;
#pragma unroll
    for (int i = 0; i < N; ++i) a[i] = a[i] * s1 + a2[i] * s2;
    m = M;
}

// KC, VC: 8-channel chunks per lane for k and v (d_qk <= 64 KC, d_v <= 64 VC);
// NT: cache rows are loaded non-temporally (each is read by this block only)
template <int KC, int VC, bool VEC, bool NT>
__global__ __launch_bounds__(kThreads) void mla_attend_kernel(MlaParams p) {
    __shared__ float red_ml[4][2];
    __shared__ float red_acc[4][8 * 8 * VC];
    const int b = blockIdx.y, s = blockIdx.z;
    // Blocks go to the eight XCDs in turn, so with H a multiple of 8, grid x
    // and x + 8 share an XCD: XCD k takes heads k H / 8 .. (k + 1) H / 8 - 1,
    // and the q heads of one kv group meet in one L2.
    const int h = (p.H & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (p.H >> 3) + (int)(blockIdx.x >> 3);
    const int pos = p.cache_len[b];
    if (pos < 0 || pos >= p.max_len || s > pos / kSplit) return;   // block-uniform
    const int hk = h / (p.H / p.H_kv);
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, tg = l >> 3, li = l & 7;
    const int dqk = p.dqk, dv = p.dv;

    // this lane's chunks of q, scale folded in
    float qr[KC][8];
    {
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(p.q, (uint32_t)((long)p.batch * p.H * dqk * 2));
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            unpack8(load_chunk<VEC>(rq, ((long)b * p.H + h) * dqk, dqk, 8 * c + li, true), qr[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) qr[c][e] *= p.scale;
        }
    }
    const long row0 = ((long)b * p.H_kv + hk) * p.max_len;   // cache row of token 0
    const __amdgpu_buffer_rsrc_t rk =
        buffer_rsrc(static_cast<const uint16_t *>(p.k_cache) + row0 * dqk, (uint32_t)((long)p.max_len * dqk * 2));
    const __amdgpu_buffer_rsrc_t rv =
        buffer_rsrc(static_cast<const uint16_t *>(p.v_cache) + row0 * dv, (uint32_t)((long)p.max_len * dv * 2));

    float m = -INFINITY, lsum = 0.0f, acc[VC * 8];
#pragma unroll
    for (int i = 0; i < VC * 8; ++i) acc[i] = 0.0f;

    // one token's score and value into this lane group's running partial
    auto absorb = [&](const u32x4 (&kr)[KC], const u32x4 (&vr)[VC], bool valid) {
        float dot = 0.0f;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            float x[8];
            unpack8(kr[c], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(qr[c][e], x[e], dot);
        }
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        dot += __shfl_xor(dot, 4);
        if (valid) {
            const float mn = fmaxf(m, dot);
            const float sc = __expf(m - mn), pj = __expf(dot - mn);
            lsum = lsum * sc + pj;
#pragma unroll
            for (int c = 0; c < VC; ++c) {
                float x[8];
                unpack8(vr[c], x);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[8 * c + e] = fmaf(pj, x[e], acc[8 * c + e] * sc);
            }
            m = mn;
        }
    };

    // the cached tokens j < pos of this wave's 64: iteration it takes tokens
    // j0 + 8 it .. + 7, lane group tg the token j0 + 8 it + tg
    const int j0 = s * kSplit + w * 64;
    if (j0 < pos) {
        u32x4 kb[2][KC], vb[2][VC];
        auto fetch = [&](int it, u32x4 (&kr)[KC], u32x4 (&vr)[VC]) {
            const int j = j0 + 8 * it + tg;
            const bool valid = j < pos;
#pragma unroll
            for (int c = 0; c < KC; ++c) kr[c] = load_chunk<VEC, NT>(rk, (long)j * dqk, dqk, 8 * c + li, valid);
#pragma unroll
            for (int c = 0; c < VC; ++c) vr[c] = load_chunk<VEC, NT>(rv, (long)j * dv, dv, 8 * c + li, valid);
        };
        fetch(0, kb[0], vb[0]);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            if (it + 1 < 8) fetch(it + 1, kb[(it + 1) & 1], vb[(it + 1) & 1]);
            absorb(kb[it & 1], vb[it & 1], j0 + 8 * it + tg < pos);
        }
    }

    // the new token, in the split that holds pos: wave 0 scores it (every
    // lane group alike), group 0 takes it
    const bool owner = s == pos / kSplit;
    if (owner && w == 0) {
        const __amdgpu_buffer_rsrc_t rkn = buffer_rsrc(p.k_new, (uint32_t)((long)p.batch * p.H_kv * dqk * 2));
        const __amdgpu_buffer_rsrc_t rvn = buffer_rsrc(p.v_new, (uint32_t)((long)p.batch * p.H_kv * dv * 2));
        u32x4 kr[KC], vr[VC];
#pragma unroll
        for (int c = 0; c < KC; ++c)
            kr[c] = load_chunk<VEC>(rkn, ((long)b * p.H_kv + hk) * dqk, dqk, 8 * c + li, true);
#pragma unroll
        for (int c = 0; c < VC; ++c)
            vr[c] = load_chunk<VEC>(rvn, ((long)b * p.H_kv + hk) * dv, dv, 8 * c + li, true);
        absorb(kr, vr, tg == 0);
        // append (one q head of the group writes)
        if (h % (p.H / p.H_kv) == 0) {
            const uint16_t *kn = static_cast<const uint16_t *>(p.k_new) + ((long)b * p.H_kv + hk) * dqk;
            const uint16_t *vn = static_cast<const uint16_t *>(p.v_new) + ((long)b * p.H_kv + hk) * dv;
            uint16_t *kc = static_cast<uint16_t *>(p.k_cache) + (row0 + pos) * dqk;
            uint16_t *vc = static_cast<uint16_t *>(p.v_cache) + (row0 + pos) * dv;
            for (int e = l; e < dqk; e += 64) kc[e] = kn[e];
            for (int e = l; e < dv; e += 64) vc[e] = vn[e];
        }
    }

    // merge the eight lane groups (lanes li, li + 8, ... hold the same channels)
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
        float a2[VC * 8];
#pragma unroll
        for (int i = 0; i < VC * 8; ++i) a2[i] = __shfl_xor(acc[i], off);
        const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(lsum, off);
        merge(m, lsum, acc, m2, l2, a2);
    }
    // then the four waves, through LDS; group 0 of each wave holds its partial
    if (tg == 0) {
#pragma unroll
        for (int c = 0; c < VC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) red_acc[w][64 * c + 8 * li + e] = acc[8 * c + e];
        if (li == 0) {
            red_ml[w][0] = m;
            red_ml[w][1] = lsum;
        }
    }
    __syncthreads();
    // thread t owns channel t: chunk t / 8 sits in register slot t / 64 of
    // lane (t / 8) % 8, stored above at 64 (t / 64) + t % 64
    const long pidx = ((long)b * p.H + h) * p.n_split + s;
    if (tid < dv) {
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k) M = fmaxf(M, red_ml[k][0]);
        float a = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (red_ml[k][0] != -INFINITY) a += red_acc[k][tid] * __expf(red_ml[k][0] - M);
        p.ws_acc[pidx * dv + tid] = a;
    }
    if (tid == 0) {
        float M = -INFINITY, L = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) M = fmaxf(M, red_ml[k][0]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (red_ml[k][0] != -INFINITY) L += red_ml[k][1] * __expf(red_ml[k][0] - M);
        p.ws_ml[2 * pidx] = M;
        p.ws_ml[2 * pidx + 1] = L;
    }
}

__global__ __launch_bounds__(256) void mla_combine_kernel(MlaParams p) {
    const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    if (t >= p.dv) return;
    const long ob = ((long)b * p.H + h) * p.dv + t;
    uint16_t *out = static_cast<uint16_t *>(p.out) + ob;
    const float gz = p.gate ? bf2f(static_cast<const uint16_t *>(p.gate)[ob]) : 0.0f;
    const int pos = p.cache_len[b];
    if (pos < 0 || pos >= p.max_len) {
        *out = 0;
        return;
    }
    const int ns = pos / kSplit + 1;   // every split below ns holds at least one token
    const long base = ((long)b * p.H + h) * p.n_split;
    // split partials past ns read as (-inf, 0, 0) through the resources' ends
    const __amdgpu_buffer_rsrc_t rml = buffer_rsrc(p.ws_ml + 2 * base, (uint32_t)(2 * ns * 4));
    const __amdgpu_buffer_rsrc_t racc = buffer_rsrc(p.ws_acc + base * p.dv, (uint32_t)((long)ns * p.dv * 4));
    float M = -INFINITY, L = 0.0f, a = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += 8) {
        float ms[8], ls[8], as[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int s = s0 + k;
            ms[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rml, (uint32_t)(8 * s), 0, 0));
            ls[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rml, (uint32_t)(8 * s + 4), 0, 0));
            as[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(racc, (uint32_t)(((long)s * p.dv + t) * 4), 0, 0));
            if (s >= ns) ms[k] = -INFINITY;
        }
        float Mn = M;
#pragma unroll
        for (int k = 0; k < 8; ++k) Mn = fmaxf(Mn, ms[k]);
        const float sc = M == -INFINITY ? 0.0f : __expf(M - Mn);   // Mn is finite: split s0 holds a token
        L *= sc;
        a *= sc;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float e = ms[k] == -INFINITY ? 0.0f : __expf(ms[k] - Mn);
            L += ls[k] * e;
            a += as[k] * e;
        }
        M = Mn;
    }
    float o = a / L;
    if (p.gate) o *= sigmoidf(gz);
    *out = f2bf(o);
}

template <int KC, int VC, bool VEC>
void launch_attend(const MlaParams &p, hipStream_t st) {
    const dim3 grid(p.H, p.batch, p.n_split);
    if (p.H == p.H_kv) hipLaunchKernelGGL((mla_attend_kernel<KC, VC, VEC, true>), grid, dim3(kThreads), 0, st, p);
    else hipLaunchKernelGGL((mla_attend_kernel<KC, VC, VEC, false>), grid, dim3(kThreads), 0, st, p);
}

}  // namespace

int mla_split_tokens() { return kSplit; }

hipError_t launch_mla_decode(const MlaParams &p, bool vec, hipStream_t st) {
    if (p.batch == 0) return hipGetLastError();
    const int kc = (p.dqk + 63) / 64, vc = (p.dv + 63) / 64;
    if (vec) {
        if (kc <= 1 && vc <= 1) launch_attend<1, 1, true>(p, st);
        else if (kc <= 2 && vc <= 2) launch_attend<2, 2, true>(p, st);
        else if (kc <= 3 && vc <= 2) launch_attend<3, 2, true>(p, st);
        else launch_attend<4, 4, true>(p, st);
    } else {
        if (kc <= 1 && vc <= 1) launch_attend<1, 1, false>(p, st);
        else launch_attend<4, 4, false>(p, st);
    }
    hipLaunchKernelGGL(mla_combine_kernel, dim3(p.H, p.batch), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace kda
