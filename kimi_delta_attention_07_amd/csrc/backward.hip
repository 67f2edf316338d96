// Backward of the chunked KDA prefill for gfx950 (head dim 128, 64-token
// chunks, bf16 forward inputs and output gradient, fp32 gradients).
//
// Per chunk, with entry state S0 and (as in the forward)
//   G = cumsum(log alpha),  Qd = Q e^G,  Kd = K e^G,  Ki = K e^-G,
//   Kg = K e^{G_L - G},  gL = e^{G_L}  (G_L: G at the chunk's last token)
//   A = tril(diag(beta) Kd Ki^T, -1),  T = (I + A)^-1,  TB = T diag(beta)
//   W = TB Kd,  U~ = TB V,  U = U~ - W S0,  Pm = tril(Qd Ki^T)
//   O = Qd S0 + Pm U,  y = scale O (.) g,  S_L = diag(gL) S0 + Kg^T U
// reverse differentiation of these products gives, with dO = scale dy (.) g
// and dS_L the gradient arriving at the chunk's end state:
//   dU  = Pm^T dO + Kg dS_L
//   dS0 = diag(gL) dS_L + Qd^T dO - W^T dU            (chained chunk to chunk)
//   dPm = tril(dO U^T),  dQd = dO S0^T + dPm Ki,  dW = -dU S0^T,  dKg = U dS_L^T
//   dTB = dW Kd^T + dU V^T,  dKd = TB^T dW,  dV = TB^T dU,  dT = dTB diag(beta)
//   dA  = -tril(T^T dT T^T, -1)
//   dKd += diag(beta) dA Ki,  dKi = (diag(beta) dA)^T Kd + dPm^T Qd
//   dbeta_j = sum_i dTB_ij T_ij + sum_m dA_jm (Kd Ki^T)_jm
//   dq = dQd e^G,  dk = dKd e^G + dKi e^-G + dKg e^{G_L - G}
//   dG = dQd Qd + dKd Kd - dKi Ki - dKg Kg,
//   dG_L = colsum(dKg Kg) + gL rowsum(S0 dS_L)
//   dlog alpha_t = sum_{s >= t} dG_s + dG_L,   dg = dy (.) scale O
// (the forward's WY/UT form is the one in chunk.hip; see the oracle for the
// same gradient taken token by token).
//
// Five kernels, all in fp32:
//   do          chunks x heads: dO = scale dy (.) g (elementwise)
//   prep        chunks x heads: G, the decayed operands, A, T (blocked
//               forward substitution), -W, U~, Pm
//   fwd_states  sequences x heads x 8 value tiles: walks the chunks forward,
//               writes each chunk's S0 and U (fp32 MFMA)
//   bwd_states  the same grid backwards: dS_L and dU per chunk, and the
//               gradient of the initial state (fp32 MFMA)
//   grads       chunks x heads: the per-chunk products above, then dq, dk, dv,
//               dlog alpha, dbeta and dgate (VALU, LDS-staged)
// Rows past a chunk's end load as zeros, which makes every padded row of
// every operand (and so of every product) zero, and keeps G at G_L there.
#include "kda_chunk_table.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kNT = 256;

// Per (chunk, head) workspace layout, in floats; [64][128] and [128][128]
// matrices row-major with 128 columns, [64][64] with 64.
constexpr long kM = 64 * 128, kSq = 64 * 64, kS = 128 * 128;
constexpr long bG = 0, bQd = bG + kM, bKd = bQd + kM, bKi = bKd + kM, bKg = bKi + kM, bV = bKg + kM;
constexpr long bW = bV + kM, bUt = bW + kM, bTB = bUt + kM, bT = bTB + kSq, bPm = bT + kSq, bGL = bPm + kSq;
constexpr long bS0 = bGL + 128, bU = bS0 + kS, bdSL = bU + kM, bdO = bdSL + kS, bdU = bdO + kM;
constexpr long bdW = bdU + kM;
constexpr long kBwdFloats = bdW + kM;   // 143,488 floats (the gradient kernel keeps its other intermediates on chip)
static_assert(kBwdFloats * 4 == 573952, "the workspace size documented in kda.h");
// The prep kernel stores -W (not W) in the bW slot: only the state passes
// read it.

__device__ __forceinline__ float *chunk_buf(const BwdParams &p, long cid, int h) {
    return p.buf + (cid * p.c.H + h) * kBwdFloats;
}

// Sequence n's chunk range [c_begin, c_end) and its first token and length,
// sanitised like the forward scan's and kept in scalar registers (chunk j of
// the sequence then starts at seq_start + 64 j: no table lookup per chunk).
__device__ __forceinline__ void seq_chunks(const ChunkParams &c, int n, int &c_begin, int &c_end, int &seq_start,
                                           int &seq_len) {
    const int off0 = c.plan_in_args ? c.plan_off[n] : c.chunk_off[n];
    const int off1 = c.plan_in_args ? c.plan_off[n + 1] : c.chunk_off[n + 1];
    const int cu0 = c.plan_in_args ? c.plan_cu[n] : c.cu[n];
    const int cu1 = c.plan_in_args ? c.plan_cu[n + 1] : c.cu[n + 1];
    c_begin = __builtin_amdgcn_readfirstlane(max(0, off0));
    c_end = __builtin_amdgcn_readfirstlane(min(c.n_chunks, off1));
    seq_start = __builtin_amdgcn_readfirstlane(min(max(cu0, 0), c.T));
    seq_len = __builtin_amdgcn_readfirstlane(max(0, min(cu1, c.T) - seq_start));
}

// C[0:64][0:N] (= or +=) alpha op(A)[64][K] op(B)[K][N], by all 256 threads.
//   op(A)[i][k] = TA ? A[k lda + i] : A[i lda + k]
//   op(B)[k][j] = TB ? B[j ldb + k] : B[k ldb + j]
// MASK 1 keeps entries j <= i, 2 keeps j < i (the rest are written as 0, or
// left alone when accumulating); rows >= mrows are not written.  N is 64 or
// 128, K a multiple of 16 HALVES; operands 16-byte aligned with lda, ldb multiples of
// 4.  The operands may be in global memory (written earlier by this block:
// the barrier on entry orders them) or in LDS.
template <bool TA, bool TB, int N, int HALVES, bool DEEP = false>
__device__ void bmm_acc(f32x4 (&acc)[N / 16], const float *A, int lda, const float *B, int ldb, int K, float *sm) {
    constexpr int LA = 68, LB = 132;   // LDS rows, padded (multiples of 4 for 16-byte accesses)
    constexpr int KS = 16 * HALVES;    // k slab
    float *As = sm;                    // [KS][LA]: As[kk][i]
    float *Bs = sm + KS * LA;          // [KS][LB]: Bs[kk][j]
    const int tid = threadIdx.x;
    // The k range goes in slabs of KS = 16 HALVES, staged in LDS as halves of 16;
    // this thread's share of a half: one 16-byte piece of op(A), one or two
    // of op(B).  The next slab is fetched while this one is used.
    const int ai = TA ? (tid & 15) * 4 : tid >> 2, ak = TA ? tid >> 4 : (tid & 3) * 4;
    auto a_ptr = [&](int k0) { return TA ? A + (long)(k0 + ak) * lda + ai : A + (long)ai * lda + k0 + ak; };
    auto b_pos = [&](int e, int &j, int &k) {
        if (TB) {
            j = e >> 2;
            k = (e & 3) * 4;
        } else {
            const int q = N >> 2;
            k = e / q;
            j = (e % q) * 4;
        }
    };
    auto b_ptr = [&](int k0, int e) {
        int j, k;
        b_pos(e, j, k);
        return TB ? B + (long)j * ldb + k0 + k : B + (long)(k0 + k) * ldb + j;
    };
    auto put_a = [&](const float4 &v, int kb) {
        if (TA) {
            *reinterpret_cast<float4 *>(As + (kb + ak) * LA + ai) = v;
        } else {
            As[(kb + ak) * LA + ai] = v.x;
            As[(kb + ak + 1) * LA + ai] = v.y;
            As[(kb + ak + 2) * LA + ai] = v.z;
            As[(kb + ak + 3) * LA + ai] = v.w;
        }
    };
    auto put_b = [&](const float4 &v, int e, int kb) {
        int j, k;
        b_pos(e, j, k);
        k += kb;
        if (TB) {
            Bs[k * LB + j] = v.x;
            Bs[(k + 1) * LB + j] = v.y;
            Bs[(k + 2) * LB + j] = v.z;
            Bs[(k + 3) * LB + j] = v.w;
        } else {
            *reinterpret_cast<float4 *>(Bs + k * LB + j) = v;
        }
    };
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    // [half]: A piece, B pieces (second only for N = 128); the s* set holds the
    // odd slabs when DEEP (two slabs in flight)
    float4 ra0, ra1 = z4, rb00, rb10 = z4, rb01 = z4, rb11 = z4;
    float4 sa0 = z4, sa1 = z4, sb00 = z4, sb10 = z4, sb01 = z4, sb11 = z4;
    auto fetch_set = [&](int k0, float4 &a0, float4 &a1, float4 &b00, float4 &b10, float4 &b01, float4 &b11) {
        a0 = *reinterpret_cast<const float4 *>(a_ptr(k0));
        b00 = *reinterpret_cast<const float4 *>(b_ptr(k0, tid));
        if constexpr (N == 128) b01 = *reinterpret_cast<const float4 *>(b_ptr(k0, tid + kNT));
        if constexpr (HALVES == 2) {
            a1 = *reinterpret_cast<const float4 *>(a_ptr(k0 + 16));
            b10 = *reinterpret_cast<const float4 *>(b_ptr(k0 + 16, tid));
            if constexpr (N == 128) b11 = *reinterpret_cast<const float4 *>(b_ptr(k0 + 16, tid + kNT));
        }
    };
    auto fetch = [&](int k0) { fetch_set(k0, ra0, ra1, rb00, rb10, rb01, rb11); };
    // wave w: output rows 16 w .. 16 w + 15, N / 16 column blocks, on fp32
    // MFMAs; lane l supplies op(A)[16 w + l % 16][k] and op(B)[k][16 nb + l % 16]
    // for k = k0 + 4 t + l / 16 and holds C[16 w + 4 (l / 16) + r][16 nb + l % 16]
    constexpr int NB = N / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lg = l >> 4, lc = l & 15;
    auto put_set = [&](const float4 &a0, const float4 &a1, const float4 &b00, const float4 &b10, const float4 &b01,
                       const float4 &b11) {
        put_a(a0, 0);
        put_b(b00, tid, 0);
        if constexpr (N == 128) put_b(b01, tid + kNT, 0);
        if constexpr (HALVES == 2) {
            put_a(a1, 16);
            put_b(b10, tid, 16);
            if constexpr (N == 128) put_b(b11, tid + kNT, 16);
        }
    };
    auto slab = [&]() {
#pragma unroll
        for (int t = 0; t < 4 * HALVES; ++t) {
            const int kk = 4 * t + lg;
            const float a = As[kk * LA + 16 * w + lc];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma_f32(a, Bs[kk * LB + 16 * nb + lc], acc[nb]);
        }
    };
    __syncthreads();   // operands written earlier by this block are complete; staging is free
    if constexpr (!DEEP) {
        fetch(0);
        for (int k0 = 0; k0 < K; k0 += KS) {
            put_set(ra0, ra1, rb00, rb10, rb01, rb11);
            __syncthreads();
            if (k0 + KS < K) fetch(k0 + KS);
            slab();
            __syncthreads();
        }
    } else {   // two register sets used in turn, each refilled right after it reached LDS
        fetch_set(0, ra0, ra1, rb00, rb10, rb01, rb11);
        if (KS < K) fetch_set(KS, sa0, sa1, sb00, sb10, sb01, sb11);
        for (int k0 = 0; k0 < K; k0 += 2 * KS) {
            put_set(ra0, ra1, rb00, rb10, rb01, rb11);
            __syncthreads();
            if (k0 + 2 * KS < K) fetch_set(k0 + 2 * KS, ra0, ra1, rb00, rb10, rb01, rb11);
            slab();
            __syncthreads();
            if (k0 + KS < K) {
                put_set(sa0, sa1, sb00, sb10, sb01, sb11);
                __syncthreads();
                if (k0 + 3 * KS < K) fetch_set(k0 + 3 * KS, sa0, sa1, sb00, sb10, sb01, sb11);
                slab();
                __syncthreads();
            }
        }
    }
}

template <int MASK, bool ACC, int N>
__device__ void bmm_store(float *C, int ldc, const f32x4 (&acc)[N / 16], float alpha, int mrows) {
    constexpr int NB = N / 16;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lg = l >> 4, lc = l & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * lg + r;
        if (i >= mrows) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int j = 16 * nb + lc;
            const bool keep = MASK == 0 || (MASK == 1 ? j <= i : j < i);
            float *dst = C + (long)i * ldc + j;
            if (ACC) {
                if (keep) *dst += alpha * acc[nb][r];
            } else {
                *dst = keep ? alpha * acc[nb][r] : 0.f;
            }
        }
    }
}


template <bool TA, bool TB, int MASK, bool ACC, int N, int HALVES = 2, bool DEEP = false>
__device__ void bmm(float *C, int ldc, const float *A, int lda, const float *B, int ldb, int K, float alpha, int mrows,
                    float *sm) {
    f32x4 acc[N / 16];
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bmm_acc<TA, TB, N, HALVES, DEEP>(acc, A, lda, B, ldb, K, sm);
    bmm_store<MASK, ACC, N>(C, ldc, acc, alpha, mrows);
}

// C[0:64][0:N] = alpha (op(A1) op(B1) + op(A2) op(B2)), the two products
// accumulated in the same registers: C is written once, not written, read
// back and written again.
template <bool TA1, bool TB1, bool TA2, bool TB2, int MASK, int N, int HALVES = 2>
__device__ void bmm2(float *C, int ldc, const float *A1, int lda1, const float *B1, int ldb1, int K1, const float *A2,
                     int lda2, const float *B2, int ldb2, int K2, float alpha, int mrows, float *sm) {
    f32x4 acc[N / 16];
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bmm_acc<TA1, TB1, N, HALVES>(acc, A1, lda1, B1, ldb1, K1, sm);
    bmm_acc<TA2, TB2, N, HALVES>(acc, A2, lda2, B2, ldb2, K2, sm);
    bmm_store<MASK, false, N>(C, ldc, acc, alpha, mrows);
}

// ---- dO = scale dy (.) g into every chunk's slot (zero past the chunk's end) --
// A bandwidth-bound pass of its own, kept out of the latency-bound prep
// kernel.  Thread: four channels of one row; rows past the chunk's end load
// its last row (in bounds) and store zeros.
__global__ __launch_bounds__(kNT) void bwd_do_kernel(BwdParams p) {
    const ChunkParams &c = p.c;
    const int H = c.H, h = blockIdx.x % H, cid = blockIdx.x / H, tid = threadIdx.x;
    const ChunkInfo ci = load_chunk(c, cid);
    float *B = chunk_buf(p, cid, h);
    uint2 dy[8], gt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int e = tid + k * kNT, i = e >> 5, c4 = (e & 31) * 4;
        const long src = (((long)ci.start + min(i, ci.len - 1)) * H + h) * kHeadDim + c4;
        dy[k] = *reinterpret_cast<const uint2 *>(p.dy + src);
        gt[k] = c.gate ? *reinterpret_cast<const uint2 *>(c.gate + src) : make_uint2(0x3f803f80u, 0x3f803f80u);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int e = tid + k * kNT, i = e >> 5, c4 = (e & 31) * 4;
        const float sc = i < ci.len ? c.scale : 0.f;
        const float4 v = make_float4(sc * lo_bf(dy[k].x) * lo_bf(gt[k].x), sc * hi_bf(dy[k].x) * hi_bf(gt[k].x),
                                     sc * lo_bf(dy[k].y) * lo_bf(gt[k].y), sc * hi_bf(dy[k].y) * hi_bf(gt[k].y));
        *reinterpret_cast<float4 *>(B + bdO + i * 128 + c4) = v;
    }
}

// ---- prep: the chunk's WY quantities -----------------------------------------
__global__ __launch_bounds__(kNT) void bwd_prep_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(16))) float sm[16 * 68 + 16 * 132];   // 16-wide slabs: three blocks per CU
    __shared__ float big[64 * 128];   // G, then A (first half) and T (second half)
    __shared__ float beta_s[64];
    const ChunkParams &c = p.c;
    const int H = c.H, h = blockIdx.x % H, cid = blockIdx.x / H, tid = threadIdx.x;
    const ChunkInfo ci = load_chunk(c, cid);
    const long tok0 = ci.start;
    const int len = ci.len;
    float *B = chunk_buf(p, cid, h);
    // Loads are issued in batches ahead of the stores that use them: vmcnt
    // counts stores too, so a load waited for behind a store would also wait
    // for that store.  Rows past the chunk's end load its last row (in bounds)
    // and count as zero.
    if (tid < 128) {
        float run = 0.f;
#pragma unroll
        for (int i0 = 0; i0 < 64; i0 += 16) {
            uint16_t la[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) la[t] = c.log_alpha[((tok0 + min(i0 + t, len - 1)) * H + h) * kHeadDim + tid];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                run += i0 + t < len ? bf2f(la[t]) : 0.f;
                big[(i0 + t) * 128 + tid] = run;
                B[bG + (i0 + t) * 128 + tid] = run;
            }
        }
        B[bGL + tid] = expf(run);
    }
    if (tid < 64) beta_s[tid] = tid < len ? c.beta[(tok0 + tid) * H + h] : 0.f;
    __syncthreads();
    {
        const int ch = tid & 127;
        const float gl = big[63 * 128 + ch];
#pragma unroll 1
        for (int k0 = 0; k0 < 32; k0 += 8) {   // element e = tid + 256 k: row 2 k + tid / 128
            uint16_t rq[8], rk[8], rv[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int i = 2 * (k0 + t) + (tid >> 7);
                const long src = ((tok0 + min(i, len - 1)) * H + h) * kHeadDim + ch;
                rq[t] = c.q[src];
                rk[t] = c.k[src];
                rv[t] = c.v[src];
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int e = tid + (k0 + t) * kNT, i = e >> 7;
                const bool in = i < len;
                const float q = in ? bf2f(rq[t]) : 0.f, k = in ? bf2f(rk[t]) : 0.f, v = in ? bf2f(rv[t]) : 0.f;
                const float g = big[e];
                const float eg = expf(g);
                B[bQd + e] = q * eg;
                B[bKd + e] = k * eg;
                B[bKi + e] = k * expf(-g);
                B[bKg + e] = k * expf(gl - g);
                B[bV + e] = v;
            }
        }
    }
    // A = tril(Kd Ki^T, -1), rows scaled by beta
    bmm<false, true, 2, false, 64, 1, true>(big, 64, B + bKd, 128, B + bKi, 128, 128, 1.f, 64, sm);
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += kNT) big[e] *= beta_s[e >> 6];
    __syncthreads();
    // T = (I + A)^-1 by 16 x 16 blocks.  (I + A) T = I gives, for block rows
    // I > J, T_IJ = -D_I sum_{J <= K < I} A_IK T_KJ with D_I = (I + A_II)^-1.
    // Wave w first forms D_w by forward substitution within its diagonal
    // block (T_ij = -sum_{j <= m < i} A_im T_mj, four lanes per column, no
    // block barrier); the off-diagonal blocks then follow one block diagonal
    // at a time (I - J = 1, 2, 3), each in two barrier-separated halves.
    float *Tm = big + 64 * 64;
    __shared__ float xs[3 * 256];   // sum_K A_IK T_KJ of up to three blocks
    for (int e = tid; e < 64 * 64; e += kNT) Tm[e] = (e >> 6) == (e & 63) ? 1.f : 0.f;
    __syncthreads();
    {
        const int w = tid >> 6, l = tid & 63, j = l & 15, q = l >> 4, o = 16 * w;
        for (int ii = 1; ii < 16; ++ii) {
            float sum = 0.f;
            for (int mm = j + q; mm < ii; mm += 4) sum += big[(o + ii) * 64 + o + mm] * Tm[(o + mm) * 64 + o + j];
            sum += __shfl_xor(sum, 16, 64);
            sum += __shfl_xor(sum, 32, 64);
            if (q == 0 && j < ii) Tm[(o + ii) * 64 + o + j] = -sum;
        }
    }
    for (int d = 1; d < 4; ++d) {
        __syncthreads();
        const int r = tid >> 4, c = tid & 15;
        for (int J = 0; J + d < 4; ++J) {   // X = sum_{J <= K < I} A_IK T_KJ
            const int I = J + d;
            float x = 0.f;
            for (int K = J; K < I; ++K)
#pragma unroll 4
                for (int m = 0; m < 16; ++m) x += big[(16 * I + r) * 64 + 16 * K + m] * Tm[(16 * K + m) * 64 + 16 * J + c];
            xs[J * 256 + tid] = x;
        }
        __syncthreads();
        for (int J = 0; J + d < 4; ++J) {   // T_IJ = -D_I X
            const int I = J + d;
            float t = 0.f;
#pragma unroll 4
            for (int m = 0; m < 16; ++m) t += Tm[(16 * I + r) * 64 + 16 * I + m] * xs[J * 256 + m * 16 + c];
            Tm[(16 * I + r) * 64 + 16 * J + c] = -t;
        }
    }
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += kNT) {
        B[bT + e] = Tm[e];
        B[bTB + e] = Tm[e] * beta_s[e & 63];
    }
    bmm<false, false, 0, false, 128, 1, true>(B + bW, 128, B + bTB, 64, B + bKd, 128, 64, -1.f, 64, sm);   // -W = -TB Kd
    bmm<false, false, 0, false, 128, 1, true>(B + bUt, 128, B + bTB, 64, B + bV, 128, 64, 1.f, 64, sm);    // U~ = TB V
    bmm<false, true, 1, false, 64, 1, true>(B + bPm, 64, B + bQd, 128, B + bKi, 128, 128, 1.f, 64, sm);    // Pm
}

// Block -> (sequence, head, value tile) for the state passes, as in the
// forward scan: blocks go to the XCDs in turn (b % 8) and the eight tiles of
// one (sequence, head) item stay on one XCD, so they share its L2.  When the
// item count divides by 8 the items are dealt to the XCDs in turn, longest
// sequences first with a host-side plan (each block's time grows with its
// sequence's length); otherwise each XCD takes a contiguous eighth.
__device__ __forceinline__ void tile_of(const ChunkParams &c, int &n, int &h, int &tile) {
    const int b = blockIdx.x;
    if ((c.n_seqs * c.H) % 8 == 0) {
        const int slot = b / 8, item = (slot / kTilesV) * 8 + b % 8;
        tile = slot % kTilesV;
        h = item % c.H;
        n = c.plan_in_args ? (int)c.plan_order[item / c.H] : item / c.H;
    } else {
        const int total = c.n_seqs * c.H * kTilesV, per_xcd = total / 8;
        const int u = (b % 8) * per_xcd + b / 8;
        tile = u % kTilesV;
        h = (u / kTilesV) % c.H;
        n = u / (kTilesV * c.H);
    }
}

// The state passes run on fp32 MFMAs (16x16x4): lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16] of a 4-wide k step and holds D[4 (l / 16) + r][l % 16]
// in element r.  The k step (b, r) of a contraction over rows of a C-layout
// operand covers rows {16 b + 4 k' + r : k' = 0..3}, so element r of that
// operand's block b, as each lane holds it, is the B operand of step (b, r).
// The matching A operand is A[row][16 b + 4 (l / 16) + r]: one element of a
// 16-byte load when A is stored row-major, or, for a transposed operand
// (A = M^T with M row-major), M[16 b + 4 (l / 16) + r][row], which sixteen
// lanes fetch as 64 contiguous bytes.  A 128 x 16 state tile is eight such
// blocks (rows 16 mm + 4 (l / 16) + r, column l % 16).
//
// Four waves share each chunk step of one (sequence, head, 16-column tile).
// Wave w forms the 16-token block w of the chunk's U (or dU), a contraction
// over the 128 state rows, and the state rows of blocks 2w and 2w + 1, a
// contraction over the 64 tokens; U and the state go round through LDS so that
// every wave holds all of U and of the state as B operands of the next
// product.  Operands are fetched two chunks ahead into two register sets used
// in turn; each set is refilled right after its last use (past the last
// chunk the refill fetches the last chunk again, so every load is issued on
// every path).
// Chunk cid's workspace as a buffer resource: 32-bit offsets from a scalar
// base, so a load needs no 64-bit address arithmetic per lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const BwdParams &p, int cid, int h) {
    return buffer_rsrc(chunk_buf(p, cid, h), (uint32_t)(kBwdFloats * 4));
}
__device__ __forceinline__ f32x4 ldv(__amdgpu_buffer_rsrc_t rs, long idx) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(idx * 4), 0, 0));
}
__device__ __forceinline__ float lds1(__amdgpu_buffer_rsrc_t rs, long idx) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(idx * 4), 0, 0));
}
__device__ __forceinline__ void st1(float v, __amdgpu_buffer_rsrc_t rs, long idx) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, (uint32_t)(idx * 4), 0, 0);
}

// ---- forward state pass: S0 and U of every chunk ----------------------------
//   U = U~ - W S0,   S_L = Diag(e^{G_L}) S0 + (K e^{G_L - G})^T U
struct FwdOps {
    f32x4 W[8];      // -W[16 w + i][16 mm + 4 g ..]
    f32x4 Kt[2][4];  // Kg[16 m + 4 g + r][16 (2 w + j) + i]
    f32x4 gl[2];     // e^{G_L} of rows 16 (2 w + j) + 4 g ..
    f32x4 ut;        // U~[16 w + 4 g + r][col]
};
__global__ __launch_bounds__(kNT) void bwd_fwd_states_kernel(BwdParams p) {
    __shared__ f32x4 xU[4][64];
    __shared__ f32x4 xS[8][64];
    const ChunkParams &c = p.c;
    const int H = c.H, tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, i = l & 15;
    int n, h, tile;
    tile_of(c, n, h, tile);
    int c_begin, c_end, seq_start, seq_len;
    seq_chunks(c, n, c_begin, c_end, seq_start, seq_len);
    const int col = tile * kTileV + i;
    const long sb = ((long)n * H + h) * kHeadDim * kHeadDim;
    if (c_begin >= c_end) return;   // block-uniform
    f32x4 S[8];
#pragma unroll
    for (int mm = 0; mm < 8; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[mm][r] = c.s0 ? c.s0[sb + (16 * mm + 4 * g + r) * kHeadDim + col] : 0.f;
    const int nch = c_end - c_begin;
    auto rsrc = [&](int j) { return chunk_rsrc(p, c_begin + min(j, nch - 1), h); };
    auto fetch_w = [&](FwdOps &o, __amdgpu_buffer_rsrc_t rs) {
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) o.W[mm] = ldv(rs, bW + (16 * w + i) * 128 + 16 * mm + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) o.ut[r] = lds1(rs, bUt + (16 * w + 4 * g + r) * 128 + col);
    };
    auto fetch_k = [&](FwdOps &o, __amdgpu_buffer_rsrc_t rs) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) o.Kt[j][m][r] = lds1(rs, bKg + (16 * m + 4 * g + r) * 128 + 16 * (2 * w + j) + i);
            o.gl[j] = ldv(rs, bGL + 16 * (2 * w + j) + 4 * g);
        }
    };
    auto step = [&](int j, FwdOps &o) {
        const __amdgpu_buffer_rsrc_t rs = rsrc(j), rn = rsrc(j + 2);
        f32x4 u = o.ut;
#pragma unroll
        for (int mm = 0; mm < 8; ++mm)
#pragma unroll
            for (int r = 0; r < 4; ++r) u = mfma_f32(o.W[mm][r], S[mm][r], u);
        fetch_w(o, rn);
        xU[w][l] = u;
        f32x4 s2[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) s2[jj] = S[2 * w + jj] * o.gl[jj];
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 um = xU[m][l];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r) s2[jj] = mfma_f32(o.Kt[jj][m][r], um[r], s2[jj]);
        }
        fetch_k(o, rn);
        // this chunk's entry state and U, for the gradient kernel
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) st1(S[2 * w + jj][r], rs, bS0 + (16 * (2 * w + jj) + 4 * g + r) * 128 + col);
#pragma unroll
        for (int r = 0; r < 4; ++r) st1(u[r], rs, bU + (16 * w + 4 * g + r) * 128 + col);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) xS[2 * w + jj][l] = s2[jj];
        __syncthreads();
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) S[mm] = xS[mm][l];
    };
    FwdOps o0, o1;
    fetch_w(o0, rsrc(0));
    fetch_k(o0, rsrc(0));
    fetch_w(o1, rsrc(1));
    fetch_k(o1, rsrc(1));
    int j = 0;
    for (; j + 1 < nch; j += 2) {
        step(j, o0);
        step(j + 1, o1);
    }
    if (j < nch) step(j, o0);
}

// ---- backward state pass: dS_L and dU of every chunk; dS of the start --------
//   dU = Pm^T dO + Kg dS_L,   dS0 = Diag(e^{G_L}) dS_L + Qd^T dO - W^T dU
// (dO = scale dy (.) g comes from bwd_do_kernel.)
struct BwdOps {
    f32x4 Pt[4];     // Pm[16 m + 4 g + r][16 w + i]
    f32x4 K[8];      // Kg[16 w + i][16 mm + 4 g ..]
    f32x4 Qt[2][4];  // Qd[16 m + 4 g + r][16 (2 w + j) + i]
    f32x4 Wt[2][4];  // -W[16 m + 4 g + r][16 (2 w + j) + i]
    f32x4 gl[2];
    f32x4 dO[4];     // dO[16 m + 4 g + r][col]
};
__global__ __launch_bounds__(kNT) void bwd_bwd_states_kernel(BwdParams p) {
    __shared__ f32x4 xU[4][64];
    __shared__ f32x4 xS[8][64];
    const ChunkParams &c = p.c;
    const int H = c.H, tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, i = l & 15;
    int n, h, tile;
    tile_of(c, n, h, tile);
    int c_begin, c_end, seq_start, seq_len;
    seq_chunks(c, n, c_begin, c_end, seq_start, seq_len);
    const int col = tile * kTileV + i;
    const long sb = ((long)n * H + h) * kHeadDim * kHeadDim;
    f32x4 dS[8];
#pragma unroll
    for (int mm = 0; mm < 8; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dS[mm][r] = p.ds_final ? p.ds_final[sb + (16 * mm + 4 * g + r) * kHeadDim + col] : 0.f;
    const int nch = max(0, c_end - c_begin);
    // the j-th chunk from the end
    auto rsrc = [&](int j) { return chunk_rsrc(p, c_end - 1 - min(j, nch - 1), h); };
    auto fetch_pk = [&](BwdOps &o, __amdgpu_buffer_rsrc_t rs) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) o.Pt[m][r] = lds1(rs, bPm + (16 * m + 4 * g + r) * 64 + 16 * w + i);
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) o.K[mm] = ldv(rs, bKg + (16 * w + i) * 128 + 16 * mm + 4 * g);
    };
    auto fetch_qo = [&](BwdOps &o, __amdgpu_buffer_rsrc_t rs) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) o.Qt[j][m][r] = lds1(rs, bQd + (16 * m + 4 * g + r) * 128 + 16 * (2 * w + j) + i);
            o.gl[j] = ldv(rs, bGL + 16 * (2 * w + j) + 4 * g);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) o.dO[m][r] = lds1(rs, bdO + (16 * m + 4 * g + r) * 128 + col);
    };
    auto fetch_w = [&](BwdOps &o, __amdgpu_buffer_rsrc_t rs) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) o.Wt[j][m][r] = lds1(rs, bW + (16 * m + 4 * g + r) * 128 + 16 * (2 * w + j) + i);
    };
    auto step = [&](int j, BwdOps &o) {
        const __amdgpu_buffer_rsrc_t rs = rsrc(j), rn = rsrc(j + 2);
        f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) du = mfma_f32(o.Pt[m][r], o.dO[m][r], du);
#pragma unroll
        for (int mm = 0; mm < 8; ++mm)
#pragma unroll
            for (int r = 0; r < 4; ++r) du = mfma_f32(o.K[mm][r], dS[mm][r], du);
        fetch_pk(o, rn);
        xU[w][l] = du;
        f32x4 s2[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            s2[jj] = dS[2 * w + jj] * o.gl[jj];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) s2[jj] = mfma_f32(o.Qt[jj][m][r], o.dO[m][r], s2[jj]);
        }
        fetch_qo(o, rn);
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 um = xU[m][l];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r) s2[jj] = mfma_f32(o.Wt[jj][m][r], um[r], s2[jj]);
        }
        fetch_w(o, rn);
        // this chunk's end-state gradient and dU, for the gradient kernel
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                st1(dS[2 * w + jj][r], rs, bdSL + (16 * (2 * w + jj) + 4 * g + r) * 128 + col);
#pragma unroll
        for (int r = 0; r < 4; ++r) st1(du[r], rs, bdU + (16 * w + 4 * g + r) * 128 + col);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) xS[2 * w + jj][l] = s2[jj];
        __syncthreads();
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) dS[mm] = xS[mm][l];
    };
    if (nch > 0) {   // block-uniform
        BwdOps o0, o1;
        fetch_pk(o0, rsrc(0));
        fetch_qo(o0, rsrc(0));
        fetch_w(o0, rsrc(0));
        fetch_pk(o1, rsrc(1));
        fetch_qo(o1, rsrc(1));
        fetch_w(o1, rsrc(1));
        int j = 0;
        for (; j + 1 < nch; j += 2) {
            step(j, o0);
            step(j + 1, o1);
        }
        if (j < nch) step(j, o0);
    }
    if (p.ds0) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) p.ds0[sb + (16 * (2 * w + j) + 4 * g + r) * kHeadDim + col] = dS[2 * w + j][r];
    }
}

// ---- per-chunk gradients -------------------------------------------------------
// Element (nb, r) of a block product's accumulators is row 16 w + 4 (l / 16) + r,
// column 16 nb + l % 16 (wave w, lane l): the same for every 64-row product,
// so gradients that sum over several products stay in registers.
// Loads go through the chunk's buffer resource: 32-bit offsets with the
// column block in the immediate, not a 64-bit address per element.
template <int N>
__device__ __forceinline__ void load_acc_layout(f32x4 (&x)[N / 16], __amdgpu_buffer_rsrc_t rs, long m, int ld) {
    const int tid = threadIdx.x, row0 = 16 * (tid >> 6) + 4 * ((tid & 63) >> 4), lc = tid & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int nb = 0; nb < N / 16; ++nb) x[nb][r] = lds1(rs, m + (row0 + r) * ld + 16 * nb + lc);
}
// Makes the values exist here: otherwise the compiler sinks the arithmetic
// that produces dG past the remaining products, to its one use at the end,
// and keeps every operand of it alive (in scratch) until then.
__device__ __forceinline__ void materialize(f32x4 (&a)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(a[i]));
}
// Keeps the compiler from hoisting the next operand's loads above this point,
// so one 32-register operand (Kd, Ki, Qd or Kg, then G) is live at a time
// beside the accumulators and the dk, dG sums.
__device__ __forceinline__ void one_operand_at_a_time() { asm volatile("" ::: "memory"); }
// Sum over the 16 rows a wave holds of one column block (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float col_sum16(float v) {
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}

// One block per (chunk, head).  The four gradients that sum to dk and dlog
// alpha (dQd, dKg, dKd, dKi) are consumed where their product ends: dq goes out
// from the accumulators, dk and dG = dQd Qd + dKd Kd - dKi Ki - dKg Kg are
// summed in registers, and dG's reverse cumulative sum is taken from LDS.  dTB and the
// strict lower part of Kd Ki^T are consumed the same way (dT, dbeta); dPm,
// T^T dT and dA never leave LDS.  Only dW goes through the workspace.
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2))) void bwd_grads_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(16))) float sm[32 * 68 + 32 * 132];
    __shared__ float beta_s[64], kk_s[64], colq_s[4][128], colb_s[4][64];
    constexpr int kLdA = 68;   // row stride of dA (so the per-row dbeta sum is not one bank)
    // s_big: dPm and T^T dT while the products run, then dG [64][128]
    __shared__ __attribute__((aligned(16))) float s_big[2 * 64 * 64], s_dA[64 * kLdA];
    float *s_dPm = s_big, *s_X = s_big + 64 * 64;
    const ChunkParams &c = p.c;
    const int H = c.H, h = blockIdx.x % H, cid = blockIdx.x / H, tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lg = l >> 4, lc = l & 15;
    const int row0 = 16 * w + 4 * lg;
    const ChunkInfo ci = load_chunk(c, cid);
    const long tok0 = ci.start;
    const int len = ci.len;
    float *B = chunk_buf(p, cid, h);
    const __amdgpu_buffer_rsrc_t rs_B = chunk_rsrc(p, cid, h);
    if (tid < 64) beta_s[tid] = tid < len ? c.beta[(tok0 + tid) * H + h] : 0.f;
    // G is reloaded for each use (an L2 hit) rather than held across the
    // products, which keeps the kernel within two blocks' registers per CU
    f32x4 acc[8], X[8], dG[8], dk[8];
    auto zero = [](f32x4 *a, int n) {
        for (int i = 0; i < n; ++i) a[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // Outputs [T][H][128] go through buffer resources that end at the chunk's
    // last token: stores of rows past it are dropped, loads of them read 0,
    // with no branch.
    const uint32_t out_bytes = (uint32_t)len * H * kHeadDim * 4;
    auto out_rs = [&](float *o) { return buffer_rsrc(o + tok0 * H * kHeadDim, out_bytes); };
    auto out_off = [&](int r, int nb) { return (uint32_t)((((row0 + r) * H + h) * kHeadDim + 16 * nb + lc) * 4); };
    auto st_out = [&](__amdgpu_buffer_rsrc_t rs, int r, int nb, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, out_off(r, nb), 0, 0);
    };
    if (p.dgate) {   // O = Qd S0 + Pm U; dgate = dy scale O
        zero(acc, 8);
        bmm_acc<false, false, 128, 2, true>(acc, B + bQd, 128, B + bS0, 128, 128, sm);
        bmm_acc<false, false, 128, 2>(acc, B + bPm, 64, B + bU, 128, 64, sm);
        uint16_t dyv[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
                dyv[r][nb] = p.dy[((tok0 + min(row0 + r, len - 1)) * H + h) * kHeadDim + 16 * nb + lc];
        const __amdgpu_buffer_rsrc_t rs = out_rs(p.dgate);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) st_out(rs, r, nb, bf2f(dyv[r][nb]) * c.scale * acc[nb][r]);
    }
    bmm<false, true, 0, false, 128, 2, true>(B + bdW, 128, B + bdU, 128, B + bS0, 128, 128, -1.f, 64, sm);   // dW = -dU S0^T
    // dTB = dW Kd^T + dU V^T: dT = dTB diag(beta) into s_dA; dbeta gets sum_i dTB_ij T_ij
    {
        f32x4 a4[4], t4[4];
        zero(a4, 4);
        bmm_acc<false, true, 64, 2, true>(a4, B + bdW, 128, B + bKd, 128, 128, sm);
        bmm_acc<false, true, 64, 2, true>(a4, B + bdU, 128, B + bV, 128, 128, sm);
        load_acc_layout<64>(t4, rs_B, bT, 64);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            float cs = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s_dA[(row0 + r) * kLdA + 16 * nb + lc] = a4[nb][r] * beta_s[16 * nb + lc];
                cs += a4[nb][r] * t4[nb][r];
            }
            cs = col_sum16(cs);
            if (lg == 0) colb_s[w][16 * nb + lc] = cs;
        }
    }
    bmm<true, false, 0, false, 128>(p.dv + (tok0 * H + h) * kHeadDim, H * kHeadDim, B + bTB, 64, B + bdU, 128, 64,
                                    1.f, len, sm);                                                     // dV = TB^T dU
    bmm<true, false, 0, false, 64>(s_X, 64, B + bT, 64, s_dA, kLdA, 64, 1.f, 64, sm);          // T^T dT
    bmm<false, true, 2, false, 64>(s_dA, kLdA, s_X, 64, B + bT, 64, 64, -1.f, 64, sm);         // dA
    // tril(Kd Ki^T, -1): dbeta_i gets sum_m dA_im (Kd Ki^T)_im
    {
        f32x4 a4[4];
        zero(a4, 4);
        bmm_acc<false, true, 64, 2, true>(a4, B + bKd, 128, B + bKi, 128, 128, sm);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + r;
            float sr = 0.f;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int j = 16 * nb + lc;
                if (j < i) sr += a4[nb][r] * s_dA[i * kLdA + j];
            }
            sr += __shfl_xor(sr, 1, 64);
            sr += __shfl_xor(sr, 2, 64);
            sr += __shfl_xor(sr, 4, 64);
            sr += __shfl_xor(sr, 8, 64);
            if (lc == 0) kk_s[i] = sr;
        }
    }
    __syncthreads();
    {   // diag(beta) dA
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int e = tid + t * kNT;
            s_dA[(e >> 6) * kLdA + (e & 63)] *= beta_s[e >> 6];
        }
    }
    bmm<false, true, 1, false, 64, 2, true>(s_dPm, 64, B + bdO, 128, B + bU, 128, 128, 1.f, 64, sm);   // dPm = tril(dO U^T)
    // The four terms of dk and dG, summed in registers.
    // dKd = TB^T dW + (beta dA) Ki: dk = dKd e^G, dG = dKd Kd
    zero(acc, 8);
    bmm_acc<true, false, 128, 2>(acc, B + bTB, 64, B + bdW, 128, 64, sm);
    bmm_acc<false, false, 128, 2>(acc, s_dA, kLdA, B + bKi, 128, 64, sm);
    load_acc_layout<128>(X, rs_B, bKd, 128);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) dG[nb] = acc[nb] * X[nb];
    materialize(dG);
    one_operand_at_a_time();
    load_acc_layout<128>(X, rs_B, bG, 128);   // X now holds G
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dk[nb][r] = acc[nb][r] * __expf(X[nb][r]);
    materialize(dk);
    // dKi = (beta dA)^T Kd + dPm^T Qd: dk += dKi e^-G, dG -= dKi Ki
    zero(acc, 8);
    bmm_acc<true, false, 128, 2>(acc, s_dA, kLdA, B + bKd, 128, 64, sm);
    bmm_acc<true, false, 128, 2>(acc, s_dPm, 64, B + bQd, 128, 64, sm);
    load_acc_layout<128>(X, rs_B, bKi, 128);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dG[nb][r] -= acc[nb][r] * X[nb][r];
    materialize(dG);
    one_operand_at_a_time();
    load_acc_layout<128>(X, rs_B, bG, 128);   // X now holds G
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dk[nb][r] += acc[nb][r] * __expf(-X[nb][r]);
    materialize(dk);
    // dQd = dO S0^T + dPm Ki: dq = dQd e^G, dG += dQd Qd
    zero(acc, 8);
    bmm_acc<false, true, 128, 2>(acc, B + bdO, 128, B + bS0, 128, 128, sm);
    bmm_acc<false, false, 128, 2>(acc, s_dPm, 64, B + bKi, 128, 64, sm);
    load_acc_layout<128>(X, rs_B, bQd, 128);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) dG[nb] += acc[nb] * X[nb];
    materialize(dG);
    one_operand_at_a_time();
    load_acc_layout<128>(X, rs_B, bG, 128);   // X now holds G
    {
        const __amdgpu_buffer_rsrc_t rs = out_rs(p.dq);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) st_out(rs, r, nb, acc[nb][r] * __expf(X[nb][r]));
    }
    // dKg = U dS_L^T: dk += dKg e^{G_L - G}, dG -= dKg Kg, and its column sums for dG_L
    zero(acc, 8);
    bmm_acc<false, true, 128, 2>(acc, B + bU, 128, B + bdSL, 128, 128, sm);
    load_acc_layout<128>(X, rs_B, bKg, 128);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        float cs = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float e = acc[nb][r] * X[nb][r];
            dG[nb][r] -= e;
            cs += e;
        }
        cs = col_sum16(cs);
        if (lg == 0) colq_s[w][16 * nb + lc] = cs;
    }
    one_operand_at_a_time();
    load_acc_layout<128>(X, rs_B, bG, 128);   // X now holds G
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const float gl = lds1(rs_B, bG + 63 * 128 + 16 * nb + lc);
#pragma unroll
        for (int r = 0; r < 4; ++r) dk[nb][r] += acc[nb][r] * __expf(gl - X[nb][r]);
    }
    {
        const __amdgpu_buffer_rsrc_t rs = out_rs(p.dk);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) st_out(rs, r, nb, dk[nb][r]);
    }
    // From here on the lane's indices are recomputed from a fresh copy of the
    // thread index: kept from the start of the kernel, they would stay live
    // across every product (and spill).
    int t2 = tid;
    asm volatile("" : "+v"(t2));
    const int row0b = 16 * (t2 >> 6) + 4 * ((t2 & 63) >> 4), lcb = t2 & 15;
    // dG to LDS (s_big is free: the last product's staging ended with a barrier)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) s_big[(row0b + r) * 128 + 16 * nb + lcb] = dG[nb][r];
    float dgl = 0.f;
    if (t2 < 128) {   // dG_L = colsum(dKg Kg) + gL rowsum(S0 dS_L)
        const int ch = t2;
        float t = 0.f;
#pragma unroll 16
        for (int j = 0; j < 128; ++j) t += B[bS0 + ch * 128 + j] * B[bdSL + ch * 128 + j];
        dgl = ((colq_s[0][ch] + colq_s[1][ch]) + (colq_s[2][ch] + colq_s[3][ch])) + B[bGL + ch] * t;
    }
    __syncthreads();
    if (t2 < 128) {   // dlog alpha: reverse cumulative sum of dG, plus dG_L
        const int ch = t2;
        float run = dgl;
#pragma unroll 8
        for (int i = 63; i >= 0; --i) {
            run += s_big[i * 128 + ch];
            if (i < len) p.dla[((tok0 + i) * H + h) * kHeadDim + ch] = run;
        }
    }
    if (t2 < len)
        p.dbeta[(tok0 + t2) * H + h] = ((colb_s[0][t2] + colb_s[1][t2]) + (colb_s[2][t2] + colb_s[3][t2])) + kk_s[t2];
}

}  // namespace

size_t bwd_workspace_bytes(int H, int n_seqs, long n_chunks) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    return al(sizeof(int32_t) * (size_t)(n_seqs + 1)) + al(sizeof(ChunkInfo) * (size_t)n_chunks) +
           (size_t)n_chunks * (size_t)H * (size_t)kBwdFloats * sizeof(float);
}

void bwd_workspace_carve(void *ws, int H, int n_seqs, long n_chunks, BwdParams &p) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    (void)H;
    unsigned char *b = static_cast<unsigned char *>(ws);
    p.c.chunk_off = reinterpret_cast<int32_t *>(b);
    b += al(sizeof(int32_t) * (size_t)(n_seqs + 1));
    p.c.chunk_info = reinterpret_cast<ChunkInfo *>(b);
    b += al(sizeof(ChunkInfo) * (size_t)n_chunks);
    p.buf = reinterpret_cast<float *>(b);
}

hipError_t launch_chunk_backward(const BwdParams &p, hipStream_t s) {
    hipError_t e = launch_chunk_plan(p.c, s);
    if (e != hipSuccess) return e;
    const unsigned per_chunk = (unsigned)((long)p.c.n_chunks * p.c.H);
    const unsigned per_tile = (unsigned)(p.c.n_seqs * p.c.H * kTilesV);
    if (per_chunk > 0) {
        hipLaunchKernelGGL(bwd_do_kernel, dim3(per_chunk), dim3(kNT), 0, s, p);
        hipLaunchKernelGGL(bwd_prep_kernel, dim3(per_chunk), dim3(kNT), 0, s, p);
    }
    if (per_tile > 0) {
        hipLaunchKernelGGL(bwd_fwd_states_kernel, dim3(per_tile), dim3(kNT), 0, s, p);
        hipLaunchKernelGGL(bwd_bwd_states_kernel, dim3(per_tile), dim3(kNT), 0, s, p);
    }
    if (per_chunk > 0) hipLaunchKernelGGL(bwd_grads_kernel, dim3(per_chunk), dim3(kNT), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
