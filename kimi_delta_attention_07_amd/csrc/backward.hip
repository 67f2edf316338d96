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
// Four kernels, all fp32 on the VALU with LDS-staged tiles:
//   prep        chunks x heads: G, the decayed operands, A, T (forward
//               substitution, one column per thread), W, U~, Pm
//   fwd_states  sequences x heads x 8 value tiles: walks the chunks forward,
//               writes each chunk's S0 and U
//   bwd_states  the same grid backwards: dO, dS_L and dU per chunk, and the
//               gradient of the initial state
//   grads       chunks x heads: the per-chunk products above, then dq, dk, dv,
//               dlog alpha, dbeta and dgate
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
constexpr long bO = bdU + kM, bdPm = bO + kM, bdQd = bdPm + kSq, bdW = bdQd + kM, bdKg = bdW + kM;
constexpr long bdTB = bdKg + kM, bdKd = bdTB + kSq, bX = bdKd + kM, bdA = bX + kSq, bKK = bdA + kSq;
constexpr long bdKi = bKK + kSq;
constexpr long kBwdFloats = bdKi + kM;

__device__ __forceinline__ float *chunk_buf(const BwdParams &p, long cid, int h) {
    return p.buf + (cid * p.c.H + h) * kBwdFloats;
}

// Sequence n's chunk range [c_begin, c_end), sanitised like the forward scan's.
__device__ __forceinline__ void seq_chunks(const ChunkParams &c, int n, int &c_begin, int &c_end) {
    const int off0 = c.plan_in_args ? c.plan_off[n] : c.chunk_off[n];
    const int off1 = c.plan_in_args ? c.plan_off[n + 1] : c.chunk_off[n + 1];
    c_begin = max(0, off0);
    c_end = min(c.n_chunks, off1);
}

// C[0:64][0:N] (= or +=) alpha op(A)[64][K] op(B)[K][N], by all 256 threads.
//   op(A)[i][k] = TA ? A[k lda + i] : A[i lda + k]
//   op(B)[k][j] = TB ? B[j ldb + k] : B[k ldb + j]
// MASK 1 keeps entries j <= i, 2 keeps j < i (the rest are written as 0, or
// left alone when accumulating); rows >= mrows are not written.  N is 64 or
// 128, K a multiple of 16.  The operands may be in global memory (written
// earlier by this block: the barrier on entry orders them) or in LDS.
template <bool TA, bool TB, int MASK, bool ACC>
__device__ void bmm(float *C, int ldc, const float *A, int lda, const float *B, int ldb, int N, int K, float alpha,
                    int mrows, float *sm) {
    constexpr int LA = 65, LB = 129;   // padded LDS rows
    float *As = sm;                    // [16][LA]: As[kk][i]
    float *Bs = sm + 16 * LA;          // [16][LB]: Bs[kk][j]
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    float acc[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
    __syncthreads();
    for (int k0 = 0; k0 < K; k0 += 16) {
        for (int e = tid; e < 16 * 64; e += kNT) {
            int kk, i;
            if (TA) {
                kk = e >> 6;
                i = e & 63;
            } else {
                i = e >> 4;
                kk = e & 15;
            }
            As[kk * LA + i] = TA ? A[(long)(k0 + kk) * lda + i] : A[(long)i * lda + k0 + kk];
        }
        for (int e = tid; e < 16 * N; e += kNT) {
            int kk, j;
            if (TB) {
                j = e >> 4;
                kk = e & 15;
            } else {
                kk = e / N;
                j = e % N;
            }
            Bs[kk * LB + j] = TB ? B[(long)j * ldb + k0 + kk] : B[(long)(k0 + kk) * ldb + j];
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = As[kk * LA + 4 * ty + r];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                b[c] = Bs[kk * LB + 4 * tx + c];
                b[4 + c] = N > 64 ? Bs[kk * LB + 64 + 4 * tx + c] : 0.f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[r][c] += a[r] * b[c];
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 4 * ty + r;
        if (i >= mrows) continue;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            if (cc >= 4 && N <= 64) continue;
            const int j = cc < 4 ? 4 * tx + cc : 64 + 4 * tx + (cc - 4);
            const bool keep = MASK == 0 || (MASK == 1 ? j <= i : j < i);
            float *dst = C + (long)i * ldc + j;
            if (ACC) {
                if (keep) *dst += alpha * acc[r][cc];
            } else {
                *dst = keep ? alpha * acc[r][cc] : 0.f;
            }
        }
    }
}

// ---- prep: the chunk's WY quantities -----------------------------------------
__global__ __launch_bounds__(kNT) void bwd_prep_kernel(BwdParams p) {
    __shared__ float sm[16 * 65 + 16 * 129];
    __shared__ float big[64 * 128];   // G, then A (first half) and T (second half)
    __shared__ float beta_s[64];
    const ChunkParams &c = p.c;
    const int H = c.H, h = blockIdx.x % H, cid = blockIdx.x / H, tid = threadIdx.x;
    const ChunkInfo ci = load_chunk(c, cid);
    const long tok0 = ci.start;
    const int len = ci.len;
    float *B = chunk_buf(p, cid, h);
    if (tid < 128) {
        float run = 0.f;
        for (int i = 0; i < 64; ++i) {
            run += i < len ? bf2f(c.log_alpha[((tok0 + i) * H + h) * kHeadDim + tid]) : 0.f;
            big[i * 128 + tid] = run;
            B[bG + i * 128 + tid] = run;
        }
        B[bGL + tid] = expf(run);
    }
    if (tid < 64) beta_s[tid] = tid < len ? c.beta[(tok0 + tid) * H + h] : 0.f;
    __syncthreads();
    for (int e = tid; e < 64 * 128; e += kNT) {
        const int i = e >> 7, ch = e & 127;
        const long src = ((tok0 + i) * H + h) * kHeadDim + ch;
        const bool in = i < len;
        const float q = in ? bf2f(c.q[src]) : 0.f, k = in ? bf2f(c.k[src]) : 0.f, v = in ? bf2f(c.v[src]) : 0.f;
        const float g = big[e];
        const float eg = expf(g);
        B[bQd + e] = q * eg;
        B[bKd + e] = k * eg;
        B[bKi + e] = k * expf(-g);
        B[bKg + e] = k * expf(big[63 * 128 + ch] - g);
        B[bV + e] = v;
    }
    // A = tril(Kd Ki^T, -1), rows scaled by beta
    bmm<false, true, 2, false>(big, 64, B + bKd, 128, B + bKi, 128, 64, 128, 1.f, 64, sm);
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += kNT) big[e] *= beta_s[e >> 6];
    __syncthreads();
    // T = (I + A)^-1: thread j solves column j top to bottom
    float *Tm = big + 64 * 64;
    if (tid < 64) {
        const int j = tid;
        for (int i = 0; i < 64; ++i) {
            float t = i == j ? 1.f : 0.f;
            if (i > j) {
                float s = 0.f;
                for (int m = j; m < i; ++m) s += big[i * 64 + m] * Tm[m * 64 + j];
                t = -s;
            }
            Tm[i * 64 + j] = t;
        }
    }
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += kNT) {
        B[bT + e] = Tm[e];
        B[bTB + e] = Tm[e] * beta_s[e & 63];
    }
    bmm<false, false, 0, false>(B + bW, 128, B + bTB, 64, B + bKd, 128, 128, 64, 1.f, 64, sm);    // W = TB Kd
    bmm<false, false, 0, false>(B + bUt, 128, B + bTB, 64, B + bV, 128, 128, 64, 1.f, 64, sm);    // U~ = TB V
    bmm<false, true, 1, false>(B + bPm, 64, B + bQd, 128, B + bKi, 128, 64, 128, 1.f, 64, sm);    // Pm
}

// ---- forward state pass: S0 and U of every chunk ----------------------------
__global__ __launch_bounds__(kNT) void bwd_fwd_states_kernel(BwdParams p) {
    __shared__ float Ss[128 * 16], Us[64 * 16];
    const ChunkParams &c = p.c;
    const int H = c.H, tid = threadIdx.x;
    const int tile = blockIdx.x % kTilesV, h = (blockIdx.x / kTilesV) % H, n = blockIdx.x / (kTilesV * H);
    int c_begin, c_end;
    seq_chunks(c, n, c_begin, c_end);
    const int r = tid >> 1, cb = (tid & 1) * 8;    // state row, 8 of the tile's columns
    const int ui = tid >> 2, uc = (tid & 3) * 4;   // U row, 4 of the tile's columns
    const int col0 = tile * kTileV;
    float S[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        S[j] = c.s0 ? c.s0[(((long)n * H + h) * kHeadDim + r) * kHeadDim + col0 + cb + j] : 0.f;
    for (int cid = c_begin; cid < c_end; ++cid) {
        float *B = chunk_buf(p, cid, h);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            B[bS0 + r * 128 + col0 + cb + j] = S[j];
            Ss[r * 16 + cb + j] = S[j];
        }
        __syncthreads();
        float u[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) u[jj] = B[bUt + ui * 128 + col0 + uc + jj];
        for (int k = 0; k < 128; ++k) {
            const float w = B[bW + ui * 128 + k];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) u[jj] -= w * Ss[k * 16 + uc + jj];
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            B[bU + ui * 128 + col0 + uc + jj] = u[jj];
            Us[ui * 16 + uc + jj] = u[jj];
        }
        __syncthreads();
        const float gl = B[bGL + r];
#pragma unroll
        for (int j = 0; j < 8; ++j) S[j] *= gl;
        for (int i = 0; i < 64; ++i) {
            const float kg = B[bKg + i * 128 + r];
#pragma unroll
            for (int j = 0; j < 8; ++j) S[j] += kg * Us[i * 16 + cb + j];
        }
        __syncthreads();
    }
}

// ---- backward state pass: dO, dS_L, dU of every chunk; dS of the start -------
__global__ __launch_bounds__(kNT) void bwd_bwd_states_kernel(BwdParams p) {
    __shared__ float dSs[128 * 16], dOs[64 * 16], dUs[64 * 16];
    const ChunkParams &c = p.c;
    const int H = c.H, tid = threadIdx.x;
    const int tile = blockIdx.x % kTilesV, h = (blockIdx.x / kTilesV) % H, n = blockIdx.x / (kTilesV * H);
    int c_begin, c_end;
    seq_chunks(c, n, c_begin, c_end);
    const int r = tid >> 1, cb = (tid & 1) * 8;
    const int ui = tid >> 2, uc = (tid & 3) * 4;
    const int col0 = tile * kTileV;
    const long sidx = (((long)n * H + h) * kHeadDim + r) * kHeadDim + col0 + cb;
    float dS[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) dS[j] = p.ds_final ? p.ds_final[sidx + j] : 0.f;
    for (int cid = c_end - 1; cid >= c_begin; --cid) {
        const ChunkInfo ci = load_chunk(c, cid);
        float *B = chunk_buf(p, cid, h);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float d = 0.f;
            if (ui < ci.len) {
                const long e = ((long)(ci.start + ui) * H + h) * kHeadDim + col0 + uc + jj;
                d = c.scale * bf2f(p.dy[e]) * (c.gate ? bf2f(c.gate[e]) : 1.f);
            }
            B[bdO + ui * 128 + col0 + uc + jj] = d;
            dOs[ui * 16 + uc + jj] = d;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            B[bdSL + r * 128 + col0 + cb + j] = dS[j];
            dSs[r * 16 + cb + j] = dS[j];
        }
        __syncthreads();
        float du[4] = {0.f, 0.f, 0.f, 0.f};
        for (int m = 0; m < 64; ++m) {
            const float pm = B[bPm + m * 64 + ui];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) du[jj] += pm * dOs[m * 16 + uc + jj];
        }
        for (int k = 0; k < 128; ++k) {
            const float kg = B[bKg + ui * 128 + k];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) du[jj] += kg * dSs[k * 16 + uc + jj];
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            B[bdU + ui * 128 + col0 + uc + jj] = du[jj];
            dUs[ui * 16 + uc + jj] = du[jj];
        }
        __syncthreads();
        const float gl = B[bGL + r];
#pragma unroll
        for (int j = 0; j < 8; ++j) dS[j] *= gl;
        for (int i = 0; i < 64; ++i) {
            const float qd = B[bQd + i * 128 + r], w = B[bW + i * 128 + r];
#pragma unroll
            for (int j = 0; j < 8; ++j) dS[j] += qd * dOs[i * 16 + cb + j] - w * dUs[i * 16 + cb + j];
        }
        __syncthreads();
    }
    if (p.ds0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) p.ds0[sidx + j] = dS[j];
    }
}

// ---- per-chunk gradients -------------------------------------------------------
__global__ __launch_bounds__(kNT) void bwd_grads_kernel(BwdParams p) {
    __shared__ float sm[16 * 65 + 16 * 129];
    __shared__ float beta_s[64], dbeta_s[64], dGL_s[128];
    const ChunkParams &c = p.c;
    const int H = c.H, h = blockIdx.x % H, cid = blockIdx.x / H, tid = threadIdx.x;
    const ChunkInfo ci = load_chunk(c, cid);
    const long tok0 = ci.start;
    const int len = ci.len;
    float *B = chunk_buf(p, cid, h);
    if (tid < 64) beta_s[tid] = tid < len ? c.beta[(tok0 + tid) * H + h] : 0.f;
    if (p.dgate) {   // O = Qd S0 + Pm U
        bmm<false, false, 0, false>(B + bO, 128, B + bQd, 128, B + bS0, 128, 128, 128, 1.f, 64, sm);
        bmm<false, false, 0, true>(B + bO, 128, B + bPm, 64, B + bU, 128, 128, 64, 1.f, 64, sm);
    }
    bmm<false, true, 1, false>(B + bdPm, 64, B + bdO, 128, B + bU, 128, 64, 128, 1.f, 64, sm);       // tril(dO U^T)
    bmm<false, true, 0, false>(B + bdQd, 128, B + bdO, 128, B + bS0, 128, 128, 128, 1.f, 64, sm);    // dO S0^T
    bmm<false, false, 0, true>(B + bdQd, 128, B + bdPm, 64, B + bKi, 128, 128, 64, 1.f, 64, sm);     //  + dPm Ki
    bmm<false, true, 0, false>(B + bdW, 128, B + bdU, 128, B + bS0, 128, 128, 128, -1.f, 64, sm);    // -dU S0^T
    bmm<false, true, 0, false>(B + bdKg, 128, B + bU, 128, B + bdSL, 128, 128, 128, 1.f, 64, sm);    // U dS_L^T
    bmm<false, true, 0, false>(B + bdTB, 64, B + bdW, 128, B + bKd, 128, 64, 128, 1.f, 64, sm);      // dW Kd^T
    bmm<false, true, 0, true>(B + bdTB, 64, B + bdU, 128, B + bV, 128, 64, 128, 1.f, 64, sm);        //  + dU V^T
    bmm<true, false, 0, false>(B + bdKd, 128, B + bTB, 64, B + bdW, 128, 128, 64, 1.f, 64, sm);      // TB^T dW
    bmm<true, false, 0, false>(p.dv + (tok0 * H + h) * kHeadDim, H * kHeadDim, B + bTB, 64, B + bdU, 128, 128, 64,
                               1.f, len, sm);                                                       // dV = TB^T dU
    __syncthreads();
    // dT = dTB diag(beta) (held in the dA slot); dbeta from TB = T diag(beta)
    for (int e = tid; e < 64 * 64; e += kNT) B[bdA + e] = B[bdTB + e] * beta_s[e & 63];
    if (tid < 64) {
        float s = 0.f;
        for (int i = 0; i < 64; ++i) s += B[bdTB + i * 64 + tid] * B[bT + i * 64 + tid];
        dbeta_s[tid] = s;
    }
    bmm<true, false, 0, false>(B + bX, 64, B + bT, 64, B + bdA, 64, 64, 64, 1.f, 64, sm);            // T^T dT
    bmm<false, true, 2, false>(B + bdA, 64, B + bX, 64, B + bT, 64, 64, 64, -1.f, 64, sm);           // dA
    bmm<false, true, 2, false>(B + bKK, 64, B + bKd, 128, B + bKi, 128, 64, 128, 1.f, 64, sm);       // tril(Kd Ki^T, -1)
    __syncthreads();
    if (tid < 64) {
        float s = 0.f;
        for (int m = 0; m < 64; ++m) s += B[bdA + tid * 64 + m] * B[bKK + tid * 64 + m];
        dbeta_s[tid] += s;
    }
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += kNT) B[bdA + e] *= beta_s[e >> 6];                          // diag(beta) dA
    bmm<false, false, 0, true>(B + bdKd, 128, B + bdA, 64, B + bKi, 128, 128, 64, 1.f, 64, sm);      // += (beta dA) Ki
    bmm<true, false, 0, false>(B + bdKi, 128, B + bdA, 64, B + bKd, 128, 128, 64, 1.f, 64, sm);      // (beta dA)^T Kd
    bmm<true, false, 0, true>(B + bdKi, 128, B + bdPm, 64, B + bQd, 128, 128, 64, 1.f, 64, sm);      //  + dPm^T Qd
    __syncthreads();
    if (tid < 128) {
        const int ch = tid;
        float s = 0.f, t = 0.f;
        for (int i = 0; i < 64; ++i) s += B[bdKg + i * 128 + ch] * B[bKg + i * 128 + ch];
        for (int j = 0; j < 128; ++j) t += B[bS0 + ch * 128 + j] * B[bdSL + ch * 128 + j];
        dGL_s[ch] = s + B[bGL + ch] * t;
    }
    __syncthreads();
    if (tid < 128) {   // dlog alpha: reverse cumulative sum of dG, plus dG_L
        const int ch = tid;
        float run = dGL_s[ch];
        for (int i = 63; i >= 0; --i) {
            const long e = i * 128 + ch;
            run += B[bdQd + e] * B[bQd + e] + B[bdKd + e] * B[bKd + e] - B[bdKi + e] * B[bKi + e] -
                   B[bdKg + e] * B[bKg + e];
            if (i < len) p.dla[((tok0 + i) * H + h) * kHeadDim + ch] = run;
        }
    }
    for (int e = tid; e < 64 * 128; e += kNT) {
        const int i = e >> 7, ch = e & 127;
        if (i >= len) continue;
        const long o = ((tok0 + i) * H + h) * kHeadDim + ch;
        const float g = B[bG + e], eg = expf(g);
        p.dq[o] = B[bdQd + e] * eg;
        p.dk[o] = B[bdKd + e] * eg + B[bdKi + e] * expf(-g) + B[bdKg + e] * expf(B[bG + 63 * 128 + ch] - g);
        if (p.dgate) p.dgate[o] = bf2f(p.dy[o]) * c.scale * B[bO + e];
    }
    if (tid < len) p.dbeta[(tok0 + tid) * H + h] = dbeta_s[tid];
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
    if (per_chunk > 0) hipLaunchKernelGGL(bwd_prep_kernel, dim3(per_chunk), dim3(kNT), 0, s, p);
    if (per_tile > 0) {
        hipLaunchKernelGGL(bwd_fwd_states_kernel, dim3(per_tile), dim3(kNT), 0, s, p);
        hipLaunchKernelGGL(bwd_bwd_states_kernel, dim3(per_tile), dim3(kNT), 0, s, p);
    }
    if (per_chunk > 0) hipLaunchKernelGGL(bwd_grads_kernel, dim3(per_chunk), dim3(kNT), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
