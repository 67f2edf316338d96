// Chunked KDA prefill for gfx950 (head dim 128, 64-token chunks, bf16 inputs,
// fp32 state).
//
// Within a chunk with entry state S and cumulative log decay
// G_i = sum_{s<=i} log alpha_s (a 128-vector per token), the recurrence
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
// unrolls to the WY/UT form
//     A = tril(beta_i sum_c k_ic k_jc e^{G_ic - G_jc}, -1),  T = (I + A)^-1
//     W = T beta (K e^G),   U~ = T beta V,   U = U~ - W S
//     P = tril(sum_c q_ic k_jc e^{G_ic - G_jc})
//     O = (Q e^G) S + P U,   S_next = Diag(e^{G_L}) S + (K e^{G_L - G})^T U
// which equals the token loop exactly in exact arithmetic.  The decay factor
// e^{G_i - G_j} is split as e^{G_i} e^{-G_j} with G counted from the chunk
// start, so every product is an MFMA contraction over channels.
//
// Two stages:
//  prepare  grid (chunks, heads), 256 threads.  Everything that does not
//           depend on S: G, the exponentials, A and P (bf16 MFMA, fp32 acc),
//           the 64x64 unit-lower-triangular inverse (fp32, LDS, blocked by
//           16), W and U~.
//           Results go to the workspace as ready-made MFMA fragments.
//  scan     grid (sequences x heads x 8 value tiles), one wave each.  Walks a
//           sequence's chunks in order; the 128 x 16 fp32 state tile stays in
//           the wave's accumulator registers the whole time.  Per chunk:
//           54 MFMAs (U, O, the state update) and one pass over the chunk's
//           fragments.  Blocks are numbered so that the eight tiles of one
//           (sequence, head) land on the same XCD and share its L2.
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Fragment convention (checked on the
// device): lane l holds row (l % 16) of A / column (l % 16) of B with k
// elements 8 (l / 16) + e, and rows 4 (l / 16) + r, column (l % 16) of C.
// Any consistent renumbering of k between A and B leaves the product
// unchanged; the scan uses k order {4g..4g+3, 16+4g..16+4g+3} inside each
// 32-wide k step so that the state and U accumulators (C layout) become the
// B operand of the next product with no data movement.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

// ---------------------------------------------------------------------------
// plan: chunk table from cu_seqlens (one workgroup, scans 256 sequences a pass)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(const int32_t *cu, int n_seqs, int n_chunks,
                                                   int32_t *chunk_off, ChunkInfo *info) {
    __shared__ int32_t buf[256];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < n_seqs; base += 256) {
        const int n = base + tid;
        int cnt = 0, start = 0, len = 0;
        if (n < n_seqs) {
            start = cu[n];
            len = cu[n + 1] - start;
            cnt = (len + kChunk - 1) / kChunk;
        }
        buf[tid] = cnt;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int v = tid >= o ? buf[tid - o] : 0;
            __syncthreads();
            buf[tid] += v;
            __syncthreads();
        }
        const int excl = carry + buf[tid] - cnt;
        if (n < n_seqs) {
            chunk_off[n] = excl;
            for (int c = 0; c < cnt && excl + c < n_chunks; ++c) {
                ChunkInfo ci;
                ci.start = start + kChunk * c;
                ci.len = min(kChunk, len - kChunk * c);
                info[excl + c] = ci;
            }
        }
        __syncthreads();
        if (tid == 255) carry += buf[255];
        __syncthreads();
    }
    if (tid == 0) chunk_off[n_seqs] = carry;
}

// A chunk record as the kernels may use it: the table is built on the device
// from cu_seqlens_dev while grids are sized from the host copy; should the two
// ever disagree, out-of-range entries become empty chunks instead of stray
// memory accesses.
__device__ __forceinline__ ChunkInfo load_chunk(const ChunkParams &p, int cid) {
    ChunkInfo ci = p.chunk_info[cid];
    if (ci.start < 0 || ci.len < 0 || ci.len > kChunk || ci.start > p.T - ci.len) {
        ci.start = 0;
        ci.len = 0;
    }
    return ci;
}

// ---------------------------------------------------------------------------
// prepare
// ---------------------------------------------------------------------------
// LDS plan (bytes).  Region R holds, in phases 1-2, Kd = K e^G, Ki = K e^-G,
// Qg = Q e^G row-major [64][136] bf16; in phases 3-5 the transposed copies
// (beta K e^G)^T, (beta V)^T, (K e^{G_L-G})^T as [128][72] bf16.
constexpr int kRowA = 136;                  // bf16 row stride of [64][128] tiles
constexpr int kRowT = 72;                   // bf16 row stride of [128][64] tiles
constexpr int kOffKd = 0;
constexpr int kOffKi = kOffKd + 64 * kRowA * 2;
constexpr int kOffQs = kOffKi + 64 * kRowA * 2;
constexpr int kOffKdT = 0;
constexpr int kOffVT = kOffKdT + 128 * kRowT * 2;
constexpr int kOffKgT = kOffVT + 128 * kRowT * 2;
constexpr int kRegionR = kOffKgT + 128 * kRowT * 2;      // 55,296 >= 3 * 17,408
constexpr int kOffA = kRegionR;                           // fp32 [64][64]
constexpr int kOffTm = kOffA + 64 * 64 * 4;               // bf16 [64][72]
constexpr int kOffBeta = kOffTm + 64 * kRowT * 2;         // fp32 [64]
constexpr int kLdsPrepare = kOffBeta + 64 * 4;            // 81,152 B: two workgroups per CU
static_assert(3 * 64 * kRowA * 2 <= kRegionR, "phase-1 tiles must fit region R");
static_assert(4 * 128 * 4 <= 64 * kRowT * 2, "cumsum totals alias the T tile");
static_assert(4 * 16 * 16 * 4 <= 64 * kRowT * 2, "inverse scratch aliases the T tile");

__device__ __forceinline__ bf16x8 lds_frag(const unsigned char *lds, int off_bytes) {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(lds + off_bytes));
}

__global__ __launch_bounds__(256, 2) void prepare_kernel(ChunkParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsPrepare];
    const int cid = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int H = p.H;
    const ChunkInfo ci = load_chunk(p, cid);
    const long tok0 = ci.start;
    const int len = ci.len;
    unsigned char *rec = p.records + ((long)cid * H + h) * kChunkRecordBytes;

    float *A = reinterpret_cast<float *>(lds + kOffA);
    uint16_t *Tm = reinterpret_cast<uint16_t *>(lds + kOffTm);
    float *beta_s = reinterpret_cast<float *>(lds + kOffBeta);
    float *tot = reinterpret_cast<float *>(lds + kOffTm);   // [4][128], dead before T is written

    if (tid < 64) beta_s[tid] = tid < len ? p.beta[(tok0 + tid) * H + h] : 0.0f;

    // ---- phase 1: cumulative log decay and decayed operands ----------------
    // wave w: tokens 16w..16w+15; lane l: channels 2l, 2l+1
    float2 G[16];
    {
        float2 run = make_float2(0.f, 0.f);
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
            const int tk = 16 * w + ii;
            float2 la = make_float2(0.f, 0.f);
            if (tk < len) {
                const uint32_t u = *reinterpret_cast<const uint32_t *>(
                    p.log_alpha + ((tok0 + tk) * H + h) * kHeadDim + 2 * l);
                la = make_float2(lo_bf(u), hi_bf(u));
            }
            run.x += la.x;
            run.y += la.y;
            G[ii] = run;
        }
        tot[w * 128 + 2 * l] = run.x;
        tot[w * 128 + 2 * l + 1] = run.y;
    }
    __syncthreads();
    float2 GL = make_float2(0.f, 0.f), off = make_float2(0.f, 0.f);
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
        const float a = tot[ww * 128 + 2 * l], b = tot[ww * 128 + 2 * l + 1];
        if (ww < w) {
            off.x += a;
            off.y += b;
        }
        GL.x += a;
        GL.y += b;
    }
    if (w == 0) {
        float2 gl = make_float2(__expf(GL.x), __expf(GL.y));
        *reinterpret_cast<float2 *>(rec + kOffGL + 8 * l) = gl;
    }
    // Operands of phase 3, packed to bf16 now so few registers stay live:
    // pk[0] = beta k^ e^G, pk[1] = beta v^, pk[2] = k^ e^{G_L - G}; per channel
    // e (0, 1) the 16 tokens of this wave, two per 32-bit word.
    uint32_t pk[3][2][8];
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
        const int tk = 16 * w + ii;
        const float gx = G[ii].x + off.x, gy = G[ii].y + off.y;
        float2 q2 = make_float2(0.f, 0.f), k2 = q2, v2 = q2;
        if (tk < len) {
            const long o = ((tok0 + tk) * H + h) * kHeadDim + 2 * l;
            const uint32_t uq = *reinterpret_cast<const uint32_t *>(p.q + o);
            const uint32_t uk = *reinterpret_cast<const uint32_t *>(p.k + o);
            const uint32_t uv = *reinterpret_cast<const uint32_t *>(p.v + o);
            q2 = make_float2(lo_bf(uq), hi_bf(uq));
            k2 = make_float2(lo_bf(uk), hi_bf(uk));
            v2 = make_float2(lo_bf(uv), hi_bf(uv));
        }
        const float ex = __expf(gx), ey = __expf(gy);
        const float ix = __expf(-gx), iy = __expf(-gy);
        const float hx = __expf(GL.x - gx), hy = __expf(GL.y - gy);
        const float bt = beta_s[tk];
        const int e = tk * kRowA + 2 * l;
        reinterpret_cast<uint32_t *>(lds + kOffKd)[e / 2] = pack_bf2(k2.x * ex, k2.y * ey);
        reinterpret_cast<uint32_t *>(lds + kOffKi)[e / 2] = pack_bf2(k2.x * ix, k2.y * iy);
        reinterpret_cast<uint32_t *>(lds + kOffQs)[e / 2] = pack_bf2(q2.x * ex, q2.y * ey);
        const uint32_t vals[3][2] = {{f2bf(bt * k2.x * ex), f2bf(bt * k2.y * ey)},
                                     {f2bf(bt * v2.x), f2bf(bt * v2.y)},
                                     {f2bf(k2.x * hx), f2bf(k2.y * hy)}};
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                if (ii % 2 == 0) pk[a][c][ii / 2] = vals[a][c];
                else pk[a][c][ii / 2] |= vals[a][c] << 16;
            }
    }
    __syncthreads();

    // ---- phase 2: A (row block I = w) and P^T (column block I = 3 - w) -----
    {
        const int I = w;
        for (int J = 0; J <= I; ++J) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 a = lds_frag(lds, kOffKd + ((16 * I + c16) * kRowA + 32 * s + 8 * g) * 2);
                const bf16x8 b = lds_frag(lds, kOffKi + ((16 * J + c16) * kRowA + 32 * s + 8 * g) * 2);
                acc = mfma16(a, b, acc);
            }
            const int j = 16 * J + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * g + r;
                if (j < i) A[i * 64 + j] = beta_s[i] * acc[r];
            }
        }
    }
    {
        const int I = 3 - w;
        f32x4 blk[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (J <= I) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 a = lds_frag(lds, kOffKi + ((16 * J + c16) * kRowA + 32 * s + 8 * g) * 2);
                    const bf16x8 b = lds_frag(lds, kOffQs + ((16 * I + c16) * kRowA + 32 * s + 8 * g) * 2);
                    acc = mfma16(a, b, acc);
                }
                const int i = 16 * I + c16;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * J + 4 * g + r > i) acc[r] = 0.f;
            }
            blk[J] = acc;
        }
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const bf16x8 f = pack8(blk[2 * sp], blk[2 * sp + 1]);
            *reinterpret_cast<bf16x8 *>(rec + kOffP + ((I * 2 + sp) * 64 + l) * 16) = f;
        }
    }
    // Qg fragments: token tile m = w, channel k-steps s = 0..3
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int base = kOffQs + ((16 * w + c16) * kRowA + 32 * s + 4 * g) * 2;
        u32x4 f;
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(lds + base);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(lds + base + 32);
        f[0] = lo[0];
        f[1] = lo[1];
        f[2] = hi[0];
        f[3] = hi[1];
        *reinterpret_cast<u32x4 *>(rec + kOffQg + ((w * 4 + s) * 64 + l) * 16) = f;
    }
    __syncthreads();

    // ---- phase 3: transposed, beta-scaled copies into region R -------------
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int rowoff = ((2 * l + e) * kRowT + 16 * w) * 2;
        const int offs[3] = {kOffKdT, kOffVT, kOffKgT};
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            u32x4 lo, hi;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                lo[q4] = pk[a][e][q4];
                hi[q4] = pk[a][e][4 + q4];
            }
            *reinterpret_cast<u32x4 *>(lds + offs[a] + rowoff) = lo;
            *reinterpret_cast<u32x4 *>(lds + offs[a] + rowoff + 16) = hi;
        }
    }
    __syncthreads();

    // ---- phase 4: Kg fragments, then T = (I + A)^-1 in fp32 ------------------
    for (int f = w; f < 16; f += 4) {
        const int mm = f >> 1, sp = f & 1;
        const int base = kOffKgT + ((16 * mm + c16) * kRowT + 32 * sp + 4 * g) * 2;
        u32x4 v;
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(lds + base);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(lds + base + 32);
        v[0] = lo[0];
        v[1] = lo[1];
        v[2] = hi[0];
        v[3] = hi[1];
        *reinterpret_cast<u32x4 *>(rec + kOffKg + ((mm * 2 + sp) * 64 + l) * 16) = v;
    }
    // Blocked inverse of the unit-lower-triangular I + A (A strictly lower,
    // only its strictly-lower entries are valid), overwriting A with T:
    //   T_II = (I + A_II)^-1 by forward substitution (wave I, lane = column),
    //   T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ for I > J (wave J, row block I).
    {
        float *Ad = A + (16 * w) * 64 + 16 * w;
        if (l < 16) {
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = (i == l) ? 1.0f : 0.0f;
#pragma unroll
                for (int k = 0; k < i; ++k) acc -= Ad[i * 64 + k] * x[k];
                x[i] = acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) Ad[i * 64 + l] = x[i];
        }
    }
    __syncthreads();
    float *Msc = reinterpret_cast<float *>(lds + kOffTm);   // [4][16][16] scratch, dead T tile
    for (int I = 1; I < 4; ++I) {
        f32x4 M = {0.f, 0.f, 0.f, 0.f};
        if (w < I) {
            for (int K = w; K < I; ++K) {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const float t_kc = A[(16 * K + k) * 64 + 16 * w + c16];
#pragma unroll
                    for (int r = 0; r < 4; ++r) M[r] += A[(16 * I + 4 * g + r) * 64 + 16 * K + k] * t_kc;
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) Msc[(w * 16 + 4 * g + r) * 16 + c16] = M[r];
        }
        __syncthreads();   // row block I of A fully read; M visible
        if (w < I) {
            f32x4 Tn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float mv = Msc[(w * 16 + m) * 16 + c16];
#pragma unroll
                for (int r = 0; r < 4; ++r) Tn[r] -= A[(16 * I + 4 * g + r) * 64 + 16 * I + m] * mv;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) A[(16 * I + 4 * g + r) * 64 + 16 * w + c16] = Tn[r];
        }
        __syncthreads();
    }
    // T to bf16, zero above the block diagonal
    for (int idx = tid; idx < 64 * 64; idx += 256) {
        const int i = idx >> 6, j = idx & 63;
        Tm[i * kRowT + j] = f2bf((j >> 4) <= (i >> 4) ? A[idx] : 0.0f);
    }
    __syncthreads();

    // ---- phase 5: W^T = (beta K e^G)^T T^T and U~ = T (beta V) --------------
    {
        // W: channel tiles 2w, 2w+1; token tiles I = 0..3; k steps s <= I/2
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
            for (int s = 0; s <= I / 2; ++s) {
                const bf16x8 b = lds_frag(lds, kOffTm + ((16 * I + c16) * kRowT + 32 * s + 8 * g) * 2);
                const bf16x8 x0 = lds_frag(lds, kOffKdT + ((32 * w + c16) * kRowT + 32 * s + 8 * g) * 2);
                const bf16x8 x1 = lds_frag(lds, kOffKdT + ((32 * w + 16 + c16) * kRowT + 32 * s + 8 * g) * 2);
                a0 = mfma16(x0, b, a0);
                a1 = mfma16(x1, b, a1);
            }
            *reinterpret_cast<bf16x8 *>(rec + kOffW + ((I * 4 + w) * 64 + l) * 16) = pack8(-a0, -a1);
        }
        // U~: value tiles 2w, 2w+1; token tiles m = 0..3; k steps s <= m/2
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
            for (int s = 0; s <= m / 2; ++s) {
                const bf16x8 a = lds_frag(lds, kOffTm + ((16 * m + c16) * kRowT + 32 * s + 8 * g) * 2);
                const bf16x8 b0 = lds_frag(lds, kOffVT + ((32 * w + c16) * kRowT + 32 * s + 8 * g) * 2);
                const bf16x8 b1 = lds_frag(lds, kOffVT + ((32 * w + 16 + c16) * kRowT + 32 * s + 8 * g) * 2);
                a0 = mfma16(a, b0, a0);
                a1 = mfma16(a, b1, a1);
            }
            u32x2 o0, o1;
            o0[0] = pack_bf2(a0[0], a0[1]);
            o0[1] = pack_bf2(a0[2], a0[3]);
            o1[0] = pack_bf2(a1[0], a1[1]);
            o1[1] = pack_bf2(a1[2], a1[3]);
            *reinterpret_cast<u32x2 *>(rec + kOffU + (((2 * w) * 4 + m) * 64 + l) * 8) = o0;
            *reinterpret_cast<u32x2 *>(rec + kOffU + (((2 * w + 1) * 4 + m) * 64 + l) * 8) = o1;
        }
    }
}

// ---------------------------------------------------------------------------
// scan
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 rec_frag(const unsigned char *rec, size_t off, int idx, int l) {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(rec + off + ((size_t)idx * 64 + l) * 16));
}

__global__ __launch_bounds__(64) void scan_kernel(ChunkParams p) {
    const int H = p.H;
    const int total = p.n_seqs * H * kTilesV;   // a multiple of 8
    const int per_xcd = total / 8;
    const int b = blockIdx.x;
    const int u = (b % 8) * per_xcd + b / 8;    // consecutive u share an XCD
    const int tile = u % kTilesV;
    const int h = (u / kTilesV) % H;
    const int n = u / (kTilesV * H);
    const int l = threadIdx.x, g = l >> 4, c16 = l & 15;
    const int col = tile * kTileV + c16;

    // state tile S[128][16] as 8 C-layout tiles: rows 16 mm + 4 g + r
    f32x4 S[8];
    const long sbase = ((long)n * H + h) * kHeadDim * kHeadDim;
#pragma unroll
    for (int mm = 0; mm < 8; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[mm][r] = p.s0 ? p.s0[sbase + (16 * mm + 4 * g + r) * kHeadDim + col] : 0.0f;

    const int c_begin = max(0, p.chunk_off[n]), c_end = min(p.n_chunks, p.chunk_off[n + 1]);
    for (int cid = c_begin; cid < c_end; ++cid) {
        const unsigned char *rec = p.records + ((long)cid * H + h) * kChunkRecordBytes;
        const ChunkInfo ci = load_chunk(p, cid);

        bf16x8 Sb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) Sb[s] = pack8(S[2 * s], S[2 * s + 1]);

        // U = U~ + (-W) S
        f32x4 U[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const u32x2 uw = *reinterpret_cast<const u32x2 *>(rec + kOffU + ((tile * 4 + m) * 64 + l) * 8);
            U[m][0] = lo_bf(uw[0]);
            U[m][1] = hi_bf(uw[0]);
            U[m][2] = lo_bf(uw[1]);
            U[m][3] = hi_bf(uw[1]);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int s = 0; s < 4; ++s) U[m] = mfma16(rec_frag(rec, kOffW, m * 4 + s, l), Sb[s], U[m]);

        // O = (Q e^G) S + P U
        f32x4 O[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            O[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) O[m] = mfma16(rec_frag(rec, kOffQg, m * 4 + s, l), Sb[s], O[m]);
        }
        bf16x8 Ub[2];
        Ub[0] = pack8(U[0], U[1]);
        Ub[1] = pack8(U[2], U[3]);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int sp = 0; sp <= m / 2; ++sp) O[m] = mfma16(rec_frag(rec, kOffP, m * 2 + sp, l), Ub[sp], O[m]);

        // S <- Diag(e^{G_L}) S + (K e^{G_L - G})^T U
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) {
            const f32x4 gl = *reinterpret_cast<const f32x4 *>(rec + kOffGL + (16 * mm + 4 * g) * 4);
            S[mm] *= gl;
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) S[mm] = mfma16(rec_frag(rec, kOffKg, mm * 2 + sp, l), Ub[sp], S[mm]);
        }

        // y = scale O (.) gate
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tk = 16 * m + 4 * g + r;
                if (tk < ci.len) {
                    const long o = ((long)(ci.start + tk) * H + h) * kHeadDim + col;
                    float y = p.scale * O[m][r];
                    if (p.gate) y *= bf2f(p.gate[o]);
                    p.out[o] = f2bf(y);
                }
            }
    }
    if (p.s_final) {
#pragma unroll
        for (int mm = 0; mm < 8; ++mm)
#pragma unroll
            for (int r = 0; r < 4; ++r) p.s_final[sbase + (16 * mm + 4 * g + r) * kHeadDim + col] = S[mm][r];
    }
}

}  // namespace

size_t chunk_workspace_bytes(int H, int n_seqs, long n_chunks) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    return al(sizeof(int32_t) * (size_t)(n_seqs + 1)) + al(sizeof(ChunkInfo) * (size_t)n_chunks) +
           (size_t)n_chunks * (size_t)H * kChunkRecordBytes;
}

void chunk_workspace_carve(void *ws, int H, int n_seqs, long n_chunks, ChunkParams &p) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    unsigned char *b = static_cast<unsigned char *>(ws);
    p.chunk_off = reinterpret_cast<int32_t *>(b);
    b += al(sizeof(int32_t) * (size_t)(n_seqs + 1));
    p.chunk_info = reinterpret_cast<ChunkInfo *>(b);
    b += al(sizeof(ChunkInfo) * (size_t)n_chunks);
    p.records = b;
    (void)H;
}

hipError_t launch_chunk_prepare(const ChunkParams &p, hipStream_t s) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p.cu, p.n_seqs, p.n_chunks, p.chunk_off,
                       p.chunk_info);
    if (p.n_chunks > 0)
        hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)p.n_chunks, (unsigned)p.H), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_chunk_scan(const ChunkParams &p, hipStream_t s) {
    const unsigned blocks = (unsigned)(p.n_seqs * p.H * kTilesV);
    if (blocks > 0) hipLaunchKernelGGL(scan_kernel, dim3(blocks), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
