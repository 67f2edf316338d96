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
// e^{G_i - G_j} is split into per-token factors so every product is an MFMA
// contraction over channels: e^{G_i} e^{-G_j} with G counted from the chunk
// start when the chunk's whole decay is small, otherwise through reference
// points at the ends of 16-token sub-chunks, so that no factor exceeds the
// decay of 16 tokens (see phase 1).  W, Q e^G, K e^{G_L - G} and e^{G_L} only
// ever take e^{<= 0}.
//
// Two stages:
//  prepare  grid chunks x heads (heads fastest), 256 threads.  Everything that does not
//           depend on S: G, the exponentials, A and P (bf16 MFMA, fp32 acc),
//           the 64x64 unit-lower-triangular inverse (fp32, LDS, blocked by
//           16), W and U~.
//           Results go to the workspace as ready-made MFMA fragments.
//  scan     grid (sequences x heads x 8 value tiles), two waves per tile (for
//           batches of many heads, two tiles per block).  Walks
//           a sequence's chunks in order; the 128 x 16 fp32 state tile stays
//           in the chain wave's accumulator registers the whole time (32
//           MFMAs per chunk on the serial path) while a second wave forms the
//           chunk's output (22 MFMAs) one chunk behind.  Blocks are numbered
//           so that the eight tiles of one (sequence, head) land on the same
//           XCD and share its L2.
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Fragment convention (checked on the
// device): lane l holds row (l % 16) of A / column (l % 16) of B with k
// elements 8 (l / 16) + e, and rows 4 (l / 16) + r, column (l % 16) of C.
// Any consistent renumbering of k between A and B leaves the product
// unchanged; the scan uses k order {4g..4g+3, 16+4g..16+4g+3} inside each
// 32-wide k step so that the state and U accumulators (C layout) become the
// B operand of the next product with no data movement.
#include "kda_chunk_table.h"
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
                ci.seq = n;
                ci.first = c == 0;
                info[excl + c] = ci;
            }
        }
        __syncthreads();
        if (tid == 255) carry += buf[255];
        __syncthreads();
    }
    if (tid == 0) chunk_off[n_seqs] = carry;
}

// Record of (chunk, head): head-major, so one head's chunks are contiguous and
// the sequential scan of a head walks forward through memory.
__device__ __forceinline__ unsigned char *record(const ChunkParams &p, long cid, int h) {
    return p.records + ((long)h * p.n_chunks + cid) * (long)kChunkRecordBytes;
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
// Per-channel decay factors of the sub-chunk form (phases 1-2 only, in the T
// tile after the totals): E_off[4] = e^{R_{w-1}}, Hd[4] = e^{R_{I-1} - R_I},
// F[3] = e^{R_{I-1} - R_J} for (I, J) = (2, 0), (3, 1), (3, 0); fp32 [128] each.
constexpr int kOffEoff = kOffTm + 4 * 128 * 4;
constexpr int kOffHd = kOffEoff + 4 * 128 * 4;
constexpr int kOffF = kOffHd + 4 * 128 * 4;
static_assert(kOffF + 3 * 128 * 4 <= kOffTm + 64 * kRowT * 2, "decay factors alias the T tile");
// A chunk whose total decay stays within this (log2 units, every channel) is
// formed with every decay referenced to the chunk start: operands e^{+-G}
// within 2^+-64.  Beyond it, the 16-token sub-chunk form.
constexpr float kChunkStartRefMax = 64.0f;

// compile-time flag for the two instances of the decay-dependent phases
template <bool B>
struct SubForm {
    static constexpr bool value = B;
};

// 8 bf16 (one MFMA fragment: channels c0 .. c0 + 7) times 8 per-channel
// factors, re-rounded to bf16.
__device__ __forceinline__ bf16x8 scale_frag(const bf16x8 &x, const float *f) {
    const u32x4 w = __builtin_bit_cast(u32x4, x);
    const f32x4 f0 = *reinterpret_cast<const f32x4 *>(f), f1 = *reinterpret_cast<const f32x4 *>(f + 4);
    u32x4 o;
    o[0] = pack_bf2(lo_bf(w[0]) * f0[0], hi_bf(w[0]) * f0[1]);
    o[1] = pack_bf2(lo_bf(w[1]) * f0[2], hi_bf(w[1]) * f0[3]);
    o[2] = pack_bf2(lo_bf(w[2]) * f1[0], hi_bf(w[2]) * f1[1]);
    o[3] = pack_bf2(lo_bf(w[3]) * f1[2], hi_bf(w[3]) * f1[3]);
    return as_bf16x8(o);
}

// A (fp32 [64][64]) keeps the 16-byte column groups of row i XORed with
// (i & 15): sixteen rows read at the same columns land in sixteen different
// bank groups.
__device__ __forceinline__ int aix(int i, int j) { return i * 64 + ((((j >> 2) ^ i) & 15) << 2) + (j & 3); }

__device__ __forceinline__ bf16x8 lds_frag(const unsigned char *lds, int off_bytes) {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(lds + off_bytes));
}

// FUSED: q, k, v, beta come raw (pre-conv bf16 rows, beta logits) and this
// kernel applies the short causal conv (K <= 4 taps, zero-padded to 4 so the
// register window is indexed statically), the activation, the L2 norm of q
// and k (a DPP wave reduction per token: lanes hold the token's channels) and
// the sigmoid of beta.  The conv reads the 3 rows before the chunk from the
// same sequence, or from the incoming conv cache at a sequence start.
// KC: conv taps, ACT: 1 = SiLU after the conv, 0 = none (both fused only; the
// unfused instance ignores them)
template <bool FUSED, int KC, int ACT>
__global__ __launch_bounds__(256, 2) void prepare_kernel(ChunkParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsPrepare];
    // heads vary fastest: concurrent blocks read adjacent heads of one chunk
    const int h = blockIdx.x % p.H, cid = blockIdx.x / p.H;
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches and addresses
    const int H = p.H;
    const ChunkInfo ci = load_chunk(p, cid);
    const long tok0 = ci.start;
    const int len = ci.len;
    unsigned char *rec = record(p, cid, h);
    // (fused) the sequence's token range, for the outgoing conv cache at the
    // end: read here, from the kernel arguments or through a buffer resource
    // over the device copy (never a flat load, whose wait would cover every
    // memory access before it), so that its use after the record stores waits
    // for this read only, not for the stores
    int seq_lo = 0, seq_hi = 0;
    if constexpr (FUSED) {
        if (p.plan_in_args) {
            seq_lo = p.plan_cu[ci.seq];
            seq_hi = p.plan_cu[ci.seq + 1];
        } else {
            const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(p.cu, (uint32_t)((p.n_seqs + 1) * 4));
            seq_lo = (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)(ci.seq * 4), 0, 0);
            seq_hi = (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)(ci.seq * 4 + 4), 0, 0);
        }
    }

    float *A = reinterpret_cast<float *>(lds + kOffA);
    uint16_t *Tm = reinterpret_cast<uint16_t *>(lds + kOffTm);
    float *beta_s = reinterpret_cast<float *>(lds + kOffBeta);
    float *tot = reinterpret_cast<float *>(lds + kOffTm);   // [4][128], dead before T is written


    // ---- phase 1: cumulative log decay and decayed operands ----------------
    // wave w: tokens 16w..16w+15; lane l: channels 2l, 2l+1.  Every wave
    // issues the same loads, in order of first use, so each wait covers only
    // what the next step needs: (fused) conv taps and incoming-cache rows,
    // then log alpha and beta, then the q, k, v rows token by token.
    float wc[3][2][4];     // fused: taps, zero-padded on the old side to 4
    float2 halo[3][3];     // fused: the 3 rows before this wave's tokens
    if constexpr (FUSED) {
        const long C = (long)H * kHeadDim;
#pragma unroll
        for (int X = 0; X < 3; ++X)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float *src = p.conv_w + (X * C + h * kHeadDim + 2 * l + e) * KC;
                if constexpr (KC == 4) {
                    const f32x4 t = *reinterpret_cast<const f32x4 *>(src);
#pragma unroll
                    for (int j = 0; j < 4; ++j) wc[X][e][j] = t[j];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) wc[X][e][j] = j >= 4 - KC ? src[j - (4 - KC)] : 0.0f;
                }
            }
        // At a sequence start the rows before it come from the incoming conv
        // cache (zeros where it has none).  Every wave issues these loads; the
        // resource is empty unless this is wave 0 of a sequence's first chunk.
        constexpr int Km1 = KC - 1;
        if constexpr (Km1 > 0) {
            const bool fetch = w == 0 && ci.first && p.cache_in;
            const __amdgpu_buffer_rsrc_t rs =
                buffer_rsrc(p.cache_in + (long)ci.seq * 3 * Km1 * C, fetch ? (uint32_t)(3 * Km1 * C * 4) : 0u);
#pragma unroll
            for (int r = 0; r < 3; ++r)
#pragma unroll
                for (int X = 0; X < 3; ++X) {
                    const int slot = r - (3 - Km1);   // cache row of token tok0 - 3 + r
                    if (slot >= 0) {
                        const uint32_t off = (uint32_t)(((X * Km1 + slot) * C + h * kHeadDim + 2 * l) * 4);
                        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
                        halo[X][r] = make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
                    } else {
                        halo[X][r] = make_float2(0.f, 0.f);
                    }
                }
        } else {
#pragma unroll
            for (int r = 0; r < 3; ++r)
#pragma unroll
                for (int X = 0; X < 3; ++X) halo[X][r] = make_float2(0.f, 0.f);
        }
    }
    // Token rows (log alpha and q, k, v) are read through buffer resources
    // that start at the first row this block reads (up to 3 before the chunk
    // for the conv window) and end with the chunk's last token: rows past the
    // end, and the missing rows before token 0, load as 0, so the later steps
    // need no masks for them (and never see another sequence's values).
    constexpr int R0 = FUSED ? 3 : 0;
    const long row0 = tok0 - R0 < 0 ? 0 : tok0 - R0;
    const uint32_t rows_bytes = (uint32_t)((tok0 + len - row0) * H * kHeadDim * 2);
    const long rows_base = (row0 * H + h) * kHeadDim;
    auto row_off = [&](int t_rel) {   // t_rel: token index relative to tok0
        return (uint32_t)(((tok0 + t_rel - row0) * H * kHeadDim + 2 * l) * 2);
    };
    uint32_t ula[16];
    {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(p.log_alpha + rows_base, rows_bytes);
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) ula[ii] = __builtin_amdgcn_raw_buffer_load_b32(rs, row_off(16 * w + ii), 0, 0);
    }
    // beta of this wave's tokens (lane l & 15 holds token 16 w + (l & 15))
    float braw;
    {
        const long ob = (tok0 + max(0, min(16 * w + (l & 15), len - 1))) * H + h;
        braw = FUSED ? bf2f(p.beta_logit[ob]) : p.beta[ob];
    }
    // unfused: the prologue's rows q^, k^, v^ of this wave's 16 tokens;
    // fused: the raw rows of tokens 16w-3 .. 16w+15 (conv window)
    constexpr int NR = FUSED ? 19 : 16;
    uint32_t uq[NR], uk[NR], uv[NR];
    {
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc((FUSED ? p.q_raw : p.q) + rows_base, rows_bytes);
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc((FUSED ? p.k_raw : p.k) + rows_base, rows_bytes);
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc((FUSED ? p.v_raw : p.v) + rows_base, rows_bytes);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint32_t o = row_off(16 * w - R0 + r);
            uq[r] = __builtin_amdgcn_raw_buffer_load_b32(rq, o, 0, 0);
            uk[r] = __builtin_amdgcn_raw_buffer_load_b32(rk, o, 0, 0);
            uv[r] = __builtin_amdgcn_raw_buffer_load_b32(rv, o, 0, 0);
        }
    }
    // G in log2 units (log2 e folded into the sum), so decays are plain exp2
    constexpr float kLog2e = 1.4426950408889634f;
    float2 G[16];
    {
        float2 run = make_float2(0.f, 0.f);
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {   // rows past the end are 0: G stays at G_L
            run.x += kLog2e * lo_bf(ula[ii]);
            run.y += kLog2e * hi_bf(ula[ii]);
            G[ii] = run;
        }
        tot[w * 128 + 2 * l] = run.x;
        tot[w * 128 + 2 * l + 1] = run.y;
    }
    {   // lanes l, l + 16, l + 32, l + 48 store the same value (no branch around the load)
        const float b = FUSED ? sigmoidf(braw) : braw;
        const int tk = 16 * w + (l & 15);
        beta_s[tk] = tk < len ? b : 0.0f;
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
    const float2 egl = make_float2(__builtin_amdgcn_exp2f(GL.x), __builtin_amdgcn_exp2f(GL.y));   // e^{G_L}
    if (w == 0) *reinterpret_cast<float2 *>(rec + kOffGL + 8 * l) = egl;
    // Reference points of the decays.  With R_J the cumulative log decay at
    // the end of sub-chunk J (16 tokens; R_{-1} = 0), e^{G_i - G_j} for token
    // i of sub-chunk I and j of J <= I is
    //   e^{G_i - R_{I-1}} * e^{R_{I-1} - R_J} * e^{R_J - G_j},
    // three factors <= 1 for J < I; for J = I the middle one is
    // e^{R_{I-1} - R_I} >= 1, bounded by the decay of 16 tokens.  The row
    // operands (K, Q of A and P) then carry e^{G_i - R_{I-1}}, the column
    // operand K e^{R_J - G_j}, and phase 2 multiplies the column fragments by
    // the middle factor.  When the whole chunk's decay is small (every
    // channel's |G_L| <= kChunkStartRefMax) the chunk-start reference R = 0
    // for all tokens is exact in range too and needs no factors: the block
    // takes that form (the choice is the same in every wave: each reduces the
    // same 128 totals).
    float gmax = fmaxf(-GL.x, -GL.y);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) gmax = fmaxf(gmax, __shfl_xor(gmax, o, 64));
    // NaN decays take the sub-chunk form; readfirstlane makes the flag
    // scalar, so every test of it below is a scalar branch
    const bool sub = __builtin_amdgcn_readfirstlane((int)!(gmax <= kChunkStartRefMax)) != 0;
    const float2 tw = make_float2(tot[w * 128 + 2 * l], tot[w * 128 + 2 * l + 1]);   // R_w - R_{w-1}
    // e^G = el * eoff and e^{G_L - G} = ec * etail for the record's operands
    float2 eoff = make_float2(1.f, 1.f), etail = egl;
    if (sub) {   // block-uniform
        eoff = make_float2(__builtin_amdgcn_exp2f(off.x), __builtin_amdgcn_exp2f(off.y));
        etail = make_float2(__builtin_amdgcn_exp2f(GL.x - off.x - tw.x), __builtin_amdgcn_exp2f(GL.y - off.y - tw.y));
        float *fv = reinterpret_cast<float *>(lds);
        *reinterpret_cast<float2 *>(fv + kOffEoff / 4 + w * 128 + 2 * l) = eoff;
        *reinterpret_cast<float2 *>(fv + kOffHd / 4 + w * 128 + 2 * l) =
            make_float2(__builtin_amdgcn_exp2f(-tw.x), __builtin_amdgcn_exp2f(-tw.y));
        if (w == 1) *reinterpret_cast<float2 *>(fv + kOffF / 4 + 0 * 128 + 2 * l) =
            make_float2(__builtin_amdgcn_exp2f(tw.x), __builtin_amdgcn_exp2f(tw.y));
        if (w == 2) {
            const float2 t1 = make_float2(tot[128 + 2 * l], tot[128 + 2 * l + 1]);
            *reinterpret_cast<float2 *>(fv + kOffF / 4 + 1 * 128 + 2 * l) =
                make_float2(__builtin_amdgcn_exp2f(tw.x), __builtin_amdgcn_exp2f(tw.y));
            *reinterpret_cast<float2 *>(fv + kOffF / 4 + 2 * 128 + 2 * l) =
                make_float2(__builtin_amdgcn_exp2f(tw.x + t1.x), __builtin_amdgcn_exp2f(tw.y + t1.y));
        }
    }
    if constexpr (FUSED) {
        if (!(w == 0 && ci.first)) {   // otherwise halo holds the incoming cache rows
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                halo[0][r] = make_float2(lo_bf(uq[r]), hi_bf(uq[r]));
                halo[1][r] = make_float2(lo_bf(uk[r]), hi_bf(uk[r]));
                halo[2][r] = make_float2(lo_bf(uv[r]), hi_bf(uv[r]));
            }
        }
    }
    // Operands of phase 3, packed to bf16 now so few registers stay live:
    // pk[0] = beta k^ e^G, pk[1] = beta v^, pk[2] = k^ e^{G_L - G}; per channel
    // e (0, 1) the 16 tokens of this wave, two per 32-bit word (even token low).
    uint32_t pk[3][2][8];
    float prev[3][2];
    // With SiLU, the conv taps carry a factor log2 e, so the sigmoid's exp2
    // needs no multiply: x = log2e * silu(conv).  The L2 norm cancels the
    // factor (eps scaled by log2e^2 to match); v's products take ln 2.
    constexpr float kLn2 = 0.6931471805599453f;
    const float eps_n = ACT == 1 ? p.eps * (kLog2e * kLog2e) : p.eps;
    const float v_unscale = FUSED && ACT == 1 ? kLn2 : 1.0f;
    if constexpr (FUSED && ACT == 1) {
#pragma unroll
        for (int X = 0; X < 3; ++X)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int j = 0; j < 4; ++j) wc[X][e][j] *= kLog2e;
    }
    // The token loop in two instances, one per decay form (block-uniform).
    auto token_loop = [&](auto form) {
        constexpr bool SUB = decltype(form)::value;
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
            const int tk = 16 * w + ii;
            float2 q2 = make_float2(0.f, 0.f), k2 = q2, v2 = q2;
            if constexpr (FUSED) {
                // conv over rows ii .. ii+3 of the window (row ii+3 is token tk)
                float x[3][2];
#pragma unroll
                for (int X = 0; X < 3; ++X) {
                    const uint32_t *u = X == 0 ? uq : (X == 1 ? uk : uv);
                    float a0 = 0.f, a1 = 0.f;
#pragma unroll
                    for (int j = 4 - KC; j < 4; ++j) {
                        const int r = ii + j;
                        const float2 v = r < 3 ? halo[X][r] : make_float2(lo_bf(u[r]), hi_bf(u[r]));
                        a0 += wc[X][0][j] * v.x;
                        a1 += wc[X][1][j] * v.y;
                    }
                    // with SiLU the taps carry log2 e (see below): x = log2e * silu(conv)
                    x[X][0] = ACT == 1 ? a0 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a0)) : a0;
                    x[X][1] = ACT == 1 ? a1 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a1)) : a1;
                }
                const float r = __builtin_amdgcn_rsqf(
                    wave_sum_pair(x[0][0] * x[0][0] + x[0][1] * x[0][1], x[1][0] * x[1][0] + x[1][1] * x[1][1]) + eps_n);
                // tokens past the end: q, k scaled to 0 (their conv window still
                // holds real rows); v needs nothing, every product of v carries
                // beta = 0
                const bool live = tk < len;
                const float rq = live ? lane_value(r, 0) : 0.0f, rk = live ? lane_value(r, 16) : 0.0f;
                q2 = make_float2(x[0][0] * rq, x[0][1] * rq);
                k2 = make_float2(x[1][0] * rk, x[1][1] * rk);
                v2 = make_float2(x[2][0], x[2][1]);
            } else {   // rows past the end are 0
                q2 = make_float2(lo_bf(uq[ii]), hi_bf(uq[ii]));
                k2 = make_float2(lo_bf(uk[ii]), hi_bf(uk[ii]));
                v2 = make_float2(lo_bf(uv[ii]), hi_bf(uv[ii]));
            }
            // row factor (chunk-start form e^{G}, sub-chunk form e^{G - R_{w-1}})
            // and column factor (e^{-G}, e^{R_w - G})
            float ex, ey, ix, iy;
            if constexpr (SUB) {
                ex = __builtin_amdgcn_exp2f(G[ii].x);
                ey = __builtin_amdgcn_exp2f(G[ii].y);
                ix = __builtin_amdgcn_exp2f(tw.x - G[ii].x);
                iy = __builtin_amdgcn_exp2f(tw.y - G[ii].y);
            } else {
                const float gx = G[ii].x + off.x, gy = G[ii].y + off.y;
                ex = __builtin_amdgcn_exp2f(gx);
                ey = __builtin_amdgcn_exp2f(gy);
                ix = __builtin_amdgcn_exp2f(-gx);
                iy = __builtin_amdgcn_exp2f(-gy);
            }
            const float bt = beta_s[tk];
            const int e = tk * kRowA + 2 * l;
            const float kx = k2.x * ex, ky = k2.y * ey, kix = k2.x * ix, kiy = k2.y * iy;
            reinterpret_cast<uint32_t *>(lds + kOffKd)[e / 2] = pack_bf2(kx, ky);
            reinterpret_cast<uint32_t *>(lds + kOffKi)[e / 2] = pack_bf2(kix, kiy);
            reinterpret_cast<uint32_t *>(lds + kOffQs)[e / 2] = pack_bf2(q2.x * ex, q2.y * ey);
            const float bv = bt * v_unscale;
            const float cur[3][2] = {{SUB ? bt * eoff.x * kx : bt * kx, SUB ? bt * eoff.y * ky : bt * ky},
                                     {bv * v2.x, bv * v2.y},
                                     {kix * (SUB ? etail.x : egl.x), kiy * (SUB ? etail.y : egl.y)}};
#pragma unroll
            for (int a = 0; a < 3; ++a)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    if (ii % 2 == 0) prev[a][c] = cur[a][c];
                    else pk[a][c][ii / 2] = pack_bf2(prev[a][c], cur[a][c]);
                }
        }
    };
    if (sub) token_loop(SubForm<true>{});
    else token_loop(SubForm<false>{});
    __syncthreads();

    // ---- phase 2: A (row block I = w) and P^T (column block I = 3 - w) -----
    // Sub-chunk form: the column fragments of block J, as used against row
    // block I, take the factor e^{R_{I-1} - R_J} (none for J = I - 1).
    auto phase2 = [&](auto form) {
        constexpr bool SUB = decltype(form)::value;
        const float *fvec = reinterpret_cast<const float *>(lds);
        auto col_factor = [&](int I, int J) -> const float * {   // per-channel factor vector, or null
            if constexpr (!SUB) {
                return nullptr;
            } else {
                if (J == I - 1) return nullptr;
                if (J == I) return fvec + kOffHd / 4 + I * 128;
                return fvec + kOffF / 4 + (I == 2 ? 0 : (J == 1 ? 1 : 2)) * 128;
            }
        };
        {
            // the row block's K e^G fragments serve every column block J
            const int I = w;
            bf16x8 a[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) a[s] = lds_frag(lds, kOffKd + ((16 * I + c16) * kRowA + 32 * s + 8 * g) * 2);
            float bi[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) bi[r] = beta_s[16 * I + 4 * g + r];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (J <= I) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    const float *fc = col_factor(I, J);
                    if (fc) {   // uniform: sub-chunk form, a scaled column block
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc = mfma16(a[s], scale_frag(lds_frag(lds, kOffKi + ((16 * J + c16) * kRowA + 32 * s + 8 * g) * 2),
                                                          fc + 32 * s + 8 * g), acc);
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc = mfma16(a[s], lds_frag(lds, kOffKi + ((16 * J + c16) * kRowA + 32 * s + 8 * g) * 2), acc);
                    }
                    // every entry is written, the diagonal and above as 0 (no
                    // divergent stores; the inverse reads the blocks unmasked)
                    const int j = 16 * J + c16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * I + 4 * g + r;
                        A[aix(i, j)] = J < I || j < i ? bi[r] * acc[r] : 0.0f;
                    }
                }
            }
        }
        {
            // the column block's Q e^G fragments serve every row block J
            const int I = 3 - w;
            bf16x8 b[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) b[s] = lds_frag(lds, kOffQs + ((16 * I + c16) * kRowA + 32 * s + 8 * g) * 2);
            f32x4 blk[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (J <= I) {
                    const float *fc = col_factor(I, J);
                    if (fc) {   // uniform: sub-chunk form, a scaled column block
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc = mfma16(scale_frag(lds_frag(lds, kOffKi + ((16 * J + c16) * kRowA + 32 * s + 8 * g) * 2),
                                                    fc + 32 * s + 8 * g), b[s], acc);
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc = mfma16(lds_frag(lds, kOffKi + ((16 * J + c16) * kRowA + 32 * s + 8 * g) * 2), b[s], acc);
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
        // Qg fragments: token tile m = w, channel k-steps s = 0..3 (sub-chunk
        // form: the tile holds Q e^{G - R_{w-1}}; e^{R_{w-1}} per channel restores Q e^G)
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
            if (SUB && w > 0) {
                const float *fe = fvec + kOffEoff / 4 + w * 128 + 32 * s + 4 * g;
                const f32x4 f0 = *reinterpret_cast<const f32x4 *>(fe), f1 = *reinterpret_cast<const f32x4 *>(fe + 16);
                f[0] = pack_bf2(lo_bf(f[0]) * f0[0], hi_bf(f[0]) * f0[1]);
                f[1] = pack_bf2(lo_bf(f[1]) * f0[2], hi_bf(f[1]) * f0[3]);
                f[2] = pack_bf2(lo_bf(f[2]) * f1[0], hi_bf(f[2]) * f1[1]);
                f[3] = pack_bf2(lo_bf(f[3]) * f1[2], hi_bf(f[3]) * f1[3]);
            }
            *reinterpret_cast<u32x4 *>(rec + kOffQg + ((w * 4 + s) * 64 + l) * 16) = f;
        }
    };
    if (sub) phase2(SubForm<true>{});
    else phase2(SubForm<false>{});
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
    // Blocked inverse of the unit-lower-triangular I + A (A strictly lower;
    // the diagonal blocks hold zeros on and above their diagonals, the blocks
    // above them are never read):
    //   T_II = (I + A_II)^-1 per wave (block w): with P = -A_ww, nilpotent
    //        (P^16 = 0), (I + P)(I + P^2)(I + P^4)(I + P^8) = I + P + .. + P^15
    //        is the inverse; six 16x16 fp32 MFMA products, written over A_II,
    //        which nothing reads afterwards;
    //   T_Iw = -T_II sum_{K=w}^{I-1} A_IK T_Kw for I > w: wave w sweeps its
    //        column block down with fp32 MFMAs (16x16x4), holding T_Kw in
    //        registers.
    // In every product the contraction index of MFMA step kk is 4 (l >> 4) +
    // kk, so an accumulator's C layout (rows 4g + r, column c16) is the B
    // operand of the next product as it stands, and an A operand is one
    // 16-byte row read (row c16, columns 4g .. 4g + 3).  T goes to the bf16
    // tile Tm straight from registers.
    auto a_row4 = [&](int i, int j4) {   // A[i][4 j4 .. 4 j4 + 3]
        return *reinterpret_cast<const f32x4 *>(A + i * 64 + (((j4 ^ i) & 15) << 2));
    };
    auto mm = [&](const f32x4 &xr, const f32x4 &yc) {   // X (row layout) * Y (C layout), C layout
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma_f32(xr[kk], yc[kk], acc);
        return acc;
    };
    {
        // per-wave scratch for C-to-row transposes: [16][20] fp32 in the dead T tile
        float *sc = reinterpret_cast<float *>(lds + kOffTm) + w * 16 * 20;
        auto to_rows = [&](const f32x4 &c) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[(4 * g + r) * 20 + c16] = c[r];
            return *reinterpret_cast<const f32x4 *>(sc + c16 * 20 + 4 * g);
        };
        f32x4 Pc, Pr;   // P = -A_ww: C layout and row layout (A_ww is 0 on and above its diagonal)
        const f32x4 arow = a_row4(16 * w + c16, 4 * w + g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            Pc[r] = -A[aix(16 * w + 4 * g + r, 16 * w + c16)];
            Pr[r] = -arow[r];
        }
        const f32x4 P2c = mm(Pr, Pc);
        const f32x4 P2r = to_rows(P2c);
        const f32x4 P4c = mm(P2r, P2c);
        const f32x4 P4r = to_rows(P4c);
        const f32x4 P8c = mm(P4r, P4c);
        f32x4 Ic;
#pragma unroll
        for (int r = 0; r < 4; ++r) Ic[r] = 4 * g + r == c16 ? 1.0f : 0.0f;
        const f32x4 Yc = Ic + P4c + P8c + mm(P4r, P8c);   // (I + P^4)(I + P^8)
        const f32x4 Zc = Yc + mm(P2r, Yc);                // (I + P^2) Y
        const f32x4 Tw = Zc + mm(Pr, Zc);                 // (I + P) Z
#pragma unroll
        for (int r = 0; r < 4; ++r) A[aix(16 * w + 4 * g + r, 16 * w + c16)] = Tw[r];
    }
    __syncthreads();   // all diagonal inverses
    {
        f32x4 Tc[4];   // Tc[K] = T_Kw in C layout, K >= w
#pragma unroll
        for (int K = 0; K < 4; ++K) {
            Tc[K] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (K == w) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Tc[K][r] = A[aix(16 * K + 4 * g + r, 16 * K + c16)];
            }
        }
#pragma unroll
        for (int I = 1; I < 4; ++I) {
            if (I > w) {
                f32x4 M = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int K = 0; K < I; ++K) {
                    if (K >= w) {
                        const f32x4 a4 = a_row4(16 * I + c16, 4 * K + g);
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) M = mfma_f32(a4[kk], Tc[K][kk], M);
                    }
                }
                const f32x4 t4 = a_row4(16 * I + c16, 4 * I + g);   // T_II[c16][4g ..]
                f32x4 Tn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) Tn = mfma_f32(t4[kk], M[kk], Tn);
                Tc[I] = -Tn;
            }
        }
        // bf16 T: this wave's column block (diagonal and below); wave 3 also
        // zeroes the two blocks above the diagonal that phase 5 reads, (0, 1)
        // and (2, 3)
#pragma unroll
        for (int I = 0; I < 4; ++I)
            if (I >= w) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Tm[(16 * I + 4 * g + r) * kRowT + 16 * w + c16] = f2bf(Tc[I][r]);
            }
        if (w == 3) {
            const u32x2 z = {0u, 0u};
            *reinterpret_cast<u32x2 *>(Tm + (l >> 2) * kRowT + 16 + 4 * (l & 3)) = z;
            *reinterpret_cast<u32x2 *>(Tm + (32 + (l >> 2)) * kRowT + 48 + 4 * (l & 3)) = z;
        }
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

    // ---- outgoing conv cache (fused): this head's channels of the last K-1
    // input rows, written by the sequence's last chunk.  One thread walks the
    // rows of a channel in ascending order, so an output that aliases the
    // incoming cache reads each old row before it is overwritten.
    if constexpr (FUSED) {
        if (p.cache_out && len > 0) {
            if (tok0 + len == seq_hi) {
                const int Km1 = p.K - 1, C = H * kHeadDim;
                const long L = seq_hi - seq_lo;
                for (int idx = tid; idx < 3 * kHeadDim; idx += 256) {
                    const int X = idx / kHeadDim;
                    const long ch = (long)h * kHeadDim + idx % kHeadDim;
                    const uint16_t *raw = X == 0 ? p.q_raw : (X == 1 ? p.k_raw : p.v_raw);
                    const long row0 = ((long)ci.seq * 3 + X) * Km1;
                    for (int j = 0; j < Km1; ++j) {
                        const long tau = seq_hi - Km1 + j;
                        float v;
                        if (tau >= seq_lo) v = bf2f(raw[tau * C + ch]);
                        else v = p.cache_in ? p.cache_in[(row0 + j + L) * C + ch] : 0.0f;
                        p.cache_out[(row0 + j) * C + ch] = v;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// scan
// ---------------------------------------------------------------------------
__device__ __forceinline__ const u32x4 *frag_ptr(const unsigned char *rec, size_t off, int idx, int l) {
    return reinterpret_cast<const u32x4 *>(rec + off + ((size_t)idx * 64 + l) * 16);
}

// Operands of the state chain for one chunk and one 16-column tile.
struct ChainOperands {
    u32x4 W[16];    // -W fragments, index m * 4 + s
    u32x4 Kg[16];   // (K e^{G_L - G})^T fragments, index mm * 2 + s'
    f32x4 gl[8];    // e^{G_L} for rows 16 mm + 4 g .. + 3
    u32x2 U[4];     // U~ tile fragments (4 bf16), index m
};
__device__ __forceinline__ void load_chain(ChainOperands &o, const unsigned char *rec, int l, int g, int tile) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
        o.U[m] = *reinterpret_cast<const u32x2 *>(rec + kOffU + ((tile * 4 + m) * 64 + l) * 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) o.W[i] = *frag_ptr(rec, kOffW, i, l);
#pragma unroll
    for (int i = 0; i < 16; ++i) o.Kg[i] = *frag_ptr(rec, kOffKg, i, l);
#pragma unroll
    for (int mm = 0; mm < 8; ++mm)
        o.gl[mm] = *reinterpret_cast<const f32x4 *>(rec + kOffGL + (16 * mm + 4 * g) * 4);
}

// The two halves of load_chain, for the one-set schedule: U~ and W (used
// first in a step), then Kg and e^{G_L}.
__device__ __forceinline__ void load_chain_uw(ChainOperands &o, const unsigned char *rec, int l, int tile) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
        o.U[m] = *reinterpret_cast<const u32x2 *>(rec + kOffU + ((tile * 4 + m) * 64 + l) * 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) o.W[i] = *frag_ptr(rec, kOffW, i, l);
}
__device__ __forceinline__ void load_chain_kg(ChainOperands &o, const unsigned char *rec, int l, int g) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o.Kg[i] = *frag_ptr(rec, kOffKg, i, l);
#pragma unroll
    for (int mm = 0; mm < 8; ++mm)
        o.gl[mm] = *reinterpret_cast<const f32x4 *>(rec + kOffGL + (16 * mm + 4 * g) * 4);
}

// Operands of the output for one chunk and one tile.
struct OutOperands {
    u32x4 Q[16];    // Q e^G fragments, index m * 4 + s
    u32x4 P[6];     // P fragments (m, s' <= m / 2): 0:(0,0) 1:(1,0) 2:(2,0) 3:(2,1) 4:(3,0) 5:(3,1)
    u32x4 gate[2];  // 8 bf16 gate values of token (l >> 1) + 32 j, columns 8 (l & 1) ..
};
// Gate and output move in row layout: lane l owns 16 contiguous bytes (8
// columns) of token (l >> 1) + 32 j of the chunk.  Both go through a buffer
// resource that spans exactly the chunk's rows, so rows past its end load as
// 0 and are not stored, without a branch.
__device__ __forceinline__ uint32_t row_byte(const ChunkParams &p, int tk, int h, int tile, int l) {
    return (uint32_t)((((long)tk * p.H + h) * kHeadDim + tile * kTileV + 8 * (l & 1)) * 2);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rows(const ChunkParams &p, const uint16_t *base,
                                                             const ChunkInfo &ci) {
    const int start = __builtin_amdgcn_readfirstlane(ci.start), len = __builtin_amdgcn_readfirstlane(ci.len);
    return buffer_rsrc(base + (long)start * p.H * kHeadDim, (uint32_t)len * p.H * kHeadDim * 2);
}
// The output's operands of one chunk: fragments first (used by the MFMAs),
// the gate apart (used last, so it can be refilled after its use).
__device__ __forceinline__ void load_out_frags(OutOperands &o, const unsigned char *rec, int l) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o.Q[i] = *frag_ptr(rec, kOffQg, i, l);
    const int idx[6] = {0, 2, 4, 5, 6, 7};   // fragment m * 2 + s'
#pragma unroll
    for (int i = 0; i < 6; ++i) o.P[i] = *frag_ptr(rec, kOffP, idx[i], l);
}
__device__ __forceinline__ void load_out_gate(OutOperands &o, const ChunkParams &p, const ChunkInfo &ci, int h,
                                              int tile, int l) {
    const __amdgpu_buffer_rsrc_t rs = chunk_rows(p, p.gate, ci);
#pragma unroll
    for (int j = 0; j < 2; ++j)
        o.gate[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, row_byte(p, (l >> 1) + 32 * j, h, tile, l), 0, 0);
}

// Two waves per (sequence, head, 16-column tile), on different SIMDs:
//   wave 0, the state chain: per chunk U = U~ - W S and
//     S <- Diag(e^{G_L}) S + (K e^{G_L - G})^T U  (32 MFMAs); the 128 x 16
//     fp32 state stays in its accumulator registers for the whole sequence;
//   wave 1, the output, one chunk behind: O = (Q e^G) S + P U (22 MFMAs) and
//     y = scale O (.) gate, with S and U of that chunk handed over through
//     LDS as ready bf16 B-operand fragments (double-buffered).
// Each wave keeps two chunks of operands in registers and refills a buffer
// right after using it.  Every path issues the same loads (the refill index
// is clamped to the last chunk, masked rows go through buffer resources), so
// a wave waits only for the buffer it is about to use, never for all of its
// loads.  One barrier per chunk keeps the two waves in step.  The eight tiles
// of one (sequence, head) land on the same XCD.
//
// TPB > 1 puts TPB adjacent tiles of one (sequence, head) in one block (waves
// 0 .. TPB-1: their chains; the next TPB: their outputs).  The waves of each
// role issue the same fragment loads at the same time, so all but the first
// are served by the CU's L1 and the block pulls the chunk's shared fragments
// from L2 once for 16 TPB columns.
//
// DEEP (one tile per block, the single-sequence launch): each wave keeps two
// chunks of operands in flight, one wave per SIMD.  Otherwise (TPB = 4 or 2,
// launched when the batch gives every CU several tiles' work) the chain wave
// keeps one: it requests the chunk's Kg and e^{G_L} once its U product is
// issued, and the next chunk's U~ and W into the registers that product has
// just read.  That fits in 256 registers, so two blocks share each CU and one
// block's waits are filled by the other's work.
template <bool GATED, int TPB, bool DEEP = true>
__global__ __launch_bounds__(128 * TPB) __attribute__((amdgpu_waves_per_eu(DEEP ? 1 : 2, DEEP ? 1 : 2))) void scan_kernel(ChunkParams p) {
    constexpr int kOS = 20;                           // fp32 row stride of the output tile
    constexpr int kUnits = kTilesV / TPB;             // blocks per (sequence, head)
    __shared__ __attribute__((aligned(16))) u32x4 xfer_all[TPB][2][6][64];   // [tile][slot][Sb0..3, Ub0..1][lane]
    __shared__ __attribute__((aligned(16))) float O_all[TPB][64 * kOS];
    const int H = p.H;
    const int total = p.n_seqs * H * kUnits;    // a multiple of 8 (the launcher checks it)
    const int b = blockIdx.x;
    // Blocks go to the eight XCDs in turn (b % 8).  A (sequence, head) item's
    // kUnits blocks stay on one XCD, so they share its L2.  When the item
    // count divides by 8, items are dealt to the XCDs in turn and dispatched
    // in rank order: every XCD gets an even share, and with a host-side plan
    // the longest sequences are dispatched first, so a batch of mixed lengths
    // does not end on one long sequence started late.  Otherwise each XCD
    // takes a contiguous eighth of the blocks.
    int n, h, unit;
    if ((p.n_seqs * H) % 8 == 0) {
        const int slot = b / 8, item = (slot / kUnits) * 8 + b % 8;
        const int rank = item / H;
        h = item % H;
        n = p.plan_in_args ? (int)p.plan_order[rank] : rank;
        unit = slot % kUnits;
    } else {
        const int u = (b % 8) * (total / 8) + b / 8;
        h = (u / kUnits) % H;
        n = u / (kUnits * H);
        unit = u % kUnits;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool chain = wave < TPB;              // wave-uniform role
    const int sub = chain ? wave : wave - TPB;  // which of the block's tiles
    const int tile = unit * TPB + sub;
    auto &xfer = xfer_all[sub];
    float *O_lds = O_all[sub];
    const int l = threadIdx.x & 63, g = l >> 4, c16 = l & 15;
    // block-uniform values live in scalar registers (buffer resources built
    // from them need no per-lane loop)
    const int off0 = p.plan_in_args ? p.plan_off[n] : p.chunk_off[n];
    const int off1 = p.plan_in_args ? p.plan_off[n + 1] : p.chunk_off[n + 1];
    const int c_begin = __builtin_amdgcn_readfirstlane(max(0, off0));
    const int c_end = __builtin_amdgcn_readfirstlane(min(p.n_chunks, off1));
    const int nch = max(0, c_end - c_begin);
    const int col = tile * kTileV + c16;
    const long sbase = ((long)n * H + h) * kHeadDim * kHeadDim;
    // refills past the last chunk reload the last chunk (in bounds, unused)
    auto rec_of = [&](int i) { return (const unsigned char *)record(p, c_begin + min(i, nch - 1), h); };

    if (nch == 0) {   // empty sequence: the state passes through unchanged
        if (chain && p.s_final) {
#pragma unroll
            for (int mm = 0; mm < 8; ++mm)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const long e = sbase + (16 * mm + 4 * g + r) * kHeadDim + col;
                    p.s_final[e] = p.s0 ? p.s0[e] : 0.0f;
                }
        }
        return;
    }

    if (chain) {
        // ---------------- state chain ----------------
        f32x4 S[8];
        if (p.s0) {
#pragma unroll
            for (int mm = 0; mm < 8; ++mm)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[mm][r] = p.s0[sbase + (16 * mm + 4 * g + r) * kHeadDim + col];
        } else {
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) S[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        ChainOperands o0, o1;
        if constexpr (DEEP) {
            load_chain(o0, rec_of(0), l, g, tile);
            load_chain(o1, rec_of(1), l, g, tile);
        } else {
            load_chain_uw(o0, rec_of(0), l, tile);
        }
        auto step = [&](int i, ChainOperands &o) {
            // The U~ tile is the first load of a chunk's set.  Used here, after
            // the barrier: its bf16 unpacking, left free, is hoisted into the
            // previous step, whose wait for it (waits are in order) would
            // then also wait for the rest of this chunk's operands.
#pragma unroll
            for (int m = 0; m < 4; ++m) asm volatile("" : "+v"(o.U[m]));
            bf16x8 Sb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                Sb[s] = pack8(S[2 * s], S[2 * s + 1]);
                xfer[i & 1][s][l] = __builtin_bit_cast(u32x4, Sb[s]);
            }
            f32x4 U[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                U[m][0] = lo_bf(o.U[m][0]);
                U[m][1] = hi_bf(o.U[m][0]);
                U[m][2] = lo_bf(o.U[m][1]);
                U[m][3] = hi_bf(o.U[m][1]);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) U[m] = mfma16(as_bf16x8(o.W[m * 4 + s]), Sb[s], U[m]);
            if constexpr (!DEEP) {
                // this chunk's Kg and e^{G_L}, then the next chunk's U~ and W
                // (into the registers the products above have just read)
                load_chain_kg(o, rec_of(i), l, g);
                load_chain_uw(o, rec_of(i + 1), l, tile);
            }
            bf16x8 Ub[2];
            Ub[0] = pack8(U[0], U[1]);
            Ub[1] = pack8(U[2], U[3]);
            xfer[i & 1][4][l] = __builtin_bit_cast(u32x4, Ub[0]);
            xfer[i & 1][5][l] = __builtin_bit_cast(u32x4, Ub[1]);
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) S[mm] *= o.gl[mm];
#pragma unroll
            for (int sp = 0; sp < 2; ++sp)
#pragma unroll
                for (int mm = 0; mm < 8; ++mm) S[mm] = mfma16(as_bf16x8(o.Kg[mm * 2 + sp]), Ub[sp], S[mm]);
            if constexpr (DEEP) load_chain(o, rec_of(i + 2), l, g, tile);
        };
        // barriers: one after each chunk, one more while the output wave
        // finishes the last chunk (nch + 1, as in the output wave)
        int i = 0;
        for (; i + 1 < nch; i += 2) {
            step(i, o0);
            __syncthreads();
            step(i + 1, DEEP ? o1 : o0);
            __syncthreads();
        }
        if (i < nch) {
            step(i, o0);
            __syncthreads();
        }
        __syncthreads();
        if (p.s_final) {
#pragma unroll
            for (int mm = 0; mm < 8; ++mm)
#pragma unroll
                for (int r = 0; r < 4; ++r) p.s_final[sbase + (16 * mm + 4 * g + r) * kHeadDim + col] = S[mm][r];
        }
    } else {
        // ---------------- output, one chunk behind ----------------
        // chunk j of this sequence covers tokens seq_start + 64 j .. (no table load per chunk:
        // a load the gate addresses depend on would drain every prefetch before it)
        const int cu0 = p.plan_in_args ? p.plan_cu[n] : p.cu[n];
        const int cu1 = p.plan_in_args ? p.plan_cu[n + 1] : p.cu[n + 1];
        const int seq_start = __builtin_amdgcn_readfirstlane(min(max(cu0, 0), p.T));
        const int seq_len = __builtin_amdgcn_readfirstlane(max(0, min(cu1, p.T) - seq_start));
        auto chunk_of = [&](int j) {
            ChunkInfo ci;
            j = min(j, nch - 1);
            ci.len = max(0, min(kChunk, seq_len - kChunk * j));
            ci.start = ci.len > 0 ? seq_start + kChunk * j : 0;
            return ci;
        };
        OutOperands o0, o1;
        load_out_frags(o0, rec_of(0), l);
        if constexpr (GATED) load_out_gate(o0, p, chunk_of(0), h, tile, l);
        load_out_frags(o1, rec_of(1), l);
        if constexpr (GATED) load_out_gate(o1, p, chunk_of(1), h, tile, l);
        auto step = [&](int j, OutOperands &o) {
            const ChunkInfo ci = chunk_of(j);
            bf16x8 Sb[4], Ub[2];
#pragma unroll
            for (int s = 0; s < 4; ++s) Sb[s] = __builtin_bit_cast(bf16x8, xfer[j & 1][s][l]);
            Ub[0] = __builtin_bit_cast(bf16x8, xfer[j & 1][4][l]);
            Ub[1] = __builtin_bit_cast(bf16x8, xfer[j & 1][5][l]);
            f32x4 O[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) O[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int m = 0; m < 4; ++m) O[m] = mfma16(as_bf16x8(o.Q[m * 4 + s]), Sb[s], O[m]);
            O[0] = mfma16(as_bf16x8(o.P[0]), Ub[0], O[0]);
            O[1] = mfma16(as_bf16x8(o.P[1]), Ub[0], O[1]);
            O[2] = mfma16(as_bf16x8(o.P[2]), Ub[0], O[2]);
            O[3] = mfma16(as_bf16x8(o.P[4]), Ub[0], O[3]);
            O[2] = mfma16(as_bf16x8(o.P[3]), Ub[1], O[2]);
            O[3] = mfma16(as_bf16x8(o.P[5]), Ub[1], O[3]);
            load_out_frags(o, rec_of(j + 2), l);
            // y = scale O (.) gate, transposed to row layout through this wave's LDS tile
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) O_lds[(16 * m + 4 * g + r) * kOS + c16] = O[m][r];
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
            f32x4 yr[2][2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const float *row = O_lds + ((l >> 1) + 32 * jj) * kOS + 8 * (l & 1);
                yr[jj][0] = *reinterpret_cast<const f32x4 *>(row);
                yr[jj][1] = *reinterpret_cast<const f32x4 *>(row + 4);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            const __amdgpu_buffer_rsrc_t rs = chunk_rows(p, p.out, ci);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                u32x4 yo;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float a = p.scale * yr[jj][q >> 1][2 * (q & 1)];
                    float bb = p.scale * yr[jj][q >> 1][2 * (q & 1) + 1];
                    if constexpr (GATED) {
                        const float g0 = lo_bf(o.gate[jj][q]), g1 = hi_bf(o.gate[jj][q]);
                        a *= p.gate_is_logit ? sigmoidf(g0) : g0;
                        bb *= p.gate_is_logit ? sigmoidf(g1) : g1;
                    }
                    yo[q] = pack_bf2(a, bb);
                }
                __builtin_amdgcn_raw_buffer_store_b128(yo, rs, row_byte(p, (l >> 1) + 32 * jj, h, tile, l), 0, 0);
            }
            if constexpr (GATED) load_out_gate(o, p, chunk_of(j + 2), h, tile, l);
        };
        __syncthreads();   // chunk 0 of the chain
        int j = 0;
        for (; j + 1 < nch; j += 2) {
            step(j, o0);
            __syncthreads();
            step(j + 1, o1);
            __syncthreads();
        }
        if (j < nch) {
            step(j, o0);
            __syncthreads();
        }
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

template <int KC>
void launch_fused_prepare(const ChunkParams &p, dim3 grid, hipStream_t s) {
    if (p.act == 1) hipLaunchKernelGGL((prepare_kernel<true, KC, 1>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prepare_kernel<true, KC, 0>), grid, dim3(256), 0, s, p);
}

hipError_t launch_chunk_plan(const ChunkParams &p, hipStream_t s) {
    if (!p.plan_in_args)
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p.cu, p.n_seqs, p.n_chunks, p.chunk_off,
                           p.chunk_info);
    return hipGetLastError();
}

hipError_t launch_chunk_prepare(const ChunkParams &p, hipStream_t s) {
    if (!p.plan_in_args)
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p.cu, p.n_seqs, p.n_chunks, p.chunk_off,
                           p.chunk_info);
    if (p.n_chunks > 0)
        hipLaunchKernelGGL((prepare_kernel<false, 4, 0>), dim3((unsigned)((long)p.n_chunks * p.H)), dim3(256), 0, s,
                           p);
    return hipGetLastError();
}

hipError_t launch_prefill_prepare(const ChunkParams &p, hipStream_t s) {
    if (!p.plan_in_args)
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p.cu, p.n_seqs, p.n_chunks, p.chunk_off,
                           p.chunk_info);
    if (p.n_chunks > 0) {
        const dim3 grid((unsigned)((long)p.n_chunks * p.H));
        switch (p.K) {
            case 1: launch_fused_prepare<1>(p, grid, s); break;
            case 2: launch_fused_prepare<2>(p, grid, s); break;
            case 3: launch_fused_prepare<3>(p, grid, s); break;
            default: launch_fused_prepare<4>(p, grid, s); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_chunk_scan(const ChunkParams &p, hipStream_t s) {
    const long heads = (long)p.n_seqs * p.H;
    if (heads == 0) return hipGetLastError();
    // several tiles per block once the one-tile grid would put two blocks on
    // every CU (256 CUs) and the grid still divides by 8 (XCDs): four when the
    // head count allows, else two
    if (heads * kTilesV >= 512 && heads % 4 == 0) {
        const dim3 grid((unsigned)(heads * kTilesV / 4));
        if (p.gate) hipLaunchKernelGGL((scan_kernel<true, 4, false>), grid, dim3(512), 0, s, p);
        else hipLaunchKernelGGL((scan_kernel<false, 4, false>), grid, dim3(512), 0, s, p);
    } else if (heads * kTilesV >= 512 && heads % 2 == 0) {
        const dim3 grid((unsigned)(heads * kTilesV / 2));
        if (p.gate) hipLaunchKernelGGL((scan_kernel<true, 2, false>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((scan_kernel<false, 2, false>), grid, dim3(256), 0, s, p);
    } else {
        const dim3 grid((unsigned)(heads * kTilesV));
        if (p.gate) hipLaunchKernelGGL((scan_kernel<true, 1>), grid, dim3(128), 0, s, p);
        else hipLaunchKernelGGL((scan_kernel<false, 1>), grid, dim3(128), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace kda
