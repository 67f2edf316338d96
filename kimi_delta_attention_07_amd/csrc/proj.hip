// Linear maps of the KDA mixer for gfx950 (the k3 README, "Use this
// repository as a template", places the projections and the output gate in
// the KDA module, around the recurrence primitive): the input projection of hidden states to the raw q, k, v, gate logits, decay
// and beta logits, and the output projection back to the hidden size.
//
// Both are C = A B^T with A [M][K] (activations) and B [N][K] (weights, one
// row per output feature), bf16, K contiguous in both, so an MFMA fragment of
// either (16 rows x 8 consecutive k per lane) is one 16-byte read.  fp32
// accumulation on v_mfma_f32_16x16x32_bf16, bf16 results.
//
// Block tile 256 (M) x 128 (N), K tile 64, four waves each owning 128 x 64
// (8 x 4 MFMA tiles, 32 fp32x4 accumulators).  The K tiles pass through LDS,
// double-buffered: iteration kt first sends out the loads of tile kt + 1 (into
// registers), computes on tile kt, then writes tile kt + 1 into the other
// buffer; loads are consumed in the iteration that issues them, so no loaded
// register is carried round the loop.  Rows are padded to 144 bytes, so the
// 16 rows of a fragment read land on 16 distinct 4-bank groups.  Out-of-range
// rows, weight rows and K tails load as zero through buffer resources.
//
// Epilogues: plain (one [M][N] bf16 output) or the KDA input projection,
// whose N columns are six segments: q, k, v, gate, decay (H d each,
// head-major) and beta (H).  The decay segment leaves as
//   log alpha = -exp(a_log[h]) * softplus(z + bias[h d + c]),
// a mapping the pages leave open (this library's reading; a_log and bias may
// be absent, giving -softplus(z)).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kBM = 256, kBN = 128, kBK = 64;
constexpr int kLdsRow = kBK + 8;                         // bf16 row stride (144 B)
constexpr int kABytes = kBM * kLdsRow * 2, kBBytes = kBN * kLdsRow * 2;
constexpr int kStage = kABytes + kBBytes;                // 55,296 B per K tile

__device__ __forceinline__ bf16x8 lds_frag16(const unsigned char *lds, int off_bytes) {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(lds + off_bytes));
}

// softplus(x) = log(1 + e^x), without overflow and accurate for small e^-|x|
__device__ __forceinline__ float softplus_f(float x) {
    const float u = __expf(-fabsf(x));
    const float lp = u < 1e-4f ? u * (1.0f - 0.5f * u) : __logf(1.0f + u);
    return fmaxf(x, 0.0f) + lp;
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_kernel(ProjParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kStage];   // two K-tile stages
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 1, wn = w & 1;
    const int tiles_m = (p.M + kBM - 1) / kBM, tiles_n = (p.N + kBN - 1) / kBN;
    const int total = tiles_m * tiles_n;
    // blocks go round the 8 XCDs in turn: give each XCD a contiguous run of
    // tiles (M fastest), so the blocks sharing a weight panel share an L2
    const int b = blockIdx.x;
    const int u = total % 8 == 0 ? (b % 8) * (total / 8) + b / 8 : b;
    const int bm = u % tiles_m, bn = u / tiles_m;
    const int row0 = bm * kBM, col0 = bn * kBN;
    const int nk = (p.K + kBK - 1) / kBK;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(p.a, (uint32_t)((long)p.M * p.K * 2));
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(p.b, (uint32_t)((long)p.N * p.K * 2));

    // tile loads: A is 256 rows x 8 chunks of 16 B (8 per thread), B 128 rows
    // x 8 chunks (4 per thread); consecutive threads read one row's chunks
    u32x4 va[8], vb[4];
    auto load_tile = [&](int kt) {
        const int k0 = min(kt, nk - 1) * kBK;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
            const int k = k0 + 8 * kc;
            const uint32_t off = k < p.K ? (uint32_t)(((long)(row0 + r) * p.K + k) * 2) : 0xffffffffu;
            va[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, row0 + r < p.M ? off : 0xffffffffu, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
            const int k = k0 + 8 * kc;
            const uint32_t off = k < p.K ? (uint32_t)(((long)(col0 + r) * p.K + k) * 2) : 0xffffffffu;
            vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, col0 + r < p.N ? off : 0xffffffffu, 0, 0);
        }
    };
    auto store_tile = [&](int stage) {
        unsigned char *s = lds + stage * kStage;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
            *reinterpret_cast<u32x4 *>(s + (r * kLdsRow + 8 * kc) * 2) = va[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
            *reinterpret_cast<u32x4 *>(s + kABytes + (r * kLdsRow + 8 * kc) * 2) = vb[i];
        }
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        load_tile(kt + 1);   // clamped: the last iteration reloads the last tile, unused
        const unsigned char *s = lds + (kt & 1) * kStage;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 fa[8], fb[4];
#pragma unroll
            for (int m = 0; m < 8; ++m)
                fa[m] = lds_frag16(s, ((128 * wm + 16 * m + c16) * kLdsRow + 32 * kk + 8 * g) * 2);
#pragma unroll
            for (int n = 0; n < 4; ++n)
                fb[n] = lds_frag16(s, kABytes + ((64 * wn + 16 * n + c16) * kLdsRow + 32 * kk + 8 * g) * 2);
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n) acc[m][n] = mfma16(fa[m], fb[n], acc[m][n]);
        }
        store_tile((kt + 1) & 1);   // the other buffer: last read in iteration kt - 1
        __syncthreads();
    }

    // epilogue: element (m, n, r) is row row0 + 128 wm + 16 m + 4 g + r,
    // column col0 + 64 wn + 16 n + c16
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int col = col0 + 64 * wn + 16 * n + c16;
        if (col >= p.N) continue;
        if constexpr (EPI == 0) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row0 + 128 * wm + 16 * m + 4 * g + r;
                    if (row < p.M) p.out[(long)row * p.N + col] = f2bf(acc[m][n][r]);
                }
        } else {
            const int C = p.H * p.d;
            const int seg = col < 5 * C ? col / C : 5;
            const int within = col - seg * C;
            const int width = seg < 5 ? C : p.H;
            uint16_t *dst = p.seg[seg];
            float A = 1.0f, bias = 0.0f;
            if (seg == 4) {
                if (p.a_log) A = __expf(p.a_log[within / p.d]);
                if (p.bias) bias = p.bias[within];
            }
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row0 + 128 * wm + 16 * m + 4 * g + r;
                    float v = acc[m][n][r];
                    if (seg == 4) v = -A * softplus_f(v + bias);
                    if (row < p.M) dst[(long)row * width + within] = f2bf(v);
                }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const ProjParams &p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipGetLastError();
    const long tiles = (long)((p.M + kBM - 1) / kBM) * ((p.N + kBN - 1) / kBN);
    const dim3 grid((unsigned)tiles);
    if (p.epi == 1) hipLaunchKernelGGL((gemm_kernel<1>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_kernel<0>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
