// Linear maps of the KDA mixer for gfx950 (the k3 README, "Use this
// repository as a template", places the projections and the output gate in
// the KDA module, around the recurrence primitive): the input projection of
// hidden states to the raw q, k, v, gate logits, decay and beta logits, and
// the output projection back to the hidden size.
//
// Both are C = A B^T with A [M][K] (activations) and B [N][K] (weights, one
// row per output feature), bf16, K contiguous in both, so an MFMA fragment of
// either (16 rows x 8 consecutive k per lane) is one 16-byte read.  fp32
// accumulation on v_mfma_f32_16x16x32_bf16, bf16 results.
//
// Block tile 256 x 256, K tile 64, eight waves (two per SIMD) in a 2 x 4
// grid, each owning 128 x 64 (8 x 4 MFMA tiles, 32 fp32x4 accumulators kept
// in architectural VGPRs, which the compiler updates in place), one block per
// CU.  While one wave of a SIMD waits for LDS, the other issues MFMAs.  Tiles
// travel from memory straight into LDS (buffer loads with the LDS
// destination: no staging registers) through two stages: tile kt + 1 is
// requested while tile kt is multiplied.  Per iteration a wave first waits
// for its own loads of tile kt and its LDS reads of tile kt - 1, then the
// block barrier makes every wave's part of tile kt visible and frees the
// stage that tile kt + 1 goes into.  The two stages are separate LDS arrays
// and the loop is unrolled by two, so the compiler sees which stage each LDS
// read touches and never waits for a load into the other one.  LDS rows are
// 128 bytes with the 16-byte chunk kc of row r stored at chunk
// kc ^ ((r >> 1) & 7): the 16 rows of a fragment read then cover all 64
// banks once.  Out-of-range rows, weight rows, K tails and the tile past K's
// end load as zero through buffer resources.
//
// Epilogues: plain (one [M][N] bf16 output) or the KDA input projection,
// whose N columns are six segments: q, k, v, gate, decay (H d each,
// head-major) and beta (H).  The beta columns go to a narrow kernel of their
// own: in the tile grid they would add a column of tiles that costs as much
// as a full one (at T = 4096, hidden 7168, H = 32: 1296 tiles, a sixth round
// on 256 CUs for 16 of them; without them 1280, five rounds).  The decay
// segment leaves as
//   log alpha = -exp(a_log[h]) * softplus(z + bias[h d + c]),
// a mapping the pages leave open (this library's reading; a_log and bias may
// be absent, giving -softplus(z)).
#include <atomic>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kBM = 256, kBK = 64;
constexpr int kABytes = kBM * kBK * 2;
constexpr int kGroupM = 4;                               // M tiles per ordering group

// Tile widths: 256 (eight waves in a 2 x 4 grid of 128 x 64 wave tiles) or
// 224 (4 x 2 waves of 64 x 112), the latter for outputs whose tile count
// would leave the last round on the CUs mostly idle: N = 7168 at M = 4096 is
// 448 tiles of 256 (two rounds on 256 CUs, the second three-quarters full)
// or 512 of 224 (two full rounds of 7/8-size tiles).
template <int BN>
struct TileShape {
    static constexpr int WN = BN == 256 ? 4 : 2;   // waves along N
    static constexpr int WM = 8 / WN;              // waves along M
    static constexpr int MT = kBM / WM / 16;       // 16 x 16 MFMA tiles per wave, along M
    static constexpr int NT = BN / WN / 16;        // ... along N
    static constexpr int kStage = kABytes + BN * kBK * 2;
    static_assert(WM * MT * 16 == kBM && WN * NT * 16 == BN, "wave tiles cover the block tile");
};

// byte offset of the 16-byte chunk kc (8 bf16) of row r in a 128-byte-row tile
__device__ __forceinline__ int swz(int r, int kc) { return r * 128 + ((kc ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ bf16x8 lds_frag16(const unsigned char *lds, int off_bytes) {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(lds + off_bytes));
}

// softplus(x) = log(1 + e^x), without overflow and accurate for small e^-|x|
__device__ __forceinline__ float softplus_f(float x) {
    const float u = __expf(-fabsf(x));
    const float lp = u < 1e-4f ? u * (1.0f - 0.5f * u) : __logf(1.0f + u);
    return fmaxf(x, 0.0f) + lp;
}

typedef __attribute__((address_space(3))) unsigned char lds_byte;

// s_waitcnt operands: vmcnt = n (n < 16), expcnt left unconstrained, and
// lgkmcnt either unconstrained or 0
constexpr int waitcnt_vm(int n) { return (n & 0xf) | (0x7 << 4) | (0xf << 8); }
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 0xf) | (0x7 << 4); }

template <int EPI, int BN>
__global__ __launch_bounds__(512, 1) void gemm_kernel(ProjParams p) {
    using TS = TileShape<BN>;
    constexpr int MT = TS::MT, NT = TS::NT, WTM = MT * 16, WTN = NT * 16;   // wave tile WTM x WTN
    __shared__ __attribute__((aligned(16))) unsigned char st0[TS::kStage], st1[TS::kStage];
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w / TS::WN, wn = w % TS::WN;
    const int tiles_m = (p.M + kBM - 1) / kBM, tiles_n = (p.N + BN - 1) / BN;
    const int total = tiles_m * tiles_n;
    // blocks go round the 8 XCDs in turn: XCD x = b % 8 takes a contiguous run
    // of tile indices u, and within it tiles are ordered in groups of kGroupM M
    // tiles by every N tile (M fastest), so the blocks an XCD runs together
    // share both their activation rows and their weight rows in its L2
    const int b = blockIdx.x, xq = total / 8, xr = total % 8, x = b % 8;
    const int u = x * xq + min(x, xr) + b / 8;
    const int per_group = kGroupM * tiles_n, first_m = (u / per_group) * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM), ug = u % per_group;
    // N tiles in reverse: a narrow last column (the input projection's beta
    // outputs) is dispatched in the first round, not alone in an extra one
    const int bm = first_m + ug % gm, bn = tiles_n - 1 - ug / gm;
    const int row0 = bm * kBM, col0 = bn * BN;
    const int nk = (p.K + kBK - 1) / kBK;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(p.a, (uint32_t)((long)p.M * p.K * 2));
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(p.b, (uint32_t)((long)p.N * p.K * 2));

    // tile kt into one stage: each load instruction fills 1 KB (8 rows) of the
    // stage, lane l the 16 bytes at 16 l; the lane fetches the chunk that the
    // swizzle puts there.  A takes 4 instructions per wave, B BN / 64 (blocks
    // of 8 rows w * 4 .. w * 4 + 3 that exist: at BN = 224 wave 7 has none).
    auto issue_tile = [&](int kt, unsigned char *st) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int blk = w * 4 + i, r = blk * 8 + (l >> 3), kc = (l & 7) ^ ((r >> 1) & 7);
            const int k = k0 + 8 * kc;
            const uint32_t off = (k < p.K && row0 + r < p.M) ? (uint32_t)(((long)(row0 + r) * p.K + k) * 2)
                                                             : 0xffffffffu;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_byte *)(st + blk * 1024), 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int blk = w * 4 + i, r = blk * 8 + (l >> 3), kc = (l & 7) ^ ((r >> 1) & 7);
            if (BN == 256 || blk < BN / 8) {   // wave-uniform
                const int k = k0 + 8 * kc;
                const uint32_t off = (k < p.K && col0 + r < p.N) ? (uint32_t)(((long)(col0 + r) * p.K + k) * 2)
                                                                 : 0xffffffffu;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_byte *)(st + kABytes + blk * 1024), 16, off, 0, 0,
                                                         0);
            }
        }
    };

    // the KDA input projection's per-column epilogue parameters, loaded now
    // so that their latency passes under the main loop: decay columns take
    // a_log[h] and their bias, every other column (and absent ones) 0
    float epi_A[NT], epi_b[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        epi_A[n] = 0.0f;
        epi_b[n] = 0.0f;
        if constexpr (EPI == 1) {
            const int C = p.H * p.d, col = col0 + WTN * wn + 16 * n + c16;
            if (col >= 4 * C && col < 5 * C) {
                const int within = col - 4 * C;
                if (p.a_log) epi_A[n] = p.a_log[within / p.d];
                if (p.bias) epi_b[n] = p.bias[within];
            }
        }
    }

    f32x4 acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one iteration: tile kt sits in stage `cur`; `nxt` (the other stage)
    // receives tile kt + 1
    auto step = [&](int kt, const unsigned char *cur, unsigned char *nxt) {
        // the barrier without __syncthreads' fences, which would wait for every
        // load in flight; the empty asm statements keep the compiler from moving
        // LDS accesses across it.  Before it, each wave waits for its own part of
        // tile kt and for its LDS reads of the previous tile (lgkmcnt 0), whose
        // stage the loads issued after the barrier overwrite
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();                            // everyone's part; stage nxt free
        asm volatile("" ::: "memory");
        issue_tile(kt + 1, nxt);
        asm volatile("" ::: "memory");   // requests out before this tile's reads
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 fa[MT], fb[NT];
#pragma unroll
            for (int m = 0; m < MT; ++m) fa[m] = lds_frag16(cur, swz(WTM * wm + 16 * m + c16, 4 * kk + g));
#pragma unroll
            for (int n = 0; n < NT; ++n) fb[n] = lds_frag16(cur, kABytes + swz(WTN * wn + 16 * n + c16, 4 * kk + g));
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[m][n] = mfma16(fa[m], fb[n], acc[m][n]);
        }
    };

    issue_tile(0, st0);
    for (int kt = 0; kt < nk; kt += 2) {   // an odd nk adds one all-zero tile
        step(kt, st0, st1);
        step(kt + 1, st1, st0);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // the trailing (all-zero) tile loads

    // epilogue: element (m, n, r) is row row0 + WTM wm + 16 m + 4 g + r,
    // column col0 + WTN wn + 16 n + c16
    // one column group of 16 (fixed n): out[row][within] for the 32 rows this
    // lane holds, through the decay activation or not
    auto store_cols = [&](int n, uint16_t *dst, int width, int within, bool decay, float A, float bias) {
        if (decay) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row0 + WTM * wm + 16 * m + 4 * g + r;
                    const float v = -A * softplus_f(acc[m][n][r] + bias);
                    if (row < p.M) dst[(long)row * width + within] = f2bf(v);
                }
        } else {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row0 + WTM * wm + 16 * m + 4 * g + r;
                    if (row < p.M) dst[(long)row * width + within] = f2bf(acc[m][n][r]);
                }
        }
    };
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int col = col0 + WTN * wn + 16 * n + c16;
        if constexpr (EPI == 0) {
            if (col < p.N) store_cols(n, p.out, p.N, col, false, 1.0f, 0.0f);
        } else {
            // one segment of the KDA input projection: q, k, v, gate, decay
            // (H d columns each) or beta (H).  With H d a multiple of 16, the
            // wave's 16 columns of this group lie in one segment: the segment
            // is then wave-uniform, and so is the decay branch
            const int C = p.H * p.d;
            int seg = col < 5 * C ? col / C : 5;
            if (C % 16 == 0) seg = __builtin_amdgcn_readfirstlane(seg);
            // the pointer is picked with constant indices (a runtime index
            // into the argument array would go through scratch memory)
            uint16_t *dst = seg == 0 ? p.seg[0] : seg == 1 ? p.seg[1] : seg == 2 ? p.seg[2]
                          : seg == 3 ? p.seg[3] : seg == 4 ? p.seg[4] : p.seg[5];
            const int within = col - seg * C, width = seg < 5 ? C : p.H;
            if (col < p.N) store_cols(n, dst, width, within, seg == 4, __expf(epi_A[n]), epi_b[n]);
        }
    }
}

// out[M][n_cols] (row stride ldo) = A B^T for a narrow B (rows b[0 .. n_cols),
// each K long).  A block takes 16 rows x 32 columns; its eight waves split
// the K steps of 32 (wave w: steps w, w + 8, ...), each with four steps' loads
// in flight, and add their partial sums in LDS in wave order.  Rows, columns
// and K chunks past the ends load as zero through the buffer resources.
__global__ __launch_bounds__(512) void gemm_narrow_kernel(ProjParams p, const uint16_t *b, int n_cols,
                                                          uint16_t *out, int ldo) {
    __shared__ __attribute__((aligned(16))) f32x4 red[8][2][64];
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, c16 = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row0 = blockIdx.x * 16, n0 = blockIdx.y * 32;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(p.a, (uint32_t)((long)p.M * p.K * 2));
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(b, (uint32_t)((long)n_cols * p.K * 2));
    // byte offset of a fragment chunk, or past every resource when the row or
    // the chunk lies outside (K is a multiple of 8: a chunk is all in or out)
    auto off = [&](long row, long rows, int k) -> uint32_t {
        return (row < rows && k < p.K) ? (uint32_t)((row * p.K + k) * 2) : 0xffffffffu;
    };
    auto load = [&](int ks, u32x4 &fa, u32x4 (&fb)[2]) {
        const int k = ks * 32 + 8 * g;
        fa = __builtin_amdgcn_raw_buffer_load_b128(ra, off(row0 + c16, p.M, k), 0, 0);
#pragma unroll
        for (int nn = 0; nn < 2; ++nn)
            fb[nn] = __builtin_amdgcn_raw_buffer_load_b128(rb, off(n0 + 16 * nn + c16, n_cols, k), 0, 0);
    };
    const int nks = (p.K + 31) / 32, steps = (nks + 31) / 32 * 4;   // per wave, a multiple of 4
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    u32x4 fa[4], fb[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) load(w + 8 * i, fa[i], fb[i]);
    for (int j = 0; j < steps; j += 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int nn = 0; nn < 2; ++nn) acc[nn] = mfma16(as_bf16x8(fa[i]), as_bf16x8(fb[i][nn]), acc[nn]);
            load(w + 8 * (j + i + 4), fa[i], fb[i]);
        }
    }
    // acc[nn][r]: row row0 + 4 g + r, column n0 + 16 nn + c16
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) red[w][nn][l] = acc[nn];
    __syncthreads();
    const int nn = tid >> 8, ll = (tid >> 2) & 63, r = tid & 3;
    float sum = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) sum += red[ww][nn][ll][r];
    const int row = row0 + 4 * (ll >> 4) + r, col = n0 + 16 * nn + (ll & 15);
    if (row < p.M && col < n_cols) out[(long)row * ldo + col] = f2bf(sum);
}

// CUs of the current device, looked up once per device ordinal (256 when
// the query fails).  Racing first calls on one device store the same value.
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace

hipError_t launch_gemm(const ProjParams &p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipGetLastError();
    ProjParams q = p;
    if (p.epi == 1) q.N = 5 * p.H * p.d;   // the beta columns: gemm_narrow_kernel below
    const long tiles_m = (q.M + kBM - 1) / kBM;
    auto tiles = [&](int bn) { return tiles_m * ((q.N + bn - 1) / bn); };
    if (tiles(256) > 0) {
        if (q.epi == 1) {
            hipLaunchKernelGGL((gemm_kernel<1, 256>), dim3((unsigned)tiles(256)), dim3(512), 0, s, q);
        } else {
            // the tile width whose rounds over the CUs, each as long as its
            // tile is wide, add up to less (ties: 256)
            const int cus = cu_count();
            auto cost = [&](int bn) { return (tiles(bn) + cus - 1) / cus * bn; };
            if (cost(224) < cost(256))
                hipLaunchKernelGGL((gemm_kernel<0, 224>), dim3((unsigned)tiles(224)), dim3(512), 0, s, q);
            else
                hipLaunchKernelGGL((gemm_kernel<0, 256>), dim3((unsigned)tiles(256)), dim3(512), 0, s, q);
        }
    }
    if (p.epi == 1) {
        const dim3 grid((unsigned)((p.M + 15) / 16), (unsigned)((p.H + 31) / 32));
        hipLaunchKernelGGL(gemm_narrow_kernel, grid, dim3(512), 0, s, p, p.b + (long)q.N * p.K, p.H, p.seg[5], p.H);
    }
    return hipGetLastError();
}

}  // namespace kda
