// KDA decode step for gfx950: one token for each of `batch` rows, fused.
//
// Order of work follows the kimi_k3 API docs (Functions: kda_decode_token):
// conv update first, then the recurrent step.  Per (row, head) one 256-thread
// workgroup
//   1. shifts the conv cache of q, k, v by one token and applies the causal
//      depthwise conv + activation (one (stream, channel) per thread);
//   2. L2-normalises q and k, forms alpha = exp(log_alpha), beta and the gate;
//   3. streams the d x d fp32 state once: every thread loads its float4s with
//      non-temporal 128-bit loads, accumulates the two column reductions
//          z = S^T (alpha q^),  w = S^T (alpha k^)
//      that both read the OLD state, then writes the new state
//          S' = Diag(alpha) S + beta k^ (v - w)^T
//      and the output  o = scale (z + beta (k^ . q^)(v - w)) (.) gate.
// (S' = (I - beta k k^T) Diag(alpha) S + beta k v^T expands to the second
// line because k^T Diag(alpha) S = w^T.)  The state is read and written once;
// everything else is small, so the kernel runs at HBM speed.  No matrix cores:
// per state element it does two FMAs for the reductions and one for the update.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ float sigmoid_acc(float x) { return 1.0f / (1.0f + expf(-x)); }

template <int D, int DTI, int DTO>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
    constexpr int NT = 256;
    constexpr int CG = D / 4;                   // float4 groups per state row
    constexpr int NF = D * D / 4;               // float4s per state matrix
    constexpr int FPT = (NF + NT - 1) / NT;     // float4s per thread
    static_assert(NT % CG == 0, "column group must be fixed per thread");

    __shared__ float xs[3][D];                  // conv outputs q~, k~, v~
    __shared__ float aq[D], ak[D], kh[D], al[D], us[D];
    __shared__ float red[8][NT];                // column partials (z[4], w[4]) per thread
    __shared__ float wred[4][3];

    // heads fastest: consecutive blocks stream consecutive 64 KB states of one row
    const int h = (int)(blockIdx.x % (unsigned)p.H), b = (int)(blockIdx.x / (unsigned)p.H), t = threadIdx.x;
    const int slot = p.slot_idx ? p.slot_idx[b] : b;
    // A row whose slot lies outside [0, n_slots) is skipped whole (the slot
    // is block-uniform, so the early exit is before every barrier): nothing
    // of it is read or written, its output row included.
    if ((unsigned)slot >= (unsigned)p.n_slots) return;
    const int C = p.H * D;
    const long row = ((long)b * p.H + h) * D;   // [b][h][0] of the per-row inputs
    const int Km1 = p.K - 1;

    // 1) conv cache shift + conv + activation
    for (int task = t; task < 3 * D; task += NT) {
        const int X = task / D, c = task - X * D, ch = h * D + c;
        const void *raw = X == 0 ? p.q_raw : (X == 1 ? p.k_raw : p.v_raw);
        const float x = load1<DTI>(raw, row + c);
        const float *w = p.conv_w + ((long)X * C + ch) * p.K;
        float acc = w[Km1] * x;
        if (Km1 > 0) {
            float *cache = p.conv_cache + ((long)slot * 3 + X) * Km1 * C + ch;
            float hist[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) hist[j] = j < Km1 ? cache[(long)j * C] : 0.0f;
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (j < Km1) acc += w[j] * hist[j];
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (j < Km1) cache[(long)j * C] = (j + 1 < Km1) ? hist[j + 1] : x;
        }
        xs[X][c] = activate(p.act, acc);
    }
    __syncthreads();

    // 2) L2 norms of q~, k~ and their dot product, block-wide
    {
        const float qv = t < D ? xs[0][t] : 0.0f, kv = t < D ? xs[1][t] : 0.0f;
        float s0 = group_sum(qv * qv, 64), s1 = group_sum(kv * kv, 64), s2 = group_sum(qv * kv, 64);
        if ((t & 63) == 0) {
            wred[t >> 6][0] = s0;
            wred[t >> 6][1] = s1;
            wred[t >> 6][2] = s2;
        }
    }
    __syncthreads();
    const float ssq = wred[0][0] + wred[1][0] + wred[2][0] + wred[3][0];
    const float ssk = wred[0][1] + wred[1][1] + wred[2][1] + wred[3][1];
    const float sqk = wred[0][2] + wred[1][2] + wred[2][2] + wred[3][2];
    const float rq = 1.0f / sqrtf(ssq + p.eps), rk = 1.0f / sqrtf(ssk + p.eps);
    const float qk = sqk * rq * rk;
    const float beta = sigmoid_acc(load1<DTI>(p.beta_logit, (long)b * p.H + h));
    if (t < D) {
        const float a = expf(load1<DTI>(p.log_alpha, row + t));
        const float qn = xs[0][t] * rq, kn = xs[1][t] * rk;
        aq[t] = a * qn;
        ak[t] = a * kn;
        kh[t] = kn;
        al[t] = a;
    }
    __syncthreads();

    // 3) one pass over the state
    float *S = p.state + ((long)slot * p.H + h) * (long)D * D;
    const int cg = t % CG;
    f32x4 sv[FPT];
#pragma unroll
    for (int r = 0; r < FPT; ++r) {
        const int f = t + r * NT;
        if (f < NF) sv[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S) + f);
    }
    float z[4] = {0.f, 0.f, 0.f, 0.f}, w[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < FPT; ++r) {
        const int f = t + r * NT;
        if (f < NF) {
            const int i = f / CG;
            const float a_q = aq[i], a_k = ak[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z[e] += sv[r][e] * a_q;
                w[e] += sv[r][e] * a_k;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        red[e][t] = z[e];
        red[4 + e][t] = w[e];
    }
    __syncthreads();
    if (t < D) {
        const int j = t, gj = j >> 2, e = j & 3;
        float zs = 0.f, ws = 0.f;
        for (int tt = gj; tt < NT; tt += CG) {
            zs += red[e][tt];
            ws += red[4 + e][tt];
        }
        const float u = beta * (xs[2][j] - ws);
        us[j] = u;
        float o = p.scale * (zs + qk * u);
        if (p.gate_logit) o *= sigmoid_acc(load1<DTI>(p.gate_logit, row + j));
        store1<DTO>(p.out, row + j, o);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < FPT; ++r) {
        const int f = t + r * NT;
        if (f < NF) {
            const int i = f / CG;
            const float a = al[i], k_i = kh[i];
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = a * sv[r][e] + k_i * us[cg * 4 + e];
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(S) + f);
        }
    }
}

template <int D>
hipError_t launch_d(const DecodeParams &p, int dti, int dto, hipStream_t s) {
    dim3 grid((unsigned)p.batch * (unsigned)p.H), block(256);
    if (dti == 1 && dto == 1) hipLaunchKernelGGL((decode_kernel<D, 1, 1>), grid, block, 0, s, p);
    else if (dti == 1) hipLaunchKernelGGL((decode_kernel<D, 1, 0>), grid, block, 0, s, p);
    else if (dto == 1) hipLaunchKernelGGL((decode_kernel<D, 0, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<D, 0, 0>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int dti, int dto, hipStream_t s) {
    switch (p.d) {
        case 4: return launch_d<4>(p, dti, dto, s);
        case 8: return launch_d<8>(p, dti, dto, s);
        case 16: return launch_d<16>(p, dti, dto, s);
        case 32: return launch_d<32>(p, dti, dto, s);
        case 64: return launch_d<64>(p, dti, dto, s);
        case 128: return launch_d<128>(p, dti, dto, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
