// Device-side helpers for the gfx950 KDA kernels: bf16 packing, typed
// loads/stores for the two input dtypes, wave64 reductions, gates.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16x2 (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two consecutive elements of a dtype-DT array (DT 0 = fp32, 1 = bf16),
// starting at an even element index.
template <int DT>
__device__ __forceinline__ float2 load2(const void *base, long idx) {
    if constexpr (DT == 1) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(base) + idx);
        return make_float2(lo_bf(w), hi_bf(w));
    } else {
        return *reinterpret_cast<const float2 *>(static_cast<const float *>(base) + idx);
    }
}
// Raw bits of two consecutive elements (bf16: one word in .x; fp32: .x, .y),
// so a load can stay in flight until unpack2() at the point of use.
template <int DT>
__device__ __forceinline__ uint2 load_raw2(const void *base, long idx) {
    if constexpr (DT == 1) {
        return make_uint2(*reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(base) + idx), 0u);
    } else {
        return *reinterpret_cast<const uint2 *>(static_cast<const float *>(base) + idx);
    }
}
template <int DT>
__device__ __forceinline__ float2 unpack2(uint2 r) {
    if constexpr (DT == 1) return make_float2(lo_bf(r.x), hi_bf(r.x));
    else return make_float2(__uint_as_float(r.x), __uint_as_float(r.y));
}
template <int DT>
__device__ __forceinline__ void store2(void *base, long idx, float a, float b) {
    if constexpr (DT == 1) {
        *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(base) + idx) = pack_bf2(a, b);
    } else {
        *reinterpret_cast<float2 *>(static_cast<float *>(base) + idx) = make_float2(a, b);
    }
}
template <int DT>
__device__ __forceinline__ float load1(const void *base, long idx) {
    if constexpr (DT == 1) return bf2f(static_cast<const uint16_t *>(base)[idx]);
    else return static_cast<const float *>(base)[idx];
}
template <int DT>
__device__ __forceinline__ void store1(void *base, long idx, float a) {
    if constexpr (DT == 1) static_cast<uint16_t *>(base)[idx] = f2bf(a);
    else static_cast<float *>(base)[idx] = a;
}

// Gates in the bf16 paths: hardware exp2 and reciprocal (about 1 ulp each),
// well inside one bf16 rounding of the result.
__device__ __forceinline__ float sigmoidf(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float activate(int act, float x) { return act == 1 ? x * sigmoidf(x) : x; }

// DPP read of another lane of the same 16-lane row (lanes a step leaves
// unselected read 0).
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_shift(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, false));
}

// Sums of a and of b over all 64 lanes in one pass.  gfx950's
// v_permlane16_swap trades the odd 16-lane rows of its first operand for the
// even rows of its second, so adding its two results gives, lane by lane, a
// summed over rows {0,1} and {2,3} in rows 0 and 2 and b likewise in rows 1
// and 3; v_permlane32_swap of that vector with itself adds the two halves, and
// DPP finishes within each row.  The returned vector holds the total of a in
// rows 0 and 2 and the total of b in rows 1 and 3 (lanes 0 and 16 are read).
// (The swap results are copied out element by element before the bit casts:
// clang lowers __builtin_bit_cast of a vector element lvalue as a load of
// element 0.)
__device__ __forceinline__ float wave_sum_pair(float a, float b) {
    const auto s16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                      __builtin_bit_cast(unsigned, b), false, false);
    const unsigned a0 = s16[0], a1 = s16[1];
    float v = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                      __builtin_bit_cast(unsigned, v), false, false);
    const unsigned b0 = s32[0], b1 = s32[1];
    v = __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
    v += dpp_shift<0xB1>(v);          // quad_perm [1,0,3,2]
    v += dpp_shift<0x4E>(v);          // quad_perm [2,3,0,1]
    v += dpp_shift<0x141>(v);         // row_half_mirror
    v += dpp_shift<0x140>(v);         // row_mirror: every lane of a row holds its row sum
    return v;
}
__device__ __forceinline__ float lane_value(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Raw buffer resource over `bytes` bytes from `base` (gfx9 format word):
// offsets at or past `bytes` load as 0 and are dropped by stores, so a
// row-masked access is issued by every lane without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// fp32 16x16x4 MFMA (layout checked on the device): lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] of the 4-wide k step and holds
// D[4 (l / 16) + r][l % 16] in element r.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// 8 bf16 from two groups of 4 fp32 (the MFMA output rows of two 16-row tiles).
__device__ __forceinline__ bf16x8 pack8(const f32x4 &a, const f32x4 &b) {
    u32x4 w;
    w[0] = pack_bf2(a[0], a[1]);
    w[1] = pack_bf2(a[2], a[3]);
    w[2] = pack_bf2(b[0], b[1]);
    w[3] = pack_bf2(b[2], b[3]);
    return as_bf16x8(w);
}

}  // namespace kda
