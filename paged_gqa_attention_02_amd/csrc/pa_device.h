// pa_device.h -- device-side building blocks for the gfx950 (CDNA4) kernels.
//
// Wave64 throughout.  MFMA operand layout of v_mfma_f32_16x16x32_bf16 (one
// wave computes D[16x16] += A[16x32] * B[32x16]):
//   A: lane l holds A[l % 16][8*(l/16) + j], j = 0..7   (8 bf16 = 4 dwords)
//   B: lane l holds B[8*(l/16) + j][l % 16], j = 0..7
//   D: lane l holds D[4*(l/16) + j][l % 16], j = 0..3   (4 fp32)
// The contraction index k = 8*(l/16) + j is shared by A and B, so any
// bijection between (l/16, j) and the logical contraction index may be used
// as long as both operands use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(16))) float f32x16;

// v_mfma_f32_32x32x16_bf16 (one wave computes D[32x32] += A[32x16] * B[16x32]):
//   A: lane l holds A[l % 32][8*(l/32) + j], j = 0..7
//   B: lane l holds B[8*(l/32) + j][l % 32], j = 0..7
//   D: lane l holds D[8*(j/4) + 4*(l/32) + j%4][l % 32], j = 0..15
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four OCP e4m3fn bytes -> four bf16 (exact: every e4m3fn value is a bf16).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
    bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
    bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Select the low (sel_hi = false) or high 16-bit halves of two dwords:
// result = half(a) | half(b) << 16.
__device__ __forceinline__ uint32_t pick_halves(uint32_t a, uint32_t b, bool sel_hi) {
    return __builtin_amdgcn_perm(b, a, sel_hi ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (one MFMA column), with
// the gfx950 lane swaps: permlane32_swap(v, v) leaves v's two 32-lane halves
// in its two results, permlane16_swap(v, v) the two 16-lane rows of each
// pair; combining the two results of each step reduces over the pair.
__device__ __forceinline__ float col4_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Max / sum over the lane pair l, l^32 (one column of a 32x32 MFMA result).
__device__ __forceinline__ float pair_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

__device__ __forceinline__ float col4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Copy of n page ids from global memory to LDS by `threads` threads (thread
// t takes entries t, t + threads, ...).  Each thread issues kInFlight loads
// before it stores any, so the copy waits on memory about
// n / (threads * kInFlight) times rather than n / threads (pages of one
// token make a chunk's list thousands of ids long).
template <int kInFlight>
__device__ __forceinline__ void copy_ids_to_lds(int* dst, const int32_t* src, int n, int t,
                                                int threads) {
    for (int i0 = t; i0 < n; i0 += kInFlight * threads) {
        int v[kInFlight];
        // (an index past the list reads its last entry: no branch between
        // the loads, and nothing read outside the list)
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) v[u] = src[min(i0 + u * threads, n - 1)];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const int i = i0 + u * threads;
            if (i < n) dst[i] = v[u];
        }
    }
}

}  // namespace pa
