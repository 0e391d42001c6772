// append.hip -- KV-cache append for gfx950.
//
// The cache write that comes before attention (`do_kv_cache_update` on the
// vLLM "b12x" backend page, which hands the new keys and values, the caches,
// `slot_mapping` and the k/v scales to `reshape_and_cache_flash`): new token i
// goes to flat slot s = slot_mapping[i], i.e. page s / P, row s % P, for every
// kv head; s < 0 marks a padding token that is not written.  A bf16 cache
// receives the bf16 rows unchanged; an e4m3fn cache receives
// e4m3fn(x / scale), the quotient an IEEE fp32 division and the conversion
// round-to-nearest-even with saturation at +-448 (NaN stays NaN).
//
// A thread moves kAppendPer<FP8> 8-element chunks (16 bytes of bf16 input each,
// 256 chunks apart so that a block's loads are contiguous) of K and the same
// chunks of V, all loads before any store, nontemporal both ways; the work is
// pure HBM traffic.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

template <typename T>
__device__ __forceinline__ u32x4 load_nt(const T* ptr) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
}
template <typename T, typename V>
__device__ __forceinline__ void store_nt(T* ptr, V val) {
    __builtin_nontemporal_store(val, reinterpret_cast<V*>(ptr));
}

// float -> OCP e4m3fn, round to nearest even, saturating (NaN -> NaN).
__device__ __forceinline__ uint32_t e4m3_encode(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;               // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;              // |f| >= 448 (incl. inf)
    if (a < 0x3c800000u) {                                   // |f| < 2^-6: subnormal codes
        const float m = __builtin_rintf(__uint_as_float(a) * 512.f);   // exact scaling, RNE
        return sign | (uint32_t)m;                           // 8 -> 0x08, the first normal
    }
    // normal: keep 3 mantissa bits, round half to even (the carry may bump
    // the exponent); e4m3 biased exponent = fp32 biased exponent - 120
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    const uint32_t code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    return sign | min(code, 0x7eu);
}

// Eight bf16 values -> eight e4m3fn codes of value / s (memory order kept).
__device__ __forceinline__ u32x2 quant8(u32x4 w, float s) {
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = e4m3_encode(bf16_lo(in[i]) / s);
        const uint32_t hi = e4m3_encode(bf16_hi(in[i]) / s);
        out[i / 2] |= (lo | (hi << 8)) << (16 * (i % 2));
    }
    return u32x2{out[0], out[1]};
}

// 8-element chunks per thread, loads issued together (fp8: 1, its division
// and encoding per element already keep the wave busy)
template <bool FP8>
constexpr int kAppendPer = FP8 ? 1 : 4;

template <bool FP8>
__global__ __launch_bounds__(256) void cache_append_kernel(AppendParams p) {
    constexpr int kPer = kAppendPer<FP8>;
    const int chunks = p.num_kv_heads * p.head_dim / 8;        // 8-element chunks per token
    const int64_t total = p.num_tokens * chunks;
    // chunk i of this thread: block base + 256 i + thread (each load
    // instruction of a block covers 256 consecutive chunks)
    const int64_t first = (int64_t)blockIdx.x * 256 * kPer + threadIdx.x;
    u32x4 k[kPer], v[kPer];
    int64_t dst[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t idx = first + 256 * i;
        dst[i] = -1;
        if (idx >= total) continue;
        const int64_t tok = idx / chunks;
        const int rem = (int)(idx - tok * chunks);
        const int h = rem / (p.head_dim / 8), c = rem % (p.head_dim / 8);
        const int64_t slot = p.slot_mapping[tok];
        if (slot < 0) continue;                                 // padding token
        const int64_t page = slot >> p.page_shift;
        const int64_t row = slot & ((1 << p.page_shift) - 1);
        const int64_t src = tok * p.row_stride + (int64_t)h * p.head_dim + 8 * c;
        k[i] = load_nt(static_cast<const uint16_t*>(p.key) + src);
        v[i] = load_nt(static_cast<const uint16_t*>(p.value) + src);
        dst[i] = page * p.s_page + row * p.s_tok + (int64_t)h * p.s_head + 8 * c;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (dst[i] < 0) continue;
        if constexpr (!FP8) {
            store_nt(static_cast<uint16_t*>(p.k_pool) + dst[i], k[i]);
            store_nt(static_cast<uint16_t*>(p.v_pool) + dst[i], v[i]);
        } else {
            store_nt(static_cast<uint8_t*>(p.k_pool) + dst[i], quant8(k[i], p.k_scale));
            store_nt(static_cast<uint8_t*>(p.v_pool) + dst[i], quant8(v[i], p.v_scale));
        }
    }
}

}  // namespace

hipError_t launch_cache_append(const AppendParams& p, bool fp8, hipStream_t stream) {
    const int64_t chunks = p.num_tokens * (p.num_kv_heads * p.head_dim / 8);
    const int per = fp8 ? kAppendPer<true> : kAppendPer<false>;
    const int64_t threads = (chunks + per - 1) / per;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (fp8)
        hipLaunchKernelGGL(cache_append_kernel<true>, dim3(blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(cache_append_kernel<false>, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
