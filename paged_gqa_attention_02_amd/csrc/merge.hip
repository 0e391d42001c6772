// merge.hip -- the merge pass of split-KV paged decode for gfx950.
#include "decode_geom.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// ---------------------------------------------------------------------------
// Merge: one block per (segment, group of `per_block` rows; a row is a
// (query token, query head) of the kv head).  Segments
// inside one wave's range were written by the split pass; the others are
// combined here from the partials of the waves w0..w1 that cover them, per
// query-head row r,
//   out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M)    (`_fwd_kernel_stage2`).
// Wave w0's piece sits in the slot its record names, every later wave's in
// slot 0 (its range starts inside the segment).  An item is (row r, column
// quad q); the block's threads are items x kR piece lanes.  A thread folds
// the pieces pl, pl + kR, ... of its item into a running (max, sum, acc) --
// the log-sum-exp values and the partial rows of a batch of pieces are loaded
// in one round -- and the kR piece lanes are combined through LDS.
// Sequences with no keys get zero rows.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeParams p,
                                                                     int per_block) {
    constexpr int kQ = D / 4;                // column quads per row
    constexpr int kBatch = 4;                // pieces in flight per thread
    const int G = p.group;
    const int groups = p.rows / per_block;   // blocks per segment
    const int items = per_block * kQ;        // <= kMergeThreads (the launch caps per_block)
    const int kR = kMergeThreads / items;    // piece lanes
    // (rows not a power of two: the threads past kR * items only join the barrier)
    const bool idle = (int)threadIdx.x >= kR * items;
    const int seg = blockIdx.x / groups;
    const int kvh = seg % p.num_kv_heads;
    const int b = seg / p.num_kv_heads;
    const int it = threadIdx.x % items, pl = threadIdx.x / items;
    // row r of the segment: query token r / G, head kvh*G + r % G
    const int r = (blockIdx.x % groups) * per_block + it / kQ, q = it % kQ;
    const int L = p.seq_lens[b];
    const int4 rec = *reinterpret_cast<const int4*>(p.seg_rec + 4 * (int64_t)seg);
    // row r, columns 4q..4q+3 of out
    uint16_t* out = static_cast<uint16_t*>(p.out) + (int64_t)b * p.out_stride_b +
                    (int64_t)(r / G) * p.out_stride_t + (int64_t)(kvh * G + r % G) * D + 4 * q;
    if (L <= 0) {
        if (pl == 0) *reinterpret_cast<u32x2*>(out) = u32x2{0u, 0u};
        return;
    }
    const int w0 = rec.x, npieces = rec.y - rec.x + 1;
    if (npieces == 1) return;                // written whole by one wave

    float m = -INFINITY, sum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = idle ? npieces : pl; i0 < npieces; i0 += kR * kBatch) {
        float lse[kBatch];
        f32x4 o[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + kR * u;
            lse[u] = -INFINITY;
            o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i < npieces) {
                const int64_t row = part_row(p, w0 + i, i == 0 ? rec.z : 0) + r;
                lse[u] = p.part_lse[row];
                o[u] = *reinterpret_cast<const f32x4*>(p.part_o + row * D + 4 * q);
            }
        }
        float bm = lse[0];
#pragma unroll
        for (int u = 1; u < kBatch; ++u) bm = fmaxf(bm, lse[u]);
        if (bm == -INFINITY) continue;
        const float mn = fmaxf(m, bm);
        const float f = m == -INFINITY ? 0.f : fast_exp2(m - mn);
        sum *= f;
        acc *= f;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            // (an empty wave range leaves lse = -inf and no partial row)
            if (lse[u] == -INFINITY) continue;
            const float w = fast_exp2(lse[u] - mn);
            sum += w;
            acc += w * o[u];
        }
        m = mn;
    }

    if (kR > 1) {
        __shared__ float sm_m[kMergeThreads], sm_s[kMergeThreads];
        __shared__ f32x4 sm_acc[kMergeThreads];
        sm_m[threadIdx.x] = m;
        sm_s[threadIdx.x] = sum;
        sm_acc[threadIdx.x] = acc;
        __syncthreads();
        if (pl != 0) return;
        float M = m;
        for (int j = 1; j < kR; ++j) M = fmaxf(M, sm_m[j * items + it]);
        float S = 0.f;
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < kR; ++j) {
            const float mj = sm_m[j * items + it];
            if (mj == -INFINITY) continue;
            const float f = fast_exp2(mj - M);
            S += f * sm_s[j * items + it];
            a += f * sm_acc[j * items + it];
        }
        sum = S;
        acc = a;
        m = M;
    }
    if (pl != 0) return;                     // (idle threads when kR == 1)
    // a sink logit joins the normaliser once (no value row)
    if (p.sinks && sum > 0.f) sum += fast_exp2(p.sinks[kvh * G + r % G] * kLog2e - m);
    const float inv = sum > 0.f ? 1.f / sum : 0.f;   // (a row with no key: zeros)
    *reinterpret_cast<u32x2*>(out) =
        u32x2{pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv)};
}

}  // namespace

hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, int B, int Hkv,
                               hipStream_t stream) {
    // Rows of a segment per block: all of them when there are enough segments
    // for two blocks per compute unit, a divisor of them (more blocks, more
    // piece lanes each) otherwise.  (A floor of 512 blocks was about 0.8 us
    // faster than 1024 at 512 segments of 4 rows; 2048 was slower.)
    const int64_t segs = (int64_t)B * Hkv;
    // at most kMergeThreads / (D/4) rows per block (8 for D = 128, 2 for 512)
    const int max_rows = kMergeThreads / (head_dim / 4);
    int per_block = p.rows;
    while (per_block > max_rows || p.rows % per_block) --per_block;
    while (per_block % 2 == 0 && segs * (p.rows / per_block) < 512) per_block /= 2;
    dim3 grid((unsigned)(segs * (p.rows / per_block)));
    switch (head_dim) {
        case 64:
            hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(kMergeThreads), 0, stream, p,
                               per_block);
            break;
        case 128:
            hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(kMergeThreads), 0, stream, p,
                               per_block);
            break;
        case 256:       // latent-cache values
            hipLaunchKernelGGL(decode_merge_kernel<256>, grid, dim3(kMergeThreads), 0, stream, p,
                               per_block);
            break;
        case 512:
            hipLaunchKernelGGL(decode_merge_kernel<512>, grid, dim3(kMergeThreads), 0, stream, p,
                               per_block);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pa
