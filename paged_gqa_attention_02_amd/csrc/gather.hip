// gather.hip -- byte copy of every cached K/V row through the address path
// of the attention kernels (a check of the block-table gather).
#include "decode_geom.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// Copy every cached row of every sequence to a dense [sum L, Hkv, D] array
// through row_ptr (the address path of the attention kernels).
template <int D, bool FP8>
__global__ __launch_bounds__(256) void gather_kernel(GatherParams p) {
    constexpr int kRowBytes = D * (FP8 ? 1 : 2);
    constexpr int kChunks = kRowBytes / 16;
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    int64_t off = 0;
    for (int i = 0; i < b; ++i) off += p.seq_lens[i];
    const int L = p.seq_lens[b];
    const int pmask = (1 << p.page_shift) - 1;
    const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;
    for (int idx = threadIdx.x; idx < L * kChunks; idx += 256) {
        const int t = idx / kChunks, ch = idx % kChunks;
        const int64_t pg = bt_row[t >> p.page_shift];
        const int64_t dst = ((off + t) * p.num_kv_heads + kvh) * kRowBytes + 16 * ch;
        const uint8_t* ks = row_ptr<FP8>(p.k_pool, pg, t & pmask, kvh, p.s_page, p.s_tok, p.s_head);
        const uint8_t* vs = row_ptr<FP8>(p.v_pool, pg, t & pmask, kvh, p.s_page, p.s_tok, p.s_head);
        *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.k_out) + dst) =
            *reinterpret_cast<const u32x4*>(ks + 16 * ch);
        *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.v_out) + dst) =
            *reinterpret_cast<const u32x4*>(vs + 16 * ch);
    }
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, int head_dim, bool fp8, hipStream_t stream) {
    dim3 grid(p.num_kv_heads, p.num_seqs);
    if (head_dim == 128) {
        if (fp8) hipLaunchKernelGGL((gather_kernel<128, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((gather_kernel<128, false>), grid, dim3(256), 0, stream, p);
    } else {
        if (fp8) hipLaunchKernelGGL((gather_kernel<64, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((gather_kernel<64, false>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace pa
