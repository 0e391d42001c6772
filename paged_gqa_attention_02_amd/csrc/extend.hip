// extend.hip -- prefix-prefill (extend) attention for gfx950.
//
// New query tokens of a sequence attend to its cached context through the
// pages (no mask) and causally to each other (contiguous new K/V rows), with
// the same window, scale and soft-cap as decode: the two loops of `_fwd_kernel`
// on the page "vllm/attention/ops/prefix_prefill.py" (context phase, then the
// new-token phase with its causal mask), finished by the division of the
// accumulator by the softmax sum.
//
// Work: one 256-thread block per (tile of 128 rows, sequence b, kv head g).
// A row is (new token t, query head h of the group): the G heads of a kv head
// share every K/V byte the block stages.  Wave w owns rows 32w..32w+31, two
// MFMA column blocks of 16.  The block walks its key range [lo, C + t_last]
// (lo from the sliding window of its first token) in tiles of 64 keys: key
// j < C comes from page block_table[b][j / P], key j >= C is new row j - C.
// Both phases are one loop; a tile is masked only where it crosses the
// causal diagonal or the window edge.
//
// Per tile, with v_mfma_f32_16x16x32_bf16:
//   S^T[64 keys x 16 rows] = K[64 x D] Q^T[D x 16]     K read from LDS in the A
//                                                     layout, Q^T in registers
//   online softmax per row (a row is one MFMA column: 4 lanes hold its keys)
//   O^T[D x 16] += V^T[D x 64] P^T[64 x 16]          P^T is the S^T accumulator
//                                                     itself; V rows read from
//                                                     LDS are transposed in
//                                                     registers (v_perm)
// K/V tiles are staged in LDS as bf16 (fp8 context rows are converted while
// staging; the cache scales are applied per key to the score and to P), with
// two buffers: the next tile's global loads are in flight while this tile is
// computed.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kExtThreads = 256;
constexpr int kExtRows = 128;     // rows (token, head) per block
constexpr int kExtKeys = 64;      // keys per tile

// Key position (0..31) inside a 32-key step for MFMA contraction slot
// (grp, jj): the S^T accumulators of key blocks 2ks and 2ks+1 are the P^T
// operand with this order.
__device__ __forceinline__ int step_key(int grp, int jj) {
    return (jj < 4) ? 4 * grp + jj : 16 + 4 * grp + (jj - 4);
}

// Global -> register -> LDS staging of one tile of K (or V) rows as bf16.
// A thread moves kElems elements of one row per pass: 8 bf16 (16 bytes), or
// 16 elements for an fp8 cache (16 bytes of fp8 context, or 32 bytes of bf16
// new rows), written to LDS as bf16.
template <int D, bool FP8>
struct Stage {
    static constexpr int kElems = FP8 ? 16 : 8;
    static constexpr int kLanesPerRow = D / kElems;
    static constexpr int kRowsPerPass = kExtThreads / kLanesPerRow;
    static constexpr int kPasses = kExtKeys / kRowsPerPass;
    static constexpr int kPitch = 2 * D + 16;          // LDS bytes per row (padded)
    u32x4 a[kPasses], b[kPasses];                       // b: second half (fp8 layout)
    bool ctx[kPasses];
};

struct SeqInfo {
    int b, kvh, n, C, q0;       // q0 = cu_seqlens_q[b]
};

template <int D, bool FP8>
__device__ __forceinline__ void stage_load(Stage<D, FP8>& S, const ExtendParams& p,
                                           const void* pool, const void* fresh,
                                           const SeqInfo& si, int jt) {
    using ST = Stage<D, FP8>;
    constexpr int kElem = FP8 ? 1 : 2;
    const int tid = threadIdx.x;
    const int chunk = tid % ST::kLanesPerRow;
    const int pmask = (1 << p.page_shift) - 1;
    const int32_t* bt = p.block_table + (int64_t)si.b * p.bt_stride;
#pragma unroll
    for (int i = 0; i < ST::kPasses; ++i) {
        const int j = jt + i * ST::kRowsPerPass + tid / ST::kLanesPerRow;
        S.ctx[i] = j < si.C;
        S.a[i] = u32x4{0, 0, 0, 0};
        S.b[i] = u32x4{0, 0, 0, 0};
        if (j < si.C) {
            const int64_t page = bt[j >> p.page_shift];
            const uint8_t* src = static_cast<const uint8_t*>(pool) +
                                 (page * p.s_page + (int64_t)(j & pmask) * p.s_tok +
                                  (int64_t)si.kvh * p.s_head) * kElem +
                                 chunk * 16;
            S.a[i] = *reinterpret_cast<const u32x4*>(src);
        } else if (j < si.C + si.n) {
            const uint8_t* src = static_cast<const uint8_t*>(fresh) +
                                 ((int64_t)(si.q0 + j - si.C) * p.num_kv_heads + si.kvh) * D * 2 +
                                 chunk * ST::kElems * 2;
            S.a[i] = *reinterpret_cast<const u32x4*>(src);
            if constexpr (FP8) S.b[i] = *reinterpret_cast<const u32x4*>(src + 16);
        }
    }
}

template <int D, bool FP8>
__device__ __forceinline__ void stage_store(const Stage<D, FP8>& S, uint8_t* lds) {
    using ST = Stage<D, FP8>;
    const int tid = threadIdx.x;
    const int chunk = tid % ST::kLanesPerRow;
#pragma unroll
    for (int i = 0; i < ST::kPasses; ++i) {
        const int row = i * ST::kRowsPerPass + tid / ST::kLanesPerRow;
        uint8_t* dst = lds + row * ST::kPitch + chunk * ST::kElems * 2;
        if constexpr (FP8) {
            u32x4 lo = S.a[i], hi = S.b[i];
            if (S.ctx[i]) {
                const u32x2 e0 = e4m3x4_to_bf16x4(S.a[i].x), e1 = e4m3x4_to_bf16x4(S.a[i].y);
                const u32x2 e2 = e4m3x4_to_bf16x4(S.a[i].z), e3 = e4m3x4_to_bf16x4(S.a[i].w);
                lo = u32x4{e0.x, e0.y, e1.x, e1.y};
                hi = u32x4{e2.x, e2.y, e3.x, e3.y};
            }
            *reinterpret_cast<u32x4*>(dst) = lo;
            *reinterpret_cast<u32x4*>(dst + 16) = hi;
        } else {
            *reinterpret_cast<u32x4*>(dst) = S.a[i];
        }
    }
}

template <int D, bool FP8, bool CAP>
__global__ __launch_bounds__(kExtThreads, 2) void extend_kernel(ExtendParams p) {
    using ST = Stage<D, FP8>;
    constexpr int kDS = D / 32;        // QK contraction steps
    constexpr int kVE = D / 16;        // PV MFMAs per (row block, key step)
    constexpr int kPitch = ST::kPitch;
    __shared__ __attribute__((aligned(16))) uint8_t sm_k[2][kExtKeys * kPitch];
    __shared__ __attribute__((aligned(16))) uint8_t sm_v[2][kExtKeys * kPitch];

    const int G = p.group;
    const int segs = p.num_seqs * p.num_kv_heads;
    // heavier tiles (later tokens, more keys) first; all tiles of one
    // (sequence, kv head) on one XCD when segs is a multiple of 8
    const int seg = blockIdx.x % segs;
    const int mt = p.q_tiles - 1 - (int)(blockIdx.x / segs);
    SeqInfo si;
    si.b = seg / p.num_kv_heads;
    si.kvh = seg % p.num_kv_heads;
    si.q0 = p.cu_seqlens_q[si.b];
    si.n = p.cu_seqlens_q[si.b + 1] - si.q0;
    si.C = p.ctx_lens[si.b];
    const int T = kExtRows / G;        // tokens per block
    const int t0 = mt * T;
    if (t0 >= si.n) return;            // (uniform over the block)
    const int t1 = min(si.n, t0 + T);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, grp = lane >> 4;

    // ---- rows of this lane's two column blocks, and Q^T as B operands ----
    int row_t[2];
    bool row_ok[2];
    u32x4 qop[2][kDS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int r = wave * 32 + rb * 16 + c;
        row_t[rb] = t0 + r / G;
        row_ok[rb] = row_t[rb] < t1;
        const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                               ((int64_t)(si.q0 + (row_ok[rb] ? row_t[rb] : t0)) * p.num_q_heads +
                                si.kvh * G + r % G) * D;
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * ds + 8 * grp);
            qop[rb][ds] = row_ok[rb] ? v : u32x4{0, 0, 0, 0};
        }
    }

    // ---- key range ----
    const int pos_first = si.C + t0, pos_last = si.C + t1 - 1;
    const int j_lo = p.window > 0 ? max(0, pos_first - p.window + 1) : 0;
    const int j_end = pos_last + 1;
    const int jt0 = j_lo & ~(kExtKeys - 1);
    const int ntiles = (j_end - jt0 + kExtKeys - 1) / kExtKeys;

    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    f32x4 acc[2][kVE];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < kVE; ++e) acc[rb][e] = f32x4{0.f, 0.f, 0.f, 0.f};

    ST sk, sv;
    stage_load<D, FP8>(sk, p, p.k_pool, p.k_new, si, jt0);
    stage_load<D, FP8>(sv, p, p.v_pool, p.v_new, si, jt0);
    stage_store<D, FP8>(sk, sm_k[0]);
    stage_store<D, FP8>(sv, sm_v[0]);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int jt = jt0 + it * kExtKeys;
        const int buf = it & 1;
        const bool more = it + 1 < ntiles;
        if (more) {
            stage_load<D, FP8>(sk, p, p.k_pool, p.k_new, si, jt + kExtKeys);
            stage_load<D, FP8>(sv, p, p.v_pool, p.v_new, si, jt + kExtKeys);
        }
        const uint8_t* kl = sm_k[buf];
        const uint8_t* vl = sm_v[buf];

        // ---- S^T = K Q^T: s[rb][kb][j] = score of key 16kb + 4grp + j, row c ----
        f32x4 s[2][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            s[0][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            s[1][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < kDS; ++ds) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(
                    kl + (16 * kb + c) * kPitch + 64 * ds + 16 * grp);
                s[0][kb] = mfma_bf16_16x16x32(a, qop[0][ds], s[0][kb]);
                s[1][kb] = mfma_bf16_16x16x32(a, qop[1][ds], s[1][kb]);
            }
        }

        // ---- scale, cap, mask, online softmax; P^T operands ----
        const bool full = (jt + kExtKeys - 1 <= pos_first) &&
                          (p.window <= 0 || pos_last - jt < p.window);
        u32x4 pop[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int pos_q = si.C + row_t[rb];
            float sc[4][4];
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = jt + 16 * kb + 4 * grp + j;
                    const bool ctx = key < si.C;
                    float v = s[rb][kb][j];
                    if constexpr (CAP) {
                        v = p.cap_c2 - 2.f * p.cap_c2 *
                                           fast_rcp(fast_exp2(v * (ctx ? p.cap_c1_ctx : p.cap_c1)) + 1.f);
                    } else {
                        v *= ctx ? p.qk_scale2_ctx : p.qk_scale2;
                    }
                    if (!full) {
                        const bool keep = key <= pos_q && (p.window <= 0 || pos_q - key < p.window);
                        v = keep ? v : -INFINITY;
                    }
                    sc[kb][j] = v;
                    tmax = fmaxf(tmax, v);
                }
            tmax = fmaxf(tmax, shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, shfl_xor(tmax, 32));
            const float m_new = fmaxf(m[rb], tmax);
            const float ms = m_new == -INFINITY ? 0.f : m_new;   // row with no key yet
            const float alpha = fast_exp2(m[rb] - ms);
            float psum = 0.f;
            float pv[4][4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float pr = fast_exp2(sc[kb][j] - ms);
                    psum += pr;
                    const int key = jt + 16 * kb + 4 * grp + j;
                    pv[kb][j] = key < si.C ? pr * p.v_scale : pr;
                }
            l[rb] = l[rb] * alpha + psum;
            m[rb] = m_new;
#pragma unroll
            for (int e = 0; e < kVE; ++e) acc[rb][e] *= alpha;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                pop[rb][ks] = u32x4{pack_bf16x2(pv[2 * ks][0], pv[2 * ks][1]),
                                    pack_bf16x2(pv[2 * ks][2], pv[2 * ks][3]),
                                    pack_bf16x2(pv[2 * ks + 1][0], pv[2 * ks + 1][1]),
                                    pack_bf16x2(pv[2 * ks + 1][2], pv[2 * ks + 1][3])};
        }

        // ---- O^T += V^T P^T: lane c supplies d = kVE*c + e of MFMA e ----
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if constexpr (kVE == 8) {
                u32x4 vr[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    vr[jj] = *reinterpret_cast<const u32x4*>(
                        vl + (32 * ks + step_key(grp, jj)) * kPitch + 16 * c);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    const bool hi = e & 1;
                    const u32x4 a = {pick_halves(vr[0][w], vr[1][w], hi),
                                     pick_halves(vr[2][w], vr[3][w], hi),
                                     pick_halves(vr[4][w], vr[5][w], hi),
                                     pick_halves(vr[6][w], vr[7][w], hi)};
                    acc[0][e] = mfma_bf16_16x16x32(a, pop[0][ks], acc[0][e]);
                    acc[1][e] = mfma_bf16_16x16x32(a, pop[1][ks], acc[1][e]);
                }
            } else {
                u32x2 vr[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    vr[jj] = *reinterpret_cast<const u32x2*>(
                        vl + (32 * ks + step_key(grp, jj)) * kPitch + 8 * c);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int w = e >> 1;
                    const bool hi = e & 1;
                    const u32x4 a = {pick_halves(vr[0][w], vr[1][w], hi),
                                     pick_halves(vr[2][w], vr[3][w], hi),
                                     pick_halves(vr[4][w], vr[5][w], hi),
                                     pick_halves(vr[6][w], vr[7][w], hi)};
                    acc[0][e] = mfma_bf16_16x16x32(a, pop[0][ks], acc[0][e]);
                    acc[1][e] = mfma_bf16_16x16x32(a, pop[1][ks], acc[1][e]);
                }
            }
        }

        if (more) {
            stage_store<D, FP8>(sk, sm_k[buf ^ 1]);
            stage_store<D, FP8>(sv, sm_v[buf ^ 1]);
        }
        __syncthreads();
    }

    // ---- finish: O^T[d][row c] / l, d = kVE*(4grp + j) + e ----
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        float lt = l[rb] + shfl_xor(l[rb], 16);
        lt += shfl_xor(lt, 32);
        if (!row_ok[rb]) continue;
        const int r = wave * 32 + rb * 16 + c;
        uint16_t* orow = static_cast<uint16_t*>(p.out) +
                         ((int64_t)(si.q0 + row_t[rb]) * p.num_q_heads + si.kvh * G + r % G) * D;
        const float inv = 1.f / lt;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t wv[kVE / 2];
#pragma unroll
            for (int e = 0; e < kVE; e += 2)
                wv[e / 2] = pack_bf16x2(acc[rb][e][j] * inv, acc[rb][e + 1][j] * inv);
            uint16_t* dst = orow + kVE * (4 * grp + j);
            if constexpr (kVE == 8)
                *reinterpret_cast<u32x4*>(dst) = u32x4{wv[0], wv[1], wv[2], wv[3]};
            else
                *reinterpret_cast<u32x2*>(dst) = u32x2{wv[0], wv[1]};
        }
    }
}

template <int D, bool FP8>
hipError_t launch_extend_t(const ExtendParams& p, unsigned blocks, hipStream_t stream) {
    if (p.has_cap)
        hipLaunchKernelGGL((extend_kernel<D, FP8, true>), dim3(blocks), dim3(kExtThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((extend_kernel<D, FP8, false>), dim3(blocks), dim3(kExtThreads), 0,
                           stream, p);
    return hipGetLastError();
}

}  // namespace

int extend_rows_per_block() { return kExtRows; }

hipError_t launch_extend(const ExtendParams& p, int head_dim, bool fp8, int num_seqs,
                         hipStream_t stream) {
    const unsigned blocks = (unsigned)p.q_tiles * (unsigned)num_seqs * (unsigned)p.num_kv_heads;
    if (head_dim == 128)
        return fp8 ? launch_extend_t<128, true>(p, blocks, stream)
                   : launch_extend_t<128, false>(p, blocks, stream);
    return fp8 ? launch_extend_t<64, true>(p, blocks, stream)
               : launch_extend_t<64, false>(p, blocks, stream);
}

}  // namespace pa
