// extend.hip -- prefix-prefill (extend) attention for gfx950.
//
// New query tokens of a sequence attend to its cached context through the
// pages (no mask) and causally to each other (contiguous new K/V rows), with
// the same window, scale and soft-cap as decode: the two loops of `_fwd_kernel`
// on the page "vllm/attention/ops/prefix_prefill.py" (context phase, then the
// new-token phase with its causal mask), finished by the division of the
// accumulator by the softmax sum.
//
// Work: one block of kExtWaves waves per (tile of kExtRows rows, sequence b,
// kv head g).  A row is (new token t, query head h of the group): the G heads
// of a kv head share every K/V byte the block stages.  Each wave owns kRB MFMA
// column blocks of 16 rows.  The block walks its key range [lo, C + t_last]
// (lo from the sliding window of its first token) in tiles of 64 keys: key
// j < C comes from page block_table[b][j / P], key j >= C is new row j - C.
// Context and new keys share the key loop; the tiles are walked in runs of
// one kind, and only the tiles that cross the causal diagonal or the window
// edge, or hold both context and new keys, take the masked per-key path.
//
// Per tile, with v_mfma_f32_16x16x32_bf16:
//   S^T[64 keys x 16 rows] = K[64 x D] Q^T[D x 16]     K read from LDS in the A
//                                                     layout, Q^T in registers
//   online softmax per row (a row is one MFMA column: 4 lanes hold its keys)
//   O^T[D x 16] += V^T[D x 64] P^T[64 x 16]          P^T is the S^T accumulator
//                                                     itself; V rows read from
//                                                     LDS are transposed in
//                                                     registers (v_perm)
// K/V tiles live in LDS as bf16 rows of 2*D bytes whose 16-byte slots are
// XOR-swizzled by the row index (slot s of row r holds chunk s ^ (r mod
// slots)), so the operand reads of 16 lanes hit 16 different bank groups.
// bf16 caches are staged with direct global->LDS loads (global_load_lds,
// lane i of a wave fills bytes 16i..16i+15 of a 1 KB run); fp8 context rows go
// through registers to be converted.  Two buffers: the next tile's loads are
// in flight while this tile is computed.  The cache scales apply per key, to
// the score (k_scale) and to P (v_scale).
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

#ifndef PA_EXTEND_WAVES
#define PA_EXTEND_WAVES 4
#endif
#ifndef PA_EXTEND_RB
#define PA_EXTEND_RB 2
#endif
#ifndef PA_EXTEND_OCCUPANCY
#define PA_EXTEND_OCCUPANCY 2
#endif
constexpr int kExtWaves = PA_EXTEND_WAVES;       // waves per block
constexpr int kRB = PA_EXTEND_RB;                // 16-row column blocks per wave
constexpr int kExtThreads = 64 * kExtWaves;
constexpr int kExtRows = 16 * kRB * kExtWaves;   // rows (token, head) per block
constexpr int kExtKeys = 64;                     // keys per tile
constexpr int kExtPages = 2048;                  // page ids staged in LDS at a time
// waves per SIMD the kernel is compiled for
constexpr int kExtOccupancy = PA_EXTEND_OCCUPANCY;

// How scores become log2-domain logits.
enum ScoreMode {
    kFold = 0,    // no cap, one positive scale per tile: max on raw scores,
                  // exp2(s*scale - m) (a positive scale commutes with the max)
    kScale = 1,   // no cap, any scale: s*scale per score
    kCap = 2,     // soft-cap c*tanh(s*scale/c), per score
};

// Key position (0..31) inside a 32-key step for MFMA contraction slot
// (grp, jj): the S^T accumulators of key blocks 2ks and 2ks+1 are the P^T
// operand with this order.
__device__ __forceinline__ int step_key(int grp, int jj) {
    return (jj < 4) ? 4 * grp + jj : 16 + 4 * grp + (jj - 4);
}

struct SeqInfo {
    int b, kvh, n, C, q0;       // q0 = cu_seqlens_q[b]
    int pg0;                    // first logical page of the staged page list
    const int* pages;           // LDS: block_table[b][pg0 .. pg0 + kExtPages)
};

// LDS tile geometry: 64 rows of 2*D bytes, 16-byte slots swizzled by row.
template <int D>
struct Tile {
    static constexpr int kPitch = 2 * D;
    static constexpr int kSlots = kPitch / 16;
    static constexpr int kBytes = kExtKeys * kPitch;
    static __device__ __forceinline__ int off(int row, int slot) {
        return row * kPitch + 16 * (slot ^ (row & (kSlots - 1)));
    }
};

// Addresses of key j's K and V rows: context rows through the staged page list
// (j < C), new rows from the contiguous k_new / v_new (bf16; keys past the
// sequence read its last new row: finite, masked by the consumer).  Both
// candidates are formed (the page-list index is clamped into the list) and
// one selected, so the address path has no branch.
template <int D, bool FP8>
__device__ __forceinline__ void key_rows(const ExtendParams& p, const SeqInfo& si, int j,
                                         const uint8_t*& k, const uint8_t*& v) {
    constexpr int kElem = FP8 ? 1 : 2;
    const int idx = min(max((j >> p.page_shift) - si.pg0, 0), kExtPages - 1);
    const int64_t page = si.pages[idx];
    const int64_t ctx = (page * p.s_page + (int64_t)(j & ((1 << p.page_shift) - 1)) * p.s_tok +
                         (int64_t)si.kvh * p.s_head) * kElem;
    const int r = min(max(j - si.C, 0), si.n - 1);
    const int64_t nw = ((int64_t)(si.q0 + r) * p.num_kv_heads + si.kvh) * D * 2;
    const bool in_ctx = j < si.C;
    k = in_ctx ? static_cast<const uint8_t*>(p.k_pool) + ctx
               : static_cast<const uint8_t*>(p.k_new) + nw;
    v = in_ctx ? static_cast<const uint8_t*>(p.v_pool) + ctx
               : static_cast<const uint8_t*>(p.v_new) + nw;
}

// bf16: one tile of K and V rows straight into LDS.  The tile is kRuns runs of
// 1 KB (kRowsPer rows); wave w issues runs w, w + kExtWaves, ...  Lane l fills
// slot l % kSlots of its row with the row's chunk (slot ^ swizzle).
template <int D>
__device__ __forceinline__ void stage_direct(const ExtendParams& p, const SeqInfo& si, int jt,
                                             uint8_t* kd, uint8_t* vd) {
    using TL = Tile<D>;
    constexpr int kRowsPer = 1024 / TL::kPitch;
    constexpr int kRuns = kExtKeys / kRowsPer;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane % TL::kSlots;
#pragma unroll
    for (int run = wave; run < kRuns; run += kExtWaves) {
        const int row = run * kRowsPer + lane / TL::kSlots;
        const uint8_t *k, *v;
        key_rows<D, false>(p, si, jt + row, k, v);
        const int chunk = 16 * (slot ^ (row & (TL::kSlots - 1)));
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(k + chunk),
            (void __attribute__((address_space(3)))*)(kd + run * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(v + chunk),
            (void __attribute__((address_space(3)))*)(vd + run * 1024), 16, 0, 0);
    }
}

// fp8: global -> registers (16 elements a thread), converted and written to
// the swizzled LDS tile as bf16.  Threads past kRowsPerPass * kLanesPerRow idle.
template <int D>
struct Stage8 {
    static constexpr int kLanesPerRow = D / 16;
    static constexpr int kRowsPerPass = kExtThreads / kLanesPerRow < kExtKeys
                                            ? kExtThreads / kLanesPerRow : kExtKeys;
    static constexpr int kPasses = kExtKeys / kRowsPerPass;
    u32x4 a[kPasses], b[kPasses];
    bool ctx[kPasses];
};

template <int D>
__device__ __forceinline__ void stage8_load(Stage8<D>& S, const ExtendParams& p,
                                            const SeqInfo& si, int jt, bool second) {
    using ST = Stage8<D>;
    if (threadIdx.x >= ST::kRowsPerPass * ST::kLanesPerRow) return;
    const int chunk = threadIdx.x % ST::kLanesPerRow;
#pragma unroll
    for (int i = 0; i < ST::kPasses; ++i) {
        const int j = jt + i * ST::kRowsPerPass + threadIdx.x / ST::kLanesPerRow;
        const uint8_t *kr, *vr;
        key_rows<D, true>(p, si, j, kr, vr);
        const uint8_t* row = second ? vr : kr;
        S.ctx[i] = j < si.C;
        if (S.ctx[i]) {
            S.a[i] = *reinterpret_cast<const u32x4*>(row + 16 * chunk);
            S.b[i] = u32x4{0, 0, 0, 0};
        } else {
            S.a[i] = *reinterpret_cast<const u32x4*>(row + 32 * chunk);
            S.b[i] = *reinterpret_cast<const u32x4*>(row + 32 * chunk + 16);
        }
    }
}

template <int D>
__device__ __forceinline__ void stage8_store(const Stage8<D>& S, uint8_t* lds) {
    using ST = Stage8<D>;
    using TL = Tile<D>;
    if (threadIdx.x >= ST::kRowsPerPass * ST::kLanesPerRow) return;
    const int chunk = threadIdx.x % ST::kLanesPerRow;
#pragma unroll
    for (int i = 0; i < ST::kPasses; ++i) {
        const int row = i * ST::kRowsPerPass + threadIdx.x / ST::kLanesPerRow;
        u32x4 lo = S.a[i], hi = S.b[i];
        if (S.ctx[i]) {
            const u32x2 e0 = e4m3x4_to_bf16x4(S.a[i].x), e1 = e4m3x4_to_bf16x4(S.a[i].y);
            const u32x2 e2 = e4m3x4_to_bf16x4(S.a[i].z), e3 = e4m3x4_to_bf16x4(S.a[i].w);
            lo = u32x4{e0.x, e0.y, e1.x, e1.y};
            hi = u32x4{e2.x, e2.y, e3.x, e3.y};
        }
        *reinterpret_cast<u32x4*>(lds + TL::off(row, 2 * chunk)) = lo;
        *reinterpret_cast<u32x4*>(lds + TL::off(row, 2 * chunk + 1)) = hi;
    }
}

// Wait for this wave's direct-to-LDS loads (vmcnt 0; expcnt and lgkmcnt
// left at their maxima).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Running state of one wave: kRB column blocks of 16 rows.
template <int D>
struct ExtAcc {
    static constexpr int kVE = D / 16;
    float m[kRB], l[kRB];
    f32x4 o[kRB][kVE];
};

// Per-lane byte offsets of the operand reads inside a swizzled tile: K row
// 16kb + c, slot 4ds + grp is at kb*16*pitch + koff[ds]; V row
// 32ks + step_key(grp, jj), slot c is at ks*32*pitch + (jj >= 4 ? 16*pitch : 0)
// + voff[jj & 3] (rows 16 apart share the swizzle).
template <int D>
struct LaneOffs {
    int koff[D / 32];
    int voff[4];
    __device__ __forceinline__ void init(int c, int grp) {
        using TL = Tile<D>;
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) koff[ds] = TL::off(c, 4 * ds + grp);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            voff[j] = (D == 128) ? TL::off(4 * grp + j, c)
                                 : TL::off(4 * grp + j, c >> 1) + 8 * (c & 1);
    }
};

// Logit (log2 domain) of a raw score for kScale / kCap.  SPLIT: the tile
// holds context and new keys, whose scales differ.
template <int MODE, bool SPLIT>
__device__ __forceinline__ float logit(float v, const ExtendParams& p, bool ctx, float qs,
                                       float c1) {
    if constexpr (MODE == kCap) {
        const float k1 = SPLIT ? (ctx ? p.cap_c1_ctx : p.cap_c1) : c1;
        return p.cap_c2 - 2.f * p.cap_c2 * fast_rcp(fast_exp2(v * k1) + 1.f);
    } else {
        return v * (SPLIT ? (ctx ? p.qk_scale2_ctx : p.qk_scale2) : qs);
    }
}

// Scale (or soft-cap), mask and online softmax of one tile's scores, then
// P^T as B operands.  MASK: the tile crosses the causal diagonal or the
// window edge; SPLIT: it holds context and new keys (per-key scales).
template <int D, int MODE, bool MASK, bool SPLIT>
__device__ __forceinline__ void tile_softmax(f32x4 (&s)[kRB][4], u32x4 (&pop)[kRB][2],
                                             ExtAcc<D>& A, const ExtendParams& p,
                                             const SeqInfo& si, const int (&pos_q)[kRB], int jt) {
    constexpr int kVE = D / 16;
    constexpr bool kFolded = MODE == kFold && !SPLIT;
    const int grp = (threadIdx.x & 63) >> 4;
    const bool all_ctx = jt + kExtKeys <= si.C;
    const float qs = all_ctx ? p.qk_scale2_ctx : p.qk_scale2;
    const float c1 = all_ctx ? p.cap_c1_ctx : p.cap_c1;
    const float vsu = all_ctx ? p.v_scale : 1.f;          // (not SPLIT)
    const int key0 = jt + 4 * grp;                          // key of s[.][kb][j]: key0 + 16kb + j
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = key0 + 16 * kb + j;
                float v = s[rb][kb][j];
                if constexpr (!kFolded)
                    v = logit<MODE == kFold ? kScale : MODE, SPLIT>(v, p, key < si.C, qs, c1);
                if constexpr (MASK) {
                    const bool keep = key <= pos_q[rb] &&
                                      (p.window <= 0 || pos_q[rb] - key < p.window);
                    v = keep ? v : -INFINITY;
                }
                s[rb][kb][j] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = col4_max(tmax);
        if constexpr (kFolded) tmax *= qs;
        // Lazy rescale: the reference max m of a row moves only when a score
        // exceeds it by more than kSlack (log2 units), so p <= 2^kSlack and
        // the accumulators are rescaled rarely (for every row of the wave at
        // once, each by its own factor).
        constexpr float kSlack = 8.f;
        const bool move = __any(tmax > A.m[rb] + kSlack);
        const float m_new = move ? fmaxf(A.m[rb], tmax) : A.m[rb];
        const float ms = m_new == -INFINITY ? 0.f : m_new;   // row with no key yet
        const float alpha = fast_exp2(A.m[rb] - ms);
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float pr;
                if constexpr (kFolded) pr = fast_exp2(__builtin_fmaf(s[rb][kb][j], qs, -ms));
                else pr = fast_exp2(s[rb][kb][j] - ms);
                psum += pr;
                if constexpr (SPLIT)
                    s[rb][kb][j] = key0 + 16 * kb + j < si.C ? pr * p.v_scale : pr;
                else
                    s[rb][kb][j] = pr;
            }
        if constexpr (!SPLIT) {
            if (vsu != 1.f) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) s[rb][kb][j] *= vsu;
            }
        }
        A.l[rb] = A.l[rb] * alpha + psum;
        A.m[rb] = m_new;
        if (move) {
#pragma unroll
            for (int e = 0; e < kVE; ++e) A.o[rb][e] *= alpha;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            pop[rb][ks] = u32x4{pack_bf16x2(s[rb][2 * ks][0], s[rb][2 * ks][1]),
                                pack_bf16x2(s[rb][2 * ks][2], s[rb][2 * ks][3]),
                                pack_bf16x2(s[rb][2 * ks + 1][0], s[rb][2 * ks + 1][1]),
                                pack_bf16x2(s[rb][2 * ks + 1][2], s[rb][2 * ks + 1][3])};
    }
}

// One tile of 64 keys starting at jt, K and V in the swizzled LDS tiles.
// FAST: the tile needs no mask and holds one kind of key (context or new).
template <int D, int MODE, bool FAST>
__device__ __forceinline__ void tile_compute(const uint8_t* kl, const uint8_t* vl,
                                             const LaneOffs<D>& lo,
                                             const u32x4 (&qop)[kRB][D / 32], ExtAcc<D>& A,
                                             const ExtendParams& p, const SeqInfo& si,
                                             const int (&pos_q)[kRB], int pos_first,
                                             int pos_last, int jt) {
    constexpr int kPitch = Tile<D>::kPitch;
    constexpr int kDS = D / 32;
    constexpr int kVE = D / 16;

    // ---- S^T = K Q^T: s[rb][kb][j] = score of key 16kb + 4grp + j, row c ----
    f32x4 s[kRB][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) {
            const u32x4 a =
                *reinterpret_cast<const u32x4*>(kl + kb * 16 * kPitch + lo.koff[ds]);
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
                s[rb][kb] = mfma_bf16_16x16x32(a, qop[rb][ds], s[rb][kb]);
        }
    }

    // ---- scale / cap, mask, online softmax; P^T operands ----
    (void)pos_first;
    (void)pos_last;
    u32x4 pop[kRB][2];
    tile_softmax<D, MODE, !FAST, !FAST>(s, pop, A, p, si, pos_q, jt);

    // ---- O^T += V^T P^T: lane c supplies d = kVE*c + e of MFMA e.  V rows
    // are read in 8-byte quarters of 4 elements (D = 128: d 8c..8c+3, then
    // 8c+4..8c+7; D = 64: d 4c..4c+3) ----
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int half = 0; half < kVE / 4; ++half) {
            u32x2 vr[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                vr[jj] = *reinterpret_cast<const u32x2*>(
                    vl + ks * 32 * kPitch + (jj >= 4 ? 16 * kPitch : 0) + lo.voff[jj & 3] +
                    8 * half);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int w = e2 >> 1, e = 4 * half + e2;
                const bool hi = e2 & 1;
                const u32x4 a = {pick_halves(vr[0][w], vr[1][w], hi),
                                 pick_halves(vr[2][w], vr[3][w], hi),
                                 pick_halves(vr[4][w], vr[5][w], hi),
                                 pick_halves(vr[6][w], vr[7][w], hi)};
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb)
                    A.o[rb][e] = mfma_bf16_16x16x32(a, pop[rb][ks], A.o[rb][e]);
            }
        }
    }
}

template <int D, bool FP8, int MODE>
__global__ __launch_bounds__(kExtThreads, kExtOccupancy) void extend_kernel(ExtendParams pk) {
    using TL = Tile<D>;
    constexpr int kDS = D / 32;        // QK contraction steps
    constexpr int kVE = D / 16;        // PV MFMAs per (row block, key step)
    // two buffers of K and V (tile `it` in buffer it & 1)
    __shared__ __attribute__((aligned(1024))) uint8_t sm_k0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_v0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_k1[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_v1[TL::kBytes];
    __shared__ int sm_pages[kExtPages];

    ExtendParams p = pk;
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
    // per-request descales of the cached part (uniform loads)
    if (p.k_desc) {
        const float kd = p.k_desc[p.desc_per_seq ? si.b : 0];
        p.qk_scale2_ctx *= kd;
        p.cap_c1_ctx *= kd;
    }
    if (p.v_desc) p.v_scale *= p.v_desc[p.desc_per_seq ? si.b : 0];
    const int T = kExtRows / G;        // tokens per block
    const int t0 = mt * T;
    if (t0 >= si.n) return;            // (uniform over the block)
    const int t1 = min(si.n, t0 + T);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, grp = lane >> 4;

    // ---- rows of this lane's column blocks, and Q^T as B operands ----
    int row_t[kRB], pos_q[kRB];
    bool row_ok[kRB];
    u32x4 qop[kRB][kDS];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const int r = (wave * kRB + rb) * 16 + c;
        row_t[rb] = t0 + r / G;
        row_ok[rb] = row_t[rb] < t1;
        pos_q[rb] = si.C + row_t[rb];
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
    const int jt0 = j_lo & ~(kExtKeys - 1);
    const int ntiles = (pos_last + 1 - jt0 + kExtKeys - 1) / kExtKeys;

    // Context page ids in LDS, kExtPages at a time: `need(jt)` reloads the list
    // (between barriers) when tile jt's context keys are not all in it.
    si.pages = sm_pages;
    si.pg0 = -kExtPages;
    auto need = [&](int jt) {
        const int last = min(jt + kExtKeys, si.C) - 1;          // last context key
        if (last < jt) return;                                 // no context keys
        if ((last >> p.page_shift) - si.pg0 < kExtPages && (jt >> p.page_shift) >= si.pg0)
            return;
        __syncthreads();                                       // old list unused
        si.pg0 = jt >> p.page_shift;
        const int cnt = min(kExtPages, ((si.C - 1) >> p.page_shift) - si.pg0 + 1);
        const int32_t* row = p.block_table + (int64_t)si.b * p.bt_stride + si.pg0;
        for (int i = threadIdx.x; i < cnt; i += kExtThreads) sm_pages[i] = row[i];
        __syncthreads();
    };

    LaneOffs<D> lo;
    lo.init(c, grp);
    ExtAcc<D> A;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        A.m[rb] = -INFINITY;
        A.l[rb] = 0.f;
#pragma unroll
        for (int e = 0; e < kVE; ++e) A.o[rb][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- the tiles, in phases of one kind: tiles [it_win, it_diag) need no
    // mask (inside every row's window and below every row's diagonal); the
    // tile holding key C mixes context and new keys.  A phase of full
    // single-kind tiles runs the FAST variant, the others the general one;
    // each phase is its own loop. ----
    const int nd = pos_first - (kExtKeys - 1) - jt0;     // tiles it <= nd/64 end at or
    const int it_diag = nd < 0 ? 0 : nd / kExtKeys + 1;   // before the first row's diagonal
    const int it_win = p.window > 0 ? max(0, (pos_last - p.window + 1 - jt0 + kExtKeys - 1) /
                                                 kExtKeys)
                                    : 0;
    const int it_split = (si.C % kExtKeys != 0 && si.C > jt0) ? (si.C - jt0) / kExtKeys : -1;
    int cut[6] = {0, min(it_win, ntiles), 0, 0, min(max(it_diag, it_win), ntiles), ntiles};
    cut[2] = (it_split >= cut[1] && it_split < cut[4]) ? it_split : cut[4];
    cut[3] = (it_split >= cut[1] && it_split < cut[4]) ? it_split + 1 : cut[4];
    // phases: [cut0,cut1) general, [cut1,cut2) fast, [cut2,cut3) general (split),
    //         [cut3,cut4) fast, [cut4,cut5) general

    if constexpr (!FP8) {
        auto stage = [&](int jt, uint8_t* kd, uint8_t* vd) {
            need(jt);
            stage_direct<D>(p, si, jt, kd, vd);
        };
        auto run = [&](int from, int to, auto fast) {
            for (int it = from; it < to; ++it) {
                const int jt = jt0 + it * kExtKeys;
                uint8_t* kc = (it & 1) ? sm_k1 : sm_k0;
                uint8_t* vc = (it & 1) ? sm_v1 : sm_v0;
                if (it + 1 < ntiles) stage(jt + kExtKeys, (it & 1) ? sm_k0 : sm_k1,
                                           (it & 1) ? sm_v0 : sm_v1);
                tile_compute<D, MODE, decltype(fast)::value>(kc, vc, lo, qop, A, p, si, pos_q,
                                                             pos_first, pos_last, jt);
                wait_vm0();
                __syncthreads();
            }
        };
        stage(jt0, sm_k0, sm_v0);
        wait_vm0();
        __syncthreads();
        run(cut[0], cut[1], std::false_type{});
        run(cut[1], cut[2], std::true_type{});
        run(cut[2], cut[3], std::false_type{});
        run(cut[3], cut[4], std::true_type{});
        run(cut[4], cut[5], std::false_type{});
    } else {
        Stage8<D> sk, sv;
        auto load = [&](int jt) {
            need(jt);
            stage8_load<D>(sk, p, si, jt, false);
            stage8_load<D>(sv, p, si, jt, true);
        };
        auto store = [&](uint8_t* kd, uint8_t* vd) {
            stage8_store<D>(sk, kd);
            stage8_store<D>(sv, vd);
        };
        auto run = [&](int from, int to, auto fast) {
            for (int it = from; it < to; ++it) {
                const int jt = jt0 + it * kExtKeys;
                const bool more = it + 1 < ntiles;
                if (more) load(jt + kExtKeys);
                tile_compute<D, MODE, decltype(fast)::value>((it & 1) ? sm_k1 : sm_k0,
                                                             (it & 1) ? sm_v1 : sm_v0, lo, qop,
                                                             A, p, si, pos_q, pos_first,
                                                             pos_last, jt);
                if (more) store((it & 1) ? sm_k0 : sm_k1, (it & 1) ? sm_v0 : sm_v1);
                __syncthreads();
            }
        };
        load(jt0);
        store(sm_k0, sm_v0);
        __syncthreads();
        run(cut[0], cut[1], std::false_type{});
        run(cut[1], cut[2], std::true_type{});
        run(cut[2], cut[3], std::false_type{});
        run(cut[3], cut[4], std::true_type{});
        run(cut[4], cut[5], std::false_type{});
    }

    // ---- finish: O^T[d][row c] / l, d = kVE*(4grp + j) + e ----
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const float lt = col4_sum(A.l[rb]);
        if (!row_ok[rb]) continue;
        const int r = (wave * kRB + rb) * 16 + c;
        uint16_t* orow = static_cast<uint16_t*>(p.out) +
                         ((int64_t)(si.q0 + row_t[rb]) * p.num_q_heads + si.kvh * G + r % G) * D;
        // a sink logit joins the normaliser (no value row)
        float den = lt;
        if (p.sinks) den += fast_exp2(p.sinks[si.kvh * G + r % G] * kLog2e - A.m[rb]);
        const float inv = 1.f / den;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t wv[kVE / 2];
#pragma unroll
            for (int e = 0; e < kVE; e += 2)
                wv[e / 2] = pack_bf16x2(A.o[rb][e][j] * inv, A.o[rb][e + 1][j] * inv);
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
    const bool fold = !p.has_cap && p.qk_scale2 > 0.f && p.qk_scale2_ctx > 0.f;
    if (p.has_cap)
        hipLaunchKernelGGL((extend_kernel<D, FP8, kCap>), dim3(blocks), dim3(kExtThreads), 0,
                           stream, p);
    else if (fold)
        hipLaunchKernelGGL((extend_kernel<D, FP8, kFold>), dim3(blocks), dim3(kExtThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((extend_kernel<D, FP8, kScale>), dim3(blocks), dim3(kExtThreads), 0,
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
