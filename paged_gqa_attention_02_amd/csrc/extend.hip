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
    kAlibi = 4,   // flag on kScale / kCap: plus slope * (key - query position)
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
    // V tiles: slot s of row r is stored at slot s ^ vswz(r), so the four
    // rows a 16-lane transposing read takes (4 consecutive keys, 32 bytes
    // each) fall on four different 32-byte bank groups.
    static __device__ __forceinline__ int vswz(int row) { return 2 * (row & 3); }
    static __device__ __forceinline__ int voff(int row, int slot) {
        return row * kPitch + 16 * (slot ^ vswz(row));
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
        const int kchunk = 16 * (slot ^ (row & (TL::kSlots - 1)));
        const int vchunk = 16 * (slot ^ TL::vswz(row));
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(k + kchunk),
            (void __attribute__((address_space(3)))*)(kd + run * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(v + vchunk),
            (void __attribute__((address_space(3)))*)(vd + run * 1024), 16, 0, 0);
    }
}

// bf16 with page size >= 16: a run (kRowsPer rows) never crosses a page, so
// each run takes one wave-uniform base address (its page from the staged
// list, or its first new row) and every lane a fixed offset: its row within
// the run times the row stride, plus its swizzled chunk (the swizzle of the
// rows a wave stages does not change from run to run).  A run that holds
// both context and new keys, or new rows past the sequence, takes the
// per-lane path above.
template <int D>
struct StageLane {
    uint32_t ctx_off, new_off;       // K
    uint32_t vctx_off, vnew_off;     // V (its own swizzle)
    __device__ __forceinline__ void init(const ExtendParams& p) {
        using TL = Tile<D>;
        constexpr int kRowsPer = 1024 / TL::kPitch;
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int slot = lane % TL::kSlots;
        const int row = wave * kRowsPer + lane / TL::kSlots;   // its first run's row
        const uint32_t kchunk = 16 * (slot ^ (row & (TL::kSlots - 1)));
        const uint32_t vchunk = 16 * (slot ^ TL::vswz(row));
        const uint32_t ctx_row = (uint32_t)(lane / TL::kSlots) * (uint32_t)(p.s_tok * 2);
        const uint32_t new_row = (uint32_t)(lane / TL::kSlots) * (uint32_t)(p.num_kv_heads * D * 2);
        ctx_off = ctx_row + kchunk;
        new_off = new_row + kchunk;
        vctx_off = ctx_row + vchunk;
        vnew_off = new_row + vchunk;
    }
};

template <int D>
__device__ __forceinline__ void stage_runs(const ExtendParams& p, const SeqInfo& si, int jt,
                                           uint8_t* kd, uint8_t* vd, const StageLane<D>& sl) {
    using TL = Tile<D>;
    constexpr int kRowsPer = 1024 / TL::kPitch;
    constexpr int kRuns = kExtKeys / kRowsPer;
    constexpr int kPer = kRuns / kExtWaves;                  // runs per wave
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pmask = (1 << p.page_shift) - 1;
    // the runs' page ids first (one wait for all of them)
    int pg[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int j0 = jt + (wave + k * kExtWaves) * kRowsPer;
        const int idx = min(max((j0 >> p.page_shift) - si.pg0, 0), kExtPages - 1);
        pg[k] = si.pages[idx];
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int run = wave + k * kExtWaves;
        const int j0 = jt + run * kRowsPer;                  // the run's first key
        const uint8_t *kb, *vb;
        uint32_t off, voff;
        if (j0 + kRowsPer <= si.C) {
            const int64_t page = __builtin_amdgcn_readfirstlane(pg[k]);
            const int64_t o = (page * p.s_page + (int64_t)(j0 & pmask) * p.s_tok +
                               (int64_t)si.kvh * p.s_head) * 2;
            kb = static_cast<const uint8_t*>(p.k_pool) + o;
            vb = static_cast<const uint8_t*>(p.v_pool) + o;
            off = sl.ctx_off;
            voff = sl.vctx_off;
        } else if (j0 >= si.C && j0 + kRowsPer <= si.C + si.n) {
            const int64_t o = ((int64_t)(si.q0 + j0 - si.C) * p.num_kv_heads + si.kvh) * D * 2;
            kb = static_cast<const uint8_t*>(p.k_new) + o;
            vb = static_cast<const uint8_t*>(p.v_new) + o;
            off = sl.new_off;
            voff = sl.vnew_off;
        } else {
            const int lane = threadIdx.x & 63;
            const int row = run * kRowsPer + lane / TL::kSlots;
            key_rows<D, false>(p, si, jt + row, kb, vb);
            off = 16 * ((lane % TL::kSlots) ^ (row & (TL::kSlots - 1)));
            voff = 16 * ((lane % TL::kSlots) ^ TL::vswz(row));
        }
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(kb + off),
            (void __attribute__((address_space(3)))*)(kd + run * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(vb + voff),
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

template <int D, bool V>
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
        const int o0 = V ? TL::voff(row, 2 * chunk) : TL::off(row, 2 * chunk);
        const int o1 = V ? TL::voff(row, 2 * chunk + 1) : TL::off(row, 2 * chunk + 1);
        *reinterpret_cast<u32x4*>(lds + o0) = lo;
        *reinterpret_cast<u32x4*>(lds + o1) = hi;
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

// Per-lane byte offsets of the operand reads inside a swizzled tile.
//   K: row 16kb + c, slot 4ds + grp is at kb*16*pitch + koff[ds].
//   V: transposing reads (ds_read_b64_tr_b16: within each 16 lanes, lane i
//      receives element e from the 8 bytes lane 4e + i/4 read, element i % 4).
//      Lane (grp, s = 4e + q) reads key row 32ks + 16h + 4grp + e, elements
//      16*dblk + 4q .. +3, at ks*32*pitch + h*16*pitch + vtr[dblk]; lane i
//      then holds d = 16*dblk + i of keys 32ks + 16h + 4grp + 0..3, the A
//      operand of O^T += V^T P^T in the step_key order.
template <int D>
struct LaneOffs {
    int koff[D / 32];
    int vtr[D / 16];
    __device__ __forceinline__ void init(int c, int grp) {
        using TL = Tile<D>;
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) koff[ds] = TL::off(c, 4 * ds + grp);
        const int e = c >> 2, q = c & 3;
        const int row = 4 * grp + e;                    // (+ 32ks + 16h: same swizzle)
#pragma unroll
        for (int dblk = 0; dblk < D / 16; ++dblk)
            vtr[dblk] = TL::voff(row, 2 * dblk + (q >> 1)) + 8 * (q & 1);
    }
};

// LDS byte address (32 bits) of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Eight transposing reads issued together and waited for inside one asm
// block, so every output is complete when the block ends.  Through the
// builtin the compiler has no alias information for these reads, and it
// waits for every direct-to-LDS load in flight before them -- here the next
// tile's loads into the other buffer, which P*V of this tile does not need.
// Nothing writes the bytes read: this tile's loads completed before the
// barrier that precedes its reads.
__device__ __forceinline__ void lds_read_tr16_x8(u32x2 (&out)[8], const uint32_t (&a)[8]) {
    uint64_t r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6),
          "=&v"(r7)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7])
        : "memory");
    out[0] = __builtin_bit_cast(u32x2, r0);
    out[1] = __builtin_bit_cast(u32x2, r1);
    out[2] = __builtin_bit_cast(u32x2, r2);
    out[3] = __builtin_bit_cast(u32x2, r3);
    out[4] = __builtin_bit_cast(u32x2, r4);
    out[5] = __builtin_bit_cast(u32x2, r5);
    out[6] = __builtin_bit_cast(u32x2, r6);
    out[7] = __builtin_bit_cast(u32x2, r7);
}

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
                                             const SeqInfo& si, const int (&pos_q)[kRB],
                                             const float (&al2)[kRB], int jt) {
    constexpr int kVE = D / 16;
    constexpr int kBase = MODE & 3;
    constexpr bool kAl = (MODE & kAlibi) != 0;
    constexpr bool kFolded = kBase == kFold && !SPLIT;
    static_assert(!(kAl && kBase == kFold), "ALiBi takes the per-score path");
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
                    v = logit<kBase == kFold ? kScale : kBase, SPLIT>(v, p, key < si.C, qs, c1);
                if constexpr (kAl) v += al2[rb] * (float)(key - pos_q[rb]);
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
                                             const int (&pos_q)[kRB], const float (&al2)[kRB],
                                             int jt) {
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
    u32x4 pop[kRB][2];
    tile_softmax<D, MODE, !FAST, !FAST>(s, pop, A, p, si, pos_q, al2, jt);

    // ---- O^T += V^T P^T: MFMA dblk covers d = 16*dblk .. +15; its A operand
    // (V^T rows d, keys in step_key order) comes from two transposing reads,
    // four blocks' reads at a time ----
    const uint32_t vb = lds_addr(vl);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int d0 = 0; d0 < kVE; d0 += 4) {
            uint32_t ad[8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ad[2 * u] = vb + ks * 32 * kPitch + lo.vtr[d0 + u];
                ad[2 * u + 1] = ad[2 * u] + 16 * kPitch;
            }
            u32x2 v[8];
            lds_read_tr16_x8(v, ad);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4 a = {v[2 * u].x, v[2 * u].y, v[2 * u + 1].x, v[2 * u + 1].y};
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb)
                    A.o[rb][d0 + u] = mfma_bf16_16x16x32(a, pop[rb][ks], A.o[rb][d0 + u]);
            }
        }
    }
}

// An item: row tile mt (kExtRows rows (token, head)) of sequence b, kv head
// kvh, and the key tiles [jt0, jt0 + 64 * ntiles) its rows attend (from the
// window start of its first token to its last token).  Items are numbered
// i = (b * Hkv + kvh) * q_tiles + mt, so the row tiles of one (sequence, kv
// head), which read the same keys, are neighbours; ntiles = 0 for a row tile
// past the sequence's new tokens.
struct Item {
    int b, kvh, mt, q0, n, C, t0, t1, jt0, ntiles;
};

__device__ __forceinline__ Item item_of(const ExtendParams& p, int64_t i) {
    Item it;
    it.mt = (int)(i % p.q_tiles);
    const int seg = (int)(i / p.q_tiles);
    it.kvh = seg % p.num_kv_heads;
    it.b = seg / p.num_kv_heads;
    it.q0 = p.cu_seqlens_q[it.b];
    it.n = p.cu_seqlens_q[it.b + 1] - it.q0;
    it.C = p.ctx_lens[it.b];
    const int T = kExtRows / p.group;                // tokens per row tile
    it.t0 = it.mt * T;
    it.t1 = min(it.n, it.t0 + T);
    it.jt0 = 0;
    it.ntiles = 0;
    if (it.t0 < it.n) {
        const int pos_first = it.C + it.t0, pos_last = it.C + it.t1 - 1;
        const int j_lo = p.window > 0 ? max(0, pos_first - p.window + 1) : 0;
        it.jt0 = j_lo & ~(kExtKeys - 1);
        it.ntiles = (pos_last + 1 - it.jt0 + kExtKeys - 1) / kExtKeys;
    }
    return it;
}

__device__ __forceinline__ int64_t ext_items(const ExtendParams& p) {
    return (int64_t)p.num_seqs * p.num_kv_heads * p.q_tiles;
}

// Partial row r of slot `slot` of persistent block w.
__device__ __forceinline__ int64_t ext_part_row(int64_t w, int slot, int r) {
    return (w * 2 + slot) * kExtRows + r;
}

// ---------------------------------------------------------------------------
// Tile prefix over the items: pfx[i] = key tiles of items 0..i-1 (one block).
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void extend_scan_kernel(ExtendParams p) {
    __shared__ int64_t sm_sum[kScanThreads / 64];
    const int64_t items = ext_items(p);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int64_t base = 0;
    if (threadIdx.x == 0) p.pfx[0] = 0;
    for (int64_t c0 = 0; c0 < items; c0 += kScanThreads) {
        const int64_t i = c0 + threadIdx.x;
        int v = i < items ? item_of(p, i).ntiles : 0;       // < 2^24 each
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(v, d, 64);
            if (lane >= d) v += u;
        }
        if (lane == 63) sm_sum[wv] = v;
        __syncthreads();
        int64_t off = 0, total = 0;
        for (int k = 0; k < kScanThreads / 64; ++k) {
            off += k < wv ? sm_sum[k] : 0;
            total += sm_sum[k];
        }
        if (i < items) p.pfx[i + 1] = base + off + v;
        base += total;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// One piece: key tiles [from, to) of item `it`, computed by the whole block.
// A complete piece (all tiles of the item) writes bf16 rows of `out`; a part
// writes normalised fp32 rows and their log2-sum-exp to the block's slot.
// ---------------------------------------------------------------------------
struct ExtLds {
    uint8_t *k0, *v0, *k1, *v1;
    int* pages;
};

template <int D, bool FP8, int MODE>
__device__ __forceinline__ void extend_piece(const ExtendParams& pk, const Item& it, int from,
                                             int to, bool complete, int64_t w, int slot,
                                             const ExtLds& L) {
    constexpr int kDS = D / 32;        // QK contraction steps
    constexpr int kVE = D / 16;        // PV MFMAs per (row block, key step)
    ExtendParams p = pk;
    const int G = p.group;
    SeqInfo si;
    si.b = it.b;
    si.kvh = it.kvh;
    si.q0 = it.q0;
    si.n = it.n;
    si.C = it.C;
    // per-request descales of the cached part (uniform loads)
    if (p.k_desc) {
        const float kd = p.k_desc[p.desc_per_seq ? si.b : 0];
        p.qk_scale2_ctx *= kd;
        p.cap_c1_ctx *= kd;
    }
    if (p.v_desc) p.v_scale *= p.v_desc[p.desc_per_seq ? si.b : 0];
    const int t0 = it.t0, t1 = it.t1;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, grp = lane >> 4;

    // ---- rows of this lane's column blocks, and Q^T as B operands ----
    int row_t[kRB], pos_q[kRB];
    bool row_ok[kRB];
    float al2[kRB];                    // ALiBi slope of the row's head, log2 units
    u32x4 qop[kRB][kDS];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const int r = (wave * kRB + rb) * 16 + c;
        row_t[rb] = t0 + r / G;
        row_ok[rb] = row_t[rb] < t1;
        pos_q[rb] = si.C + row_t[rb];
        al2[rb] = p.alibi ? p.alibi[si.kvh * G + r % G] * kLog2e : 0.f;
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
    const int jt0 = it.jt0;
    const int ntiles = it.ntiles;

    // Context page ids in LDS, kExtPages at a time: `need(jt)` reloads the list
    // (between barriers) when tile jt's context keys are not all in it.
    si.pages = L.pages;
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
        for (int i = threadIdx.x; i < cnt; i += kExtThreads) L.pages[i] = row[i];
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

    // ---- the tiles [from, to), in phases of one kind: tiles [it_win,
    // it_diag) need no mask (inside every row's window and below every row's
    // diagonal); the tile holding key C mixes context and new keys.  A phase
    // of full single-kind tiles runs the FAST variant, the others the general
    // one; each phase is its own loop. ----
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
    //         [cut3,cut4) fast, [cut4,cut5) general; each clipped to [from, to)
#pragma unroll
    for (int k = 0; k < 6; ++k) cut[k] = min(max(cut[k], from), to);

    if constexpr (!FP8) {
        StageLane<D> sl;
        sl.init(p);
        const bool runs = p.page_shift >= 4;                 // runs stay inside a page
        auto stage = [&](int jt, uint8_t* kd, uint8_t* vd) {
            need(jt);
            if (runs) stage_runs<D>(p, si, jt, kd, vd, sl);
            else stage_direct<D>(p, si, jt, kd, vd);
        };
        auto run = [&](int a, int e, auto fast) {
            for (int i = a; i < e; ++i) {
                const int jt = jt0 + i * kExtKeys;
                uint8_t* kc = (i & 1) ? L.k1 : L.k0;
                uint8_t* vc = (i & 1) ? L.v1 : L.v0;
                if (i + 1 < to) stage(jt + kExtKeys, (i & 1) ? L.k0 : L.k1,
                                      (i & 1) ? L.v0 : L.v1);
                tile_compute<D, MODE, decltype(fast)::value>(kc, vc, lo, qop, A, p, si, pos_q,
                                                             al2, jt);
                wait_vm0();
                __syncthreads();
            }
        };
        stage(jt0 + from * kExtKeys, (from & 1) ? L.k1 : L.k0, (from & 1) ? L.v1 : L.v0);
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
            stage8_store<D, false>(sk, kd);
            stage8_store<D, true>(sv, vd);
        };
        auto run = [&](int a, int e, auto fast) {
            for (int i = a; i < e; ++i) {
                const int jt = jt0 + i * kExtKeys;
                const bool more = i + 1 < to;
                if (more) load(jt + kExtKeys);
                tile_compute<D, MODE, decltype(fast)::value>((i & 1) ? L.k1 : L.k0,
                                                             (i & 1) ? L.v1 : L.v0, lo, qop,
                                                             A, p, si, pos_q, al2, jt);
                if (more) store((i & 1) ? L.k0 : L.k1, (i & 1) ? L.v0 : L.v1);
                __syncthreads();
            }
        };
        load(jt0 + from * kExtKeys);
        store((from & 1) ? L.k1 : L.k0, (from & 1) ? L.v1 : L.v0);
        __syncthreads();
        run(cut[0], cut[1], std::false_type{});
        run(cut[1], cut[2], std::true_type{});
        run(cut[2], cut[3], std::false_type{});
        run(cut[3], cut[4], std::true_type{});
        run(cut[4], cut[5], std::false_type{});
    }

    // ---- finish: O^T[d][row c] / l; MFMA dblk, accumulator row 4grp + j
    // holds d = 16*dblk + 4grp + j ----
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        const float lt = col4_sum(A.l[rb]);
        if (!row_ok[rb]) continue;
        const int r = (wave * kRB + rb) * 16 + c;
        if (complete) {
            uint16_t* orow = static_cast<uint16_t*>(p.out) +
                             ((int64_t)(si.q0 + row_t[rb]) * p.num_q_heads + si.kvh * G + r % G) *
                                 D;
            // a sink logit joins the normaliser (no value row)
            float den = lt;
            if (p.sinks) den += fast_exp2(p.sinks[si.kvh * G + r % G] * kLog2e - A.m[rb]);
            const float inv = 1.f / den;
#pragma unroll
            for (int dblk = 0; dblk < kVE; ++dblk)
                *reinterpret_cast<u32x2*>(orow + 16 * dblk + 4 * grp) =
                    u32x2{pack_bf16x2(A.o[rb][dblk][0] * inv, A.o[rb][dblk][1] * inv),
                          pack_bf16x2(A.o[rb][dblk][2] * inv, A.o[rb][dblk][3] * inv)};
        } else {
            // a part: normalised rows and log2-sum-exp (no sink), for the merge
            const int64_t prow = ext_part_row(w, slot, r);
            const float inv = 1.f / lt;
            float* po = p.part_o + prow * D;
#pragma unroll
            for (int dblk = 0; dblk < kVE; ++dblk)
                *reinterpret_cast<f32x4*>(po + 16 * dblk + 4 * grp) = A.o[rb][dblk] * inv;
            if (grp == 0) p.part_lse[prow] = A.m[rb] + __log2f(lt);
        }
    }
}

// ---------------------------------------------------------------------------
// Persistent blocks: block w owns key tiles [w*N/W, (w+1)*N/W) of the items
// laid end to end (N tiles in all), cut into pieces at item boundaries.  The
// owner of an item's first tile records which blocks cover it.
// ---------------------------------------------------------------------------
template <int D, bool FP8, int MODE>
__global__ __launch_bounds__(kExtThreads, kExtOccupancy) void extend_kernel(ExtendParams p) {
    using TL = Tile<D>;
    // two buffers of K and V (tile `it` in buffer it & 1)
    __shared__ __attribute__((aligned(1024))) uint8_t sm_k0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_v0[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_k1[TL::kBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_v1[TL::kBytes];
    __shared__ int sm_pages[kExtPages];
    const ExtLds L{sm_k0, sm_v0, sm_k1, sm_v1, sm_pages};

    // Blocks are dealt to the 8 XCDs in turn; the logical index w gives each
    // XCD a contiguous run of the tile stream, so the row tiles of one
    // (sequence, kv head) share its L2.
    const int64_t W = gridDim.x;
    const int64_t w = (W % 8 == 0) ? (int64_t)(blockIdx.x % 8) * (W / 8) + blockIdx.x / 8
                                    : (int64_t)blockIdx.x;
    const int64_t items = ext_items(p);
    const int64_t N = p.pfx[items];
    const int64_t r0 = w * N / W, r1 = (w + 1) * N / W;
    if (r0 >= r1) {
        // an empty range (N < W): the merge may read this block's slot 0
        for (int r = threadIdx.x; r < kExtRows; r += kExtThreads)
            p.part_lse[ext_part_row(w, 0, r)] = -INFINITY;
        return;
    }
    // the item holding tile r0: the last i with pfx[i] <= r0
    int64_t lo = 0, hi = items;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (p.pfx[mid] <= r0) lo = mid;
        else hi = mid;
    }
    int64_t i = lo;
    int64_t pos = r0;
    int slot = 0;
    while (pos < r1) {
        while (p.pfx[i + 1] <= pos) ++i;                 // (items without tiles)
        const Item it = item_of(p, i);
        const int64_t start = p.pfx[i], end = p.pfx[i + 1];
        const int from = (int)(pos - start);
        const int to = (int)(min(r1, end) - start);
        const bool complete = from == 0 && to == it.ntiles;
        if (from == 0 && threadIdx.x == 0) {
            // the owner of the item's first tile: which blocks cover it
            const int64_t w_last = complete ? w : ((end * W + N - 1) / N - 1);
            *reinterpret_cast<int4*>(p.rec + 4 * i) = int4{(int)w, (int)w_last, slot, 0};
        }
        extend_piece<D, FP8, MODE>(p, it, from, to, complete, w, slot, L);
        pos += to - from;
        slot = 1;
    }
}

// ---------------------------------------------------------------------------
// Merge: kMergeSlices blocks per item covered by several blocks, each taking a
// slice of its rows; per row and column quad, the pieces' rows weighted by
// 2^(lse - max) (the stage-2 merge of the decode page), a sink joining the
// sum once.  A thread folds kMergeUnits (row, quad) units side by side.
// ---------------------------------------------------------------------------
constexpr int kExtMergeThreads = 256;
constexpr int kMergeSlices = 4;

template <int D>
__global__ __launch_bounds__(kExtMergeThreads) void extend_merge_kernel(ExtendParams p) {
    constexpr int kQ = D / 4;
    constexpr int kSliceRows = kExtRows / kMergeSlices;
    constexpr int kUnits = kSliceRows * kQ / kExtMergeThreads;
    const int64_t i = blockIdx.x / kMergeSlices;
    const int slice = blockIdx.x % kMergeSlices;
    const Item it = item_of(p, i);
    if (it.ntiles == 0) return;
    const int4 rec = *reinterpret_cast<const int4*>(p.rec + 4 * i);
    if (rec.x == rec.y) return;                          // written whole by one block
    const int G = p.group;
    const int rows = (it.t1 - it.t0) * G;
    if (slice * kSliceRows >= rows) return;
    float m[kUnits], sum[kUnits];
    f32x4 acc[kUnits];
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
        m[k] = -INFINITY;
        sum[k] = 0.f;
        acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int piece = 0; piece <= rec.y - rec.x; ++piece) {
        const int64_t base = ext_part_row(rec.x + piece, piece == 0 ? rec.z : 0, 0);
        float lse[kUnits];
        f32x4 o[kUnits];
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            const int u = threadIdx.x + kExtMergeThreads * k;
            const int r = slice * kSliceRows + u / kQ, q = u % kQ;
            lse[k] = -INFINITY;
            o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (r < rows) {
                lse[k] = p.part_lse[base + r];
                o[k] = *reinterpret_cast<const f32x4*>(p.part_o + (base + r) * D + 4 * q);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
            if (lse[k] == -INFINITY) continue;          // (an empty block's slot)
            const float mn = fmaxf(m[k], lse[k]);
            const float f = m[k] == -INFINITY ? 0.f : fast_exp2(m[k] - mn);
            const float wt = fast_exp2(lse[k] - mn);
            sum[k] = sum[k] * f + wt;
            acc[k] = acc[k] * f + wt * o[k];
            m[k] = mn;
        }
    }
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
        const int u = threadIdx.x + kExtMergeThreads * k;
        const int r = slice * kSliceRows + u / kQ, q = u % kQ;
        if (r >= rows) continue;
        const int h = it.kvh * G + r % G;
        float s = sum[k];
        if (p.sinks && s > 0.f) s += fast_exp2(p.sinks[h] * kLog2e - m[k]);
        const float inv = s > 0.f ? 1.f / s : 0.f;
        uint16_t* dst = static_cast<uint16_t*>(p.out) +
                        ((int64_t)(it.q0 + it.t0 + r / G) * p.num_q_heads + h) * D + 4 * q;
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(acc[k].x * inv, acc[k].y * inv),
                                               pack_bf16x2(acc[k].z * inv, acc[k].w * inv)};
    }
}

template <int D, bool FP8>
const void* extend_kernel_ptr(int mode) {
    switch (mode) {
        case kCap: return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kCap>);
        case kFold: return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kFold>);
        case kScale | kAlibi:
            return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kScale | kAlibi>);
        case kCap | kAlibi:
            return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kCap | kAlibi>);
        default: return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kScale>);
    }
}

const void* extend_kernel_for(int head_dim, bool fp8, int mode) {
    if (head_dim == 128)
        return fp8 ? extend_kernel_ptr<128, true>(mode) : extend_kernel_ptr<128, false>(mode);
    return fp8 ? extend_kernel_ptr<64, true>(mode) : extend_kernel_ptr<64, false>(mode);
}

}  // namespace

int extend_rows_per_block() { return kExtRows; }

hipError_t launch_extend(const ExtendParams& p, int head_dim, bool fp8, int workers,
                         hipStream_t stream) {
    const int mode = p.has_cap ? (p.alibi ? kCap | kAlibi : kCap)
                     : p.alibi ? kScale | kAlibi
                     : (p.qk_scale2 > 0.f && p.qk_scale2_ctx > 0.f) ? kFold : kScale;
    hipLaunchKernelGGL(extend_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, p);
    const void* f = extend_kernel_for(head_dim, fp8, mode);
    void* args[] = {const_cast<ExtendParams*>(&p)};
    hipError_t e = hipLaunchKernel(f, dim3(workers), dim3(kExtThreads), args, 0, stream);
    if (e != hipSuccess) return e;
    const int64_t items = (int64_t)p.num_seqs * p.num_kv_heads * p.q_tiles;
    if (head_dim == 128)
        hipLaunchKernelGGL(extend_merge_kernel<128>, dim3((unsigned)(items * kMergeSlices)),
                           dim3(kExtMergeThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(extend_merge_kernel<64>, dim3((unsigned)(items * kMergeSlices)),
                           dim3(kExtMergeThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t extend_blocks_per_cu(int head_dim, bool fp8, int* out) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, extend_kernel_for(head_dim, fp8, kFold), kExtThreads, 0);
}

}  // namespace pa
