// extend.hip -- prefix-prefill (extend) attention for gfx950.
//
// New query tokens of a sequence attend to its cached context through the
// pages (no mask) and causally to each other (contiguous new K/V rows), with
// the same window, scale and soft-cap as decode: the two loops of `_fwd_kernel`
// on the page "vllm/attention/ops/prefix_prefill.py" (context phase, then the
// new-token phase with its causal mask), finished by the division of the
// accumulator by the softmax sum.
//
// Work: an item is (sequence b, kv head g, row tile): kExtRows rows, a row
// being (new token t, query head h of the group), so the G heads of a kv head
// share every K/V byte a block stages.  Its keys are [lo, C + t_last] (lo from
// the sliding window of its first token) in tiles of 64: key j < C comes from
// page block_table[b][j / P], key j >= C is new row j - C.  Persistent blocks
// take equal ranges of the key tiles of all items laid end to end (stream-K);
// an item several blocks cover is finished by a log-sum-exp merge.
//
// Each wave owns 32 rows; per tile, with v_mfma_f32_32x32x16_bf16:
//   S^T[64 keys x 32 rows] = K[64 x D] Q^T[D x 32]   K from LDS (A operand),
//                                                   Q^T in registers
//   online softmax: a row is one MFMA column, held by a lane pair (l, l^32)
//   O^T[D x 32] += V^T[D x 64] P^T[64 x 32]          P^T is the S^T accumulator
//                                                   itself; V^T comes from
//                                                   transposing LDS reads
// The LDS operand reads run ahead of the MFMAs that take them: key half 1's
// K operands behind half 0's MFMAs, each P V step's V operands behind the
// previous step's, the first step's under the softmax.
//
// K/V tiles live in LDS as bf16 rows of 2*D bytes with 16-byte slots
// XOR-swizzled by row, so that operand reads hit distinct banks, in a ring
// of four buffers per kind.  bf16 caches are staged with direct global->LDS
// loads two tiles ahead (a wave fills whole 1 KB runs of its own rows of a
// tile, K and V at once; with pages of >= 8 rows a run has one page, so its
// base is wave-uniform and each lane adds a fixed offset); fp8 context rows
// go through registers to be converted, one tile ahead.
#include <climits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

#ifndef PA_EXTEND_WAVES
#define PA_EXTEND_WAVES 8
#endif
#ifndef PA_EXTEND_OCCUPANCY
#define PA_EXTEND_OCCUPANCY 2
#endif
constexpr int kExtWaves = PA_EXTEND_WAVES;       // waves per block
constexpr int kExtThreads = 64 * kExtWaves;
constexpr int kExtRows = 32 * kExtWaves;         // rows (token, head) per block
constexpr int kExtKeys = 64;                     // keys per tile
constexpr int kExtPages = 2048;                  // page ids staged in LDS at a time
constexpr int kExtOccupancy = PA_EXTEND_OCCUPANCY;   // waves per SIMD (bf16 caches)
constexpr int kStageRows = kExtKeys / kExtWaves; // rows of a tile one wave stages
// K and V tile buffers: tile i lives in buffer gray(i mod 4) (consecutive tiles
// differ in one bit of the buffer index, so moving to the next tile's buffer
// is one XOR); bf16 loads run two tiles ahead.
constexpr int kExtBuffers = 4;
#ifndef PA_EXTEND_PIPE
#define PA_EXTEND_PIPE 1
#endif
__host__ __device__ constexpr int gray4(int i) { return (i & 3) ^ ((i & 3) >> 1); }
static_assert(gray4(0) == 0 && gray4(1) == 1 && gray4(2) == 3 && gray4(3) == 2 &&
                  gray4(4) == 0 && gray4(7) == 2,
              "the buffer sequence 0 1 3 2 repeats every four tiles");

// How scores become log2-domain logits.
enum ScoreMode {
    kFold = 0,    // no cap, one positive scale per tile: max on raw scores,
                  // exp2(s*scale - m) (a positive scale commutes with the max)
    kScale = 1,   // no cap, any scale: s*scale per score
    kCap = 2,     // soft-cap c*tanh(s*scale/c), per score
    kAlibi = 4,   // flag on kScale / kCap: plus slope * (key - query position)
    kVScale = 8,  // flag: cached values are scaled (v_scale != 1 or per-request
                  // value descales); without it P V takes the values as stored
};

// What a tile's softmax must handle.
enum TileKind {
    kTileMixed = 0,   // masks, and context and new keys scored differently
    kTileFast = 1,    // no mask, one key kind (or both kinds scored alike)
    kTileMasked = 2,  // masks (causal limit, window), one key kind
};

// LDS tile geometry: 64 rows of 2*D bytes, 16-byte slots swizzled by row.
template <int D>
struct Tile {
    static constexpr int kPitch = 2 * D;
    static constexpr int kSlots = kPitch / 16;
    static constexpr int kBytes = kExtKeys * kPitch;
    static constexpr int kRowsPerRun = 1024 / kPitch;       // rows of a 1 KB run
    static constexpr int kRuns = kStageRows / kRowsPerRun;  // runs one wave stages
    static_assert(kRuns >= 1, "a wave stages whole runs");
    // K: the 16-byte operand reads of 16 consecutive rows at one logical slot
    // land on 16 different 16-byte bank groups.
    static __device__ __forceinline__ int kswz(int r) {
        return (kPitch == 256 ? r : (r >> 1)) & (kSlots - 1);
    }
    // V: a half-wave's transposing reads cover one 64-byte window of four
    // consecutive rows; the window moves with the row so the four are disjoint.
    static __device__ __forceinline__ int vswz(int r) {
        return kPitch == 256 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
    }
};

struct SeqInfo {
    int b, kvh, n, C, q0;       // q0 = cu_seqlens_q[b]
    int pg0;                    // first logical page of the staged page list
    const int* pages;           // LDS: block_table[b][pg0 .. pg0 + kExtPages)
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

// A value the compiler can neither see through nor hoist out of a loop.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// LDS byte address (32 bits) of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Global -> LDS loads of 16 bytes a lane: lane i fills LDS bytes lds + 16i ..
// + 15 (lds wave-uniform).  They are issued in inline asm, so the compiler
// does not track these LDS writes and puts no wait for them in front of the
// operand reads of the other buffer; the kernel waits for them itself
// (s_waitcnt vmcnt(0)) before the barrier that hands the buffer to its
// readers.  Two address forms: a wave-uniform base plus a 32-bit lane offset,
// or a per-lane 64-bit address.
// (M0, which the instruction takes the LDS address from, is saved and
// restored around it.)
__device__ __forceinline__ void load_lds16(const uint8_t* base, uint32_t off, uint32_t lds) {
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "v"(off), "s"(base), "s"(lds) : "memory");
}
__device__ __forceinline__ void load_lds16(const uint8_t* addr, uint32_t lds) {
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\t"
                 "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "v"(addr), "s"(lds) : "memory");
}

// bf16: this wave's rows of tile jt of K and of V straight into LDS at the
// byte addresses kdst and vdst.  In a 1 KB run (kRowsPerRun rows) lane i fills LDS
// bytes 16i..16i+15, i.e. slot i % kSlots of row i / kSlots, with the row's
// chunk (slot ^ swizzle).  Rows in one page (pages of >= kStageRows rows) or
// all new rows inside the sequence take one wave-uniform base and a 32-bit
// lane offset; others go lane by lane.
template <int D>
__device__ __forceinline__ void stage_kv(const ExtendParams& p, const SeqInfo& si, int jt,
                                         uint32_t kdst, uint32_t vdst) {
    using TL = Tile<D>;
    // (the lane's row and slot are recomputed per call: nothing lane-dependent
    // of the staging stays live across the tile loop)
    const int lane = (int)opaque(threadIdx.x & 63);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rr = lane / TL::kSlots, sl = lane % TL::kSlots;
    const int j0 = jt + wave * kStageRows;
    const uint32_t dk = kdst + wave * TL::kRuns * 1024, dv = vdst + wave * TL::kRuns * 1024;
    auto kchunk = [&](int k) {
        const int r = wave * kStageRows + k * TL::kRowsPerRun + rr;
        return (uint32_t)(16 * (sl ^ TL::kswz(r)));
    };
    auto vchunk = [&](int k) {
        const int r = wave * kStageRows + k * TL::kRowsPerRun + rr;
        return (uint32_t)(16 * (sl ^ TL::vswz(r)));
    };
    if ((1 << p.page_shift) >= kStageRows && j0 + kStageRows <= si.C) {
        // K and V rows sit at the same offsets of their pools: one page
        // lookup for both
        const int idx = min(max((j0 >> p.page_shift) - si.pg0, 0), kExtPages - 1);
        const int64_t page = __builtin_amdgcn_readfirstlane(si.pages[idx]);
        const int pmask = (1 << p.page_shift) - 1;
        const int64_t off = (page * p.s_page + (int64_t)(j0 & pmask) * p.s_tok +
                             (int64_t)si.kvh * p.s_head) * 2;
        const uint8_t* kb = static_cast<const uint8_t*>(p.k_pool) + off;
        const uint8_t* vb = static_cast<const uint8_t*>(p.v_pool) + off;
        const int64_t run = (int64_t)TL::kRowsPerRun * p.s_tok * 2;
        const uint32_t lrow = (uint32_t)rr * (uint32_t)(p.s_tok * 2);
#pragma unroll
        for (int k = 0; k < TL::kRuns; ++k) load_lds16(kb + k * run, lrow + kchunk(k), dk + k * 1024);
#pragma unroll
        for (int k = 0; k < TL::kRuns; ++k) load_lds16(vb + k * run, lrow + vchunk(k), dv + k * 1024);
    } else if (j0 >= si.C && j0 + kStageRows <= si.C + si.n) {
        const int64_t rs = (int64_t)p.num_kv_heads * D * 2;
        const int64_t off = ((int64_t)(si.q0 + j0 - si.C) * p.num_kv_heads + si.kvh) * D * 2;
        const uint8_t* kb = static_cast<const uint8_t*>(p.k_new) + off;
        const uint8_t* vb = static_cast<const uint8_t*>(p.v_new) + off;
        const uint32_t lrow = (uint32_t)rr * (uint32_t)rs;
#pragma unroll
        for (int k = 0; k < TL::kRuns; ++k)
            load_lds16(kb + k * TL::kRowsPerRun * rs, lrow + kchunk(k), dk + k * 1024);
#pragma unroll
        for (int k = 0; k < TL::kRuns; ++k)
            load_lds16(vb + k * TL::kRowsPerRun * rs, lrow + vchunk(k), dv + k * 1024);
    } else {
        // lane by lane: context rows through the page list, new rows (clamped
        // to the sequence's last one: finite, masked by the consumer) from
        // k_new / v_new
        const int pmask = (1 << p.page_shift) - 1;
#pragma unroll
        for (int k = 0; k < TL::kRuns; ++k) {
            const int j = jt + wave * kStageRows + k * TL::kRowsPerRun + rr;
            const int idx = min(max((j >> p.page_shift) - si.pg0, 0), kExtPages - 1);
            const int64_t ctx = ((int64_t)si.pages[idx] * p.s_page +
                                 (int64_t)(j & pmask) * p.s_tok + (int64_t)si.kvh * p.s_head) * 2;
            const int r = min(max(j - si.C, 0), si.n - 1);
            const int64_t nw = ((int64_t)(si.q0 + r) * p.num_kv_heads + si.kvh) * D * 2;
            const bool in_ctx = j < si.C;
            const uint8_t* ks = in_ctx ? static_cast<const uint8_t*>(p.k_pool) + ctx
                                       : static_cast<const uint8_t*>(p.k_new) + nw;
            const uint8_t* vs = in_ctx ? static_cast<const uint8_t*>(p.v_pool) + ctx
                                       : static_cast<const uint8_t*>(p.v_new) + nw;
            load_lds16(ks + kchunk(k), dk + k * 1024);
            load_lds16(vs + vchunk(k), dv + k * 1024);
        }
    }
}

// fp8 caches: a tile of K or V through registers, 16 elements a thread per
// pass: context rows are e4m3fn (converted to bf16 while stored), new rows
// bf16.  Threads past the tile's chunks idle.
template <int D>
struct Stage8 {
    static constexpr int kChunks = kExtKeys * D / 16;        // 16-element chunks a tile
    static constexpr int kPasses = (kChunks + kExtThreads - 1) / kExtThreads;
    u32x4 a[kPasses], b[kPasses];
    bool ctx[kPasses];
};

template <int D>
__device__ __forceinline__ void stage8_load(Stage8<D>& S, const ExtendParams& p,
                                            const SeqInfo& si, int jt, bool second) {
    using ST = Stage8<D>;
#pragma unroll
    for (int i = 0; i < ST::kPasses; ++i) {
        const int c = threadIdx.x + i * kExtThreads;
        S.ctx[i] = true;
        S.a[i] = S.b[i] = u32x4{0, 0, 0, 0};
        if (c >= ST::kChunks) continue;
        const int row = c / (D / 16), ch = c % (D / 16);
        const uint8_t *kr, *vr;
        key_rows<D, true>(p, si, jt + row, kr, vr);
        const uint8_t* r = second ? vr : kr;
        S.ctx[i] = jt + row < si.C;
        if (S.ctx[i]) {
            S.a[i] = *reinterpret_cast<const u32x4*>(r + 16 * ch);
        } else {
            S.a[i] = *reinterpret_cast<const u32x4*>(r + 32 * ch);
            S.b[i] = *reinterpret_cast<const u32x4*>(r + 32 * ch + 16);
        }
    }
}

template <int D, bool V>
__device__ __forceinline__ void stage8_store(const Stage8<D>& S, uint8_t* lds) {
    using ST = Stage8<D>;
    using TL = Tile<D>;
#pragma unroll
    for (int i = 0; i < ST::kPasses; ++i) {
        const int c = threadIdx.x + i * kExtThreads;
        if (c >= ST::kChunks) continue;
        const int row = c / (D / 16), ch = c % (D / 16);
        u32x4 lo = S.a[i], hi = S.b[i];
        if (S.ctx[i]) {
            const u32x2 e0 = e4m3x4_to_bf16x4(S.a[i].x), e1 = e4m3x4_to_bf16x4(S.a[i].y);
            const u32x2 e2 = e4m3x4_to_bf16x4(S.a[i].z), e3 = e4m3x4_to_bf16x4(S.a[i].w);
            lo = u32x4{e0.x, e0.y, e1.x, e1.y};
            hi = u32x4{e2.x, e2.y, e3.x, e3.y};
        }
        const int sw = V ? TL::vswz(row) : TL::kswz(row);
        *reinterpret_cast<u32x4*>(lds + row * TL::kPitch + 16 * ((2 * ch) ^ sw)) = lo;
        *reinterpret_cast<u32x4*>(lds + row * TL::kPitch + 16 * ((2 * ch + 1) ^ sw)) = hi;
    }
}

// Wait for this wave's direct-to-LDS loads (vmcnt 0; expcnt and lgkmcnt
// left at their maxima).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }


// Per-lane LDS byte offsets of the operand reads (lane l, h = l / 32).
//   K (A operand of S^T): key row 32kb + l%32, d = 16ds + 8h .. +7, i.e.
//     logical slot 2ds + h: koff[ds] (+ 32kb rows; the swizzle depends on
//     l % 32 only).
//   V^T (A operand of O^T, 32 d x 16 keys for 32x32x16): transposing reads
//     (ds_read_b64_tr_b16: within each 16 lanes, lane i receives element e
//     from the 8 bytes lane 4e + i/4 read, element i % 4).  Lane (group g =
//     l/16, e = (l%16)/4, q = l%4) reads key row R + 4h + e (and R + 8 + 4h + e)
//     at d = 32db + 16(g%2) + 4q; lane l then holds d = 32db + l%32 of keys
//     R + 4h + 0..3 (and R + 8 + 4h + 0..3): contraction slots 0..7 of lane
//     half h.  R = 32kb + 16(s%2) for P V step s: voff[db] (R = 0).
template <int D>
struct LaneOffs {
    int koff[D / 16];
    int voff[D / 32];
    // offsets into buffer `buf` of the K and V tile rings
    __device__ __forceinline__ void init(int lane, int buf) {
        using TL = Tile<D>;
        const int r = lane & 31, h = lane >> 5;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds)
            koff[ds] = buf * TL::kBytes + r * TL::kPitch + 16 * ((2 * ds + h) ^ TL::kswz(r));
        const int g = lane >> 4, e = (lane & 15) >> 2, q = lane & 3;
        const int row = 4 * h + e;                   // (+ R: same swizzle)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            voff[db] = buf * TL::kBytes + row * TL::kPitch +
                       16 * ((4 * db + 2 * (g & 1) + (q >> 1)) ^ TL::vswz(row)) + 8 * (q & 1);
    }
    // from tile i's buffer to tile i + 1's: one bit of the buffer index flips
    // (bit 0 after an even tile, bit 1 after an odd one)
    __device__ __forceinline__ void next(int i) {
        const int x = (i & 1) ? 2 * Tile<D>::kBytes : Tile<D>::kBytes;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) koff[ds] ^= x;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) voff[db] ^= x;
    }
};

// S^T = K Q^T for key half H (keys 32H .. 32H+31) of a 64-key tile (kt: the
// K buffer pair; koff selects the buffer): s[j] is the score of key
// 32H + 8(j/4) + 4h + j%4 against the lane's row.
template <int D, int H>
__device__ __forceinline__ void qk_half(f32x16& s, const uint8_t* kt, const LaneOffs<D>& lo,
                                        const u32x4 (&q)[D / 16]) {
    constexpr int kPitch = Tile<D>::kPitch;
    // every operand read is issued before the first MFMA, so the reads'
    // latencies overlap
    u32x4 a[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
        a[ds] = *reinterpret_cast<const u32x4*>(kt + H * 32 * kPitch + lo.koff[ds]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = {};
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) acc = mfma_bf16_32x32x16(a[ds], q[ds], acc);
    s = acc;
}

typedef __attribute__((ext_vector_type(4))) short i16x4;

// One transposing read (ds_read_b64_tr_b16) of 8 bytes at an LDS address.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4 __attribute__((address_space(3)))*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// O^T += V^T P^T for key half H (vt: the V buffer pair; voff selects the
// buffer): P V steps s = 2H + t (t = 0, 1) cover keys
// 32H + 16t + ..., with B operands pk[t] (accumulator slots 8t .. 8t+7).
// The D/32 operands of a step are read (two transposing reads each) before
// its MFMAs.
template <int D, int H>
__device__ __forceinline__ void pv_half(f32x16 (&o)[D / 32], const uint8_t* vt,
                                        const LaneOffs<D>& lo, const u32x4 (&pk)[2]) {
    constexpr int kPitch = Tile<D>::kPitch;
    constexpr int kDB = D / 32;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        u32x2 v[2 * kDB];
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            const uint8_t* r = vt + (32 * H + 16 * t) * kPitch + lo.voff[db];
            v[2 * db] = lds_read_tr16(r);
            v[2 * db + 1] = lds_read_tr16(r + 8 * kPitch);
        }
#pragma unroll
        for (int db = 0; db < kDB; ++db)
            o[db] = mfma_bf16_32x32x16(u32x4{v[2 * db].x, v[2 * db].y, v[2 * db + 1].x,
                                             v[2 * db + 1].y},
                                       pk[t], o[db]);
    }
}

__device__ __forceinline__ float vmax(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}

// Running state of one wave's lane: its row's max (log2 units, lazy) and this
// lane's share of the row sum; O^T accumulators.
template <int D>
struct ExtAcc {
    float m, l;
    f32x16 o[D / 32];
};

// Per-tile constants of the softmax (one key kind).
struct TileScale {
    float qs, c1, vs;       // score scale, soft-cap factor, value scale
};

// The online softmax of one key half's scores, in steps:
//   logits: scale (or soft-cap) in place -- tiles of one key kind with MODE
//     kFold keep raw scores, the positive scale is folded into the exponent
//     -- masks of a masked tile (causal limit and window of the lane's row),
//     per-key scales of a mixed one, and the lane's max;
//   row_max: the lane pair's max; whether any row of the wave moves its
//     reference max (lazy rescale: only when a score exceeds it by more than
//     8 in log2 units, so p <= 2^8), and the rescale factor;
//   exps: p = 2^(logit - m) in place;
//   pack: value scales and the bf16 B operands of P V.
struct SoftmaxState {
    float m_new, ms, alpha;
    bool move;
};

template <int MODE, int KIND>
__device__ __forceinline__ float sm_logits(f32x16& s, const ExtendParams& p, const SeqInfo& si,
                                           const TileScale& ts, int pos_q, float al2,
                                           int key0) {
    constexpr bool kAl = (MODE & kAlibi) != 0;
    constexpr bool kFolded = (MODE & 7) == kFold && KIND != kTileMixed;
    // key key0 + c is kept iff lo_c < c <= hi_c (causal limit; window start)
    const int hi_c = pos_q - key0;
    const int lo_c = p.window > 0 ? hi_c - p.window : INT_MIN;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float v = s[j];
        const int key = key0 + 8 * (j >> 2) + (j & 3);
        if constexpr (!kFolded) {
            const bool ctx = key < si.C;
            const float qs = KIND != kTileMixed ? ts.qs : (ctx ? p.qk_scale2_ctx : p.qk_scale2);
            if constexpr ((MODE & 3) == kCap) {
                const float c1 = KIND != kTileMixed ? ts.c1 : (ctx ? p.cap_c1_ctx : p.cap_c1);
                v = p.cap_c2 - 2.f * p.cap_c2 * fast_rcp(fast_exp2(v * c1) + 1.f);
            } else {
                v *= qs;
            }
        }
        if constexpr (kAl) v += al2 * (float)(key - pos_q);
        if constexpr (KIND != kTileFast) {
            const int c = 8 * (j >> 2) + (j & 3);
            v = (c <= hi_c && c > lo_c) ? v : -INFINITY;
        }
        s[j] = v;
    }
    // (maximum: NaN-propagating, no input canonicalisation; three-input
    // instructions on gfx950)
    const float a = vmax(vmax(s[0], s[1]), s[2]), b = vmax(vmax(s[3], s[4]), s[5]);
    const float c = vmax(vmax(s[6], s[7]), s[8]), d = vmax(vmax(s[9], s[10]), s[11]);
    const float e = vmax(vmax(s[12], s[13]), s[14]);
    return vmax(vmax(vmax(a, b), c), vmax(vmax(d, e), s[15]));
}

template <int MODE, int KIND>
__device__ __forceinline__ SoftmaxState sm_row_max(float lane_max, float m, const TileScale& ts) {
    constexpr float kSlack = 8.f;
    float tmax = pair_max(lane_max);
    if constexpr ((MODE & 7) == kFold && KIND != kTileMixed) tmax *= ts.qs;
    SoftmaxState st;
    st.move = __builtin_amdgcn_ballot_w64(tmax > m + kSlack) != 0;
    st.m_new = st.move ? fmaxf(m, tmax) : m;
    st.ms = st.m_new == -INFINITY ? 0.f : st.m_new;   // a row with no key yet
    st.alpha = fast_exp2(m - st.ms);
    return st;
}

template <int MODE, int KIND>
__device__ __forceinline__ void sm_exps(f32x16& s, const SoftmaxState& st, float qs) {
    constexpr bool kFolded = (MODE & 7) == kFold && KIND != kTileMixed;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        s[j] = kFolded ? fast_exp2(__builtin_fmaf(s[j], qs, -st.ms)) : fast_exp2(s[j] - st.ms);
}

template <int MODE, int KIND>
__device__ __forceinline__ void sm_pack(f32x16& s, u32x4 (&pk)[2], const SeqInfo& si,
                                        const TileScale& ts, int key0) {
    if constexpr ((MODE & kVScale) != 0) {
        if constexpr (KIND != kTileMixed) {
            s *= ts.vs;
        } else {
            // context keys take the cache's value scale, new keys none
#pragma unroll
            for (int j = 0; j < 16; ++j)
                s[j] *= key0 + 8 * (j >> 2) + (j & 3) < si.C ? ts.vs : 1.f;
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
        pk[t] = u32x4{pack_bf16x2(s[8 * t], s[8 * t + 1]), pack_bf16x2(s[8 * t + 2], s[8 * t + 3]),
                      pack_bf16x2(s[8 * t + 4], s[8 * t + 5]),
                      pack_bf16x2(s[8 * t + 6], s[8 * t + 7])};
}

// The online softmax of one tile's scores (s[H]: key half H): updates the
// row statistics and returns the packed probabilities (pk[2H + t]: P V step
// 2H + t) and whether (and by what) to rescale O.
template <int MODE, int KIND>
__device__ __forceinline__ SoftmaxState tile_softmax(f32x16 (&s)[2], u32x4 (&pk)[4], float& m,
                                                     float& l, const ExtendParams& p,
                                                     const SeqInfo& si, const TileScale& ts,
                                                     int pos_q, float al2, int key0) {
    const float m0 = sm_logits<MODE, KIND>(s[0], p, si, ts, pos_q, al2, key0);
    const float m1 = sm_logits<MODE, KIND>(s[1], p, si, ts, pos_q, al2, key0 + 32);
    const SoftmaxState st = sm_row_max<MODE, KIND>(vmax(m0, m1), m, ts);
    sm_exps<MODE, KIND>(s[0], st, ts.qs);
    sm_exps<MODE, KIND>(s[1], st, ts.qs);
    // the row sum (before any value scale), as a tree of independent adds
    float t4[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const f32x16& v = s[i >> 2];
        const int o = 4 * (i & 3);
        t4[i] = (v[o] + v[o + 1]) + (v[o + 2] + v[o + 3]);
    }
    l = l * st.alpha + (((t4[0] + t4[1]) + (t4[2] + t4[3])) + ((t4[4] + t4[5]) + (t4[6] + t4[7])));
    sm_pack<MODE, KIND>(s[0], reinterpret_cast<u32x4(&)[2]>(pk[0]), si, ts, key0);
    sm_pack<MODE, KIND>(s[1], reinterpret_cast<u32x4(&)[2]>(pk[2]), si, ts, key0 + 32);
    m = st.m_new;
    return st;
}

// The V^T operands of P V step st (keys 16 st .. 16 st + 15), block db.
template <int D>
__device__ __forceinline__ void read_v_step(u32x2 (&v)[D / 16], const uint8_t* vt,
                                            const LaneOffs<D>& lo, int st) {
    constexpr int kPitch = Tile<D>::kPitch;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const uint8_t* r = vt + 16 * st * kPitch + lo.voff[db];
        v[2 * db] = lds_read_tr16(r);
        v[2 * db + 1] = lds_read_tr16(r + 8 * kPitch);
    }
}

// S^T = K Q^T for both key halves with the operand reads of key half 1
// issued one by one behind the MFMAs of half 0 (each register takes its
// half-1 operand as soon as its half-0 MFMA has it), and the V^T operands
// of the first P V step read after them, to arrive during the softmax.
template <int D>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], u32x2 (&v0)[D / 16],
                                        const uint8_t* kt, const uint8_t* vt,
                                        const LaneOffs<D>& lo, const u32x4 (&q)[D / 16]) {
    constexpr int kPitch = Tile<D>::kPitch;
    constexpr int kDS = D / 16;
    u32x4 a[kDS];
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds)
        a[ds] = *reinterpret_cast<const u32x4*>(kt + lo.koff[ds]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = {};
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) {
        acc = mfma_bf16_32x32x16(a[ds], q[ds], acc);
        a[ds] = *reinterpret_cast<const u32x4*>(kt + 32 * kPitch + lo.koff[ds]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    }
    s[0] = acc;
    __builtin_amdgcn_sched_barrier(0);
    acc = f32x16{};
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) acc = mfma_bf16_32x32x16(a[ds], q[ds], acc);
    read_v_step<D>(v0, vt, lo, 0);
    s[1] = acc;
    __builtin_amdgcn_sched_barrier(0);
}

// O^T += V^T P^T over the four 16-key steps; step st's operands (v, read
// ahead) feed its MFMAs while step st + 1's are read into the registers
// each MFMA has just taken.
template <int D>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[D / 32], u32x2 (&v)[D / 16],
                                        const uint8_t* vt, const LaneOffs<D>& lo,
                                        const u32x4 (&pk)[4]) {
    constexpr int kPitch = Tile<D>::kPitch;
    constexpr int kDB = D / 32;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            o[db] = mfma_bf16_32x32x16(u32x4{v[2 * db].x, v[2 * db].y, v[2 * db + 1].x,
                                             v[2 * db + 1].y},
                                       pk[st], o[db]);
            if (st < 3) {
                const uint8_t* r = vt + 16 * (st + 1) * kPitch + lo.voff[db];
                v[2 * db] = lds_read_tr16(r);
                v[2 * db + 1] = lds_read_tr16(r + 8 * kPitch);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
    }
}

// One 64-key tile (K and V at the offsets lo selects): S^T = K Q^T for both
// key halves, the online softmax (the variant of the tile's kind), P V.  Only
// the softmax differs between the variants, so the accumulators never pass
// through the branch.
template <int D, int MODE>
__device__ __forceinline__ void tile_compute(int kind, const uint8_t* kbuf,
                                             const uint8_t* vbuf, const LaneOffs<D>& lo,
                                             const u32x4 (&q)[D / 16], ExtAcc<D>& A,
                                             const ExtendParams& p, const SeqInfo& si,
                                             const TileScale& ts, int pos_q, float al2, int jt) {
    constexpr int kDB = D / 32;
    const int key0 = jt + 4 * ((threadIdx.x & 63) >> 5);
    f32x16 s[2];
#if PA_EXTEND_PIPE
    u32x2 v[D / 16];
    qk_tile<D>(s, v, kbuf, vbuf, lo, q);
#else
    qk_half<D, 0>(s[0], kbuf, lo, q);
    qk_half<D, 1>(s[1], kbuf, lo, q);
#endif
    u32x4 pk[4];
    const SoftmaxState st =
        kind == kTileFast
            ? tile_softmax<MODE, kTileFast>(s, pk, A.m, A.l, p, si, ts, pos_q, al2, key0)
        : kind == kTileMasked
            ? tile_softmax<MODE, kTileMasked>(s, pk, A.m, A.l, p, si, ts, pos_q, al2, key0)
            : tile_softmax<MODE, kTileMixed>(s, pk, A.m, A.l, p, si, ts, pos_q, al2, key0);
    if (st.move) {
#pragma unroll
        for (int db = 0; db < kDB; ++db) A.o[db] *= st.alpha;
    }
#if PA_EXTEND_PIPE
    pv_tile<D>(A.o, v, vbuf, lo, pk);
#else
    pv_half<D, 0>(A.o, vbuf, lo, reinterpret_cast<const u32x4(&)[2]>(pk[0]));
    pv_half<D, 1>(A.o, vbuf, lo, reinterpret_cast<const u32x4(&)[2]>(pk[2]));
#endif
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
// Unit prefix over the items: pfx[i] = stream units of items 0..i-1 (one
// block).
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
        // an item with tiles takes piece_cost units, then one a tile
        int v = 0;
        if (i < items) {
            const int nt = item_of(p, i).ntiles;           // < 2^24
            v = nt > 0 ? nt + p.piece_cost : 0;
        }
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
    uint8_t *k, *v;     // rings of kExtBuffers K and V tiles
    int* pages;
};

template <int D, bool FP8, int MODE>
__device__ __forceinline__ void extend_piece(const ExtendParams& pk, const Item& it, int from,
                                             int to, bool complete, int64_t w, int slot,
                                             const ExtLds& L) {
    constexpr int kDS = D / 16;        // QK contraction steps
    constexpr int kDB = D / 32;        // O^T blocks of 32 d
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
    const int h = lane >> 5;

    // ---- this lane's row (a lane pair shares it) and Q^T as B operands:
    // lane l holds Q[row][16ds + 8h .. +7] ----
    const int r = wave * 32 + (lane & 31);
    const int row_t = t0 + r / G;
    const bool row_ok = row_t < t1;
    const int head = si.kvh * G + r % G;
    const int pos_q = si.C + row_t;
    const float al2 = p.alibi ? p.alibi[head] * kLog2e : 0.f;
    u32x4 q[kDS];
    {
        const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                               ((int64_t)(si.q0 + (row_ok ? row_t : t0)) * p.num_q_heads + head) * D;
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * ds + 8 * h);
            q[ds] = row_ok ? v : u32x4{0, 0, 0, 0};
        }
    }

    const int jt0 = it.jt0;
    const int pos_first = si.C + t0, pos_last = si.C + t1 - 1;
    // a tile needs no mask when it ends at or before the first row's diagonal
    // and starts inside the last row's window; it has one key kind when it
    // does not straddle the context's end
    // context and new keys are scored and weighted alike (unit cache scales)
    const bool one_scale = p.qk_scale2_ctx == p.qk_scale2 && p.cap_c1_ctx == p.cap_c1 &&
                           (MODE & kVScale) == 0;
    auto tile_kind = [&](int jt) {
        const bool one_kind = one_scale || jt + kExtKeys <= si.C || jt >= si.C;
        const bool unmasked = jt + kExtKeys - 1 <= pos_first &&
                              (p.window <= 0 || jt >= pos_last - p.window + 1);
        return !one_kind ? kTileMixed : unmasked ? kTileFast : kTileMasked;
    };
    auto tile_scale = [&](int jt) {
        const bool ctx = jt < si.C;
        return TileScale{ctx ? p.qk_scale2_ctx : p.qk_scale2, ctx ? p.cap_c1_ctx : p.cap_c1,
                         ctx ? p.v_scale : 1.f};
    };

    LaneOffs<D> lo;
    ExtAcc<D> A;
    A.m = -INFINITY;
    A.l = 0.f;
#pragma unroll
    for (int db = 0; db < kDB; ++db) A.o[db] = f32x16{};

    si.pages = L.pages;
    si.pg0 = 0;
    auto jt_of = [&](int i) { return jt0 + i * kExtKeys; };

    // Tile i's K and V live in buffer gray(i mod 4).  bf16: tile i's loads
    // are issued at the start of tile i - 2 (the prologue issues the chunk's
    // first two tiles); the end of tile i waits for tile i + 1's (the loads
    // issued during this tile may stay in flight) and a barrier publishes
    // them.  Tile i + 2's buffer last held tile i - 2, released by the
    // barrier that ended tile i - 2.  fp8 goes through registers one tile
    // ahead: loads at the start of tile i, converted stores at its end.
    using TL = Tile<D>;
    const uint32_t k_lds = lds_addr(L.k), v_lds = lds_addr(L.v);
    auto buf_of = [](int i) { return (uint32_t)(gray4(i) * TL::kBytes); };
    auto stage_bf16 = [&](int i) {
        stage_kv<D>(p, si, jt_of(i), k_lds + buf_of(i), v_lds + buf_of(i));
    };
    constexpr int kLoads = 2 * TL::kRuns;                   // a wave's loads per tile
    auto tile = [&](int i, int c1) {
        const int jt = jt_of(i);
        bool issued = false;
        Stage8<D> sk, sv;
        if constexpr (!FP8) {
            if (i + 2 < c1) {
                stage_bf16(i + 2);
                issued = true;
            }
        } else {
            if (i + 1 < c1) {
                stage8_load<D>(sk, p, si, jt_of(i + 1), false);
                stage8_load<D>(sv, p, si, jt_of(i + 1), true);
            }
        }
        const TileScale ts = tile_scale(jt);
        tile_compute<D, MODE>(tile_kind(jt), L.k, L.v, lo, q, A, p, si, ts, pos_q, al2, jt);
        if constexpr (FP8) {
            if (i + 1 < c1) {
                stage8_store<D, false>(sk, L.k + buf_of(i + 1));
                stage8_store<D, true>(sv, L.v + buf_of(i + 1));
            }
        } else {
            // vmcnt(kLoads) / vmcnt(0), expcnt and lgkmcnt left at their maxima
            if (issued) __builtin_amdgcn_s_waitcnt(0x0F70 | (kLoads & 15) | ((kLoads >> 4) << 14));
            else wait_vm0();
        }
        __syncthreads();
        lo.next(i);
    };

    // The tiles in chunks whose context pages fit the LDS page list.
    lo.init(lane, gray4(from));
    const int chunk_tiles = max(1, ((kExtPages - 2) << p.page_shift) / kExtKeys);
#pragma nounroll
    for (int c0 = from; c0 < to; c0 += chunk_tiles) {
        const int c1 = min(to, c0 + chunk_tiles);
        {
            __syncthreads();                                   // the old list is unused
            const int jlo = jt_of(c0);
            const int jhi = min(jt_of(c1), si.C) - 1;          // last context key
            si.pg0 = jlo >> p.page_shift;
            const int cnt = jhi >= jlo ? (jhi >> p.page_shift) - si.pg0 + 1 : 0;
            const int32_t* row = p.block_table + (int64_t)si.b * p.bt_stride + si.pg0;
            copy_ids_to_lds<4>(L.pages, row, cnt, threadIdx.x, kExtThreads);
            __syncthreads();
        }
        if constexpr (!FP8) {
            stage_bf16(c0);
            if (c0 + 1 < c1) stage_bf16(c0 + 1);
            wait_vm0();
        } else {
            Stage8<D> sk, sv;
            stage8_load<D>(sk, p, si, jt_of(c0), false);
            stage8_load<D>(sv, p, si, jt_of(c0), true);
            stage8_store<D, false>(sk, L.k + buf_of(c0));
            stage8_store<D, true>(sv, L.v + buf_of(c0));
        }
        __syncthreads();
#pragma nounroll
        for (int i = c0; i < c1; ++i) tile(i, c1);
    }

    // ---- finish: the lane pair's sums; O^T[d][row] / l, d = 32db + 8(j/4) +
    // 4h + j%4 for accumulator slot j ----
    const float lt = pair_sum(A.l);
    if (!row_ok) return;
    if (complete) {
        uint16_t* orow = static_cast<uint16_t*>(p.out) +
                         ((int64_t)(si.q0 + row_t) * p.num_q_heads + head) * D;
        // a sink logit joins the normaliser (no value row)
        float den = lt;
        if (p.sinks) den += fast_exp2(p.sinks[head] * kLog2e - A.m);
        const float inv = 1.f / den;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * jj + 4 * h) =
                    u32x2{pack_bf16x2(A.o[db][4 * jj] * inv, A.o[db][4 * jj + 1] * inv),
                          pack_bf16x2(A.o[db][4 * jj + 2] * inv, A.o[db][4 * jj + 3] * inv)};
    } else {
        // a part: normalised rows and log2-sum-exp (no sink), for the merge
        const int64_t prow = ext_part_row(w, slot, r);
        const float inv = 1.f / lt;
        float* po = p.part_o + prow * D;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *reinterpret_cast<f32x4*>(po + 32 * db + 8 * jj + 4 * h) =
                    f32x4{A.o[db][4 * jj], A.o[db][4 * jj + 1], A.o[db][4 * jj + 2],
                          A.o[db][4 * jj + 3]} * inv;
        if (h == 0) p.part_lse[prow] = A.m + __log2f(lt);
    }
}

// ---------------------------------------------------------------------------
// Persistent blocks: the items are laid end to end as a stream of N units,
// an item with tiles taking piece_cost units (what starting a piece costs a
// block, in tiles' worth) and then one unit a key tile; block w owns the
// tiles whose units fall in [w*N/W, (w+1)*N/W), cut into pieces at item
// boundaries.  The owner of an item's first tile records which blocks cover
// it.
// ---------------------------------------------------------------------------
template <int D, bool FP8>
constexpr int ext_occupancy() { return FP8 ? 1 : kExtOccupancy; }

template <int D, bool FP8, int MODE>
__global__ __launch_bounds__(kExtThreads)
__attribute__((amdgpu_waves_per_eu(ext_occupancy<D, FP8>(), ext_occupancy<D, FP8>())))
void extend_kernel(ExtendParams p) {
    using TL = Tile<D>;
    // rings of K and V tile buffers
    __shared__ __attribute__((aligned(1024))) uint8_t sm_k[kExtBuffers * TL::kBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_v[kExtBuffers * TL::kBytes];
    __shared__ int sm_pages[kExtPages];
    const ExtLds L{sm_k, sm_v, sm_pages};

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
    // the item holding unit r0: the last i with pfx[i] <= r0, by a 64-way
    // search (each round a lane reads one candidate of [lo, lo + cnt); the
    // last one at or below r0 narrows the range to its step)
    int64_t lo = 0, cnt = items;         // pfx[lo] <= r0 < pfx[lo + cnt]
    while (cnt > 1) {
        const int64_t step = (cnt + 63) / 64;
        const int64_t k = lo + (int64_t)(threadIdx.x & 63) * step;
        const bool at_or_below = k < lo + cnt && p.pfx[k] <= r0;
        const int j = 63 - __builtin_clzll(__ballot(at_or_below));   // lane 0's k = lo is
        const int64_t kj = lo + (int64_t)j * step;                   // always at or below
        cnt = min(step, lo + cnt - kj);
        lo = kj;
    }
    int64_t i = lo;
    int64_t pos = r0;
    int slot = 0;
    while (pos < r1) {
        while (p.pfx[i + 1] <= pos) ++i;                 // (items without tiles)
        const Item it = item_of(p, i);
        const int64_t end = p.pfx[i + 1];
        const int64_t u0 = end - it.ntiles;              // unit of the item's first tile
        // the item's tiles whose units are in [pos, r1); none when the range
        // ends in front of its first tile
        const int from = (int)max(pos - u0, (int64_t)0);
        const int to = (int)(min(r1, end) - u0);
        if (to <= from) break;
        const bool complete = from == 0 && to == it.ntiles;
        if (from == 0 && threadIdx.x == 0) {
            // the owner of the item's first tile: which blocks cover it
            const int64_t w_last = complete ? w : ((end * W + N - 1) / N - 1);
            *reinterpret_cast<int4*>(p.rec + 4 * i) = int4{(int)w, (int)w_last, slot, 0};
        }
        extend_piece<D, FP8, MODE>(p, it, from, to, complete, w, slot, L);
        pos = min(r1, end);
        slot = 1;
    }
}

// ---------------------------------------------------------------------------
// Merge: kMergeSlices blocks per item covered by several blocks, each taking a
// slice of its rows; per row and column quad, the pieces' rows weighted by
// 2^(lse - max) (the stage-2 merge of the decode page), a sink joining the
// sum once.  A thread folds kUnits (row, quad) units side by side, the loads
// of two pieces in flight together.
// ---------------------------------------------------------------------------
constexpr int kExtMergeThreads = 256;
#ifndef PA_EXTEND_MERGE_SLICES
#define PA_EXTEND_MERGE_SLICES 16
#endif
constexpr int kMergeSlices = PA_EXTEND_MERGE_SLICES;

template <int D>
__global__ __launch_bounds__(kExtMergeThreads) void extend_merge_kernel(ExtendParams p) {
    constexpr int kQ = D / 4;
    constexpr int kSliceRows = kExtRows / kMergeSlices;
    constexpr int kUnits = (kSliceRows * kQ + kExtMergeThreads - 1) / kExtMergeThreads;
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
    // two pieces at a time: both pieces' loads are in flight together
    const int npieces = rec.y - rec.x + 1;
    for (int piece0 = 0; piece0 < npieces; piece0 += 2) {
        float lse[2][kUnits];
        f32x4 o[2][kUnits];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const int piece = piece0 + pp;
            const int64_t base = ext_part_row(rec.x + piece, piece == 0 ? rec.z : 0, 0);
#pragma unroll
            for (int k = 0; k < kUnits; ++k) {
                const int u = threadIdx.x + kExtMergeThreads * k;
                const int r = slice * kSliceRows + u / kQ, q = u % kQ;
                lse[pp][k] = -INFINITY;
                o[pp][k] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (piece < npieces && u < kSliceRows * kQ && r < rows) {
                    lse[pp][k] = p.part_lse[base + r];
                    o[pp][k] = *reinterpret_cast<const f32x4*>(p.part_o + (base + r) * D + 4 * q);
                }
            }
        }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int k = 0; k < kUnits; ++k) {
                if (lse[pp][k] == -INFINITY) continue;      // (an empty block's slot)
                const float mn = fmaxf(m[k], lse[pp][k]);
                const float f = m[k] == -INFINITY ? 0.f : fast_exp2(m[k] - mn);
                const float wt = fast_exp2(lse[pp][k] - mn);
                sum[k] = sum[k] * f + wt;
                acc[k] = acc[k] * f + wt * o[pp][k];
                m[k] = mn;
            }
    }
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
        const int u = threadIdx.x + kExtMergeThreads * k;
        const int r = slice * kSliceRows + u / kQ, q = u % kQ;
        if (u >= kSliceRows * kQ || r >= rows) continue;
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

template <int D, bool FP8, int V>
const void* extend_kernel_mode(int mode) {
    switch (mode) {
        case kCap: return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kCap | V>);
        case kFold: return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kFold | V>);
        case kScale | kAlibi:
            return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kScale | kAlibi | V>);
        case kCap | kAlibi:
            return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kCap | kAlibi | V>);
        default: return reinterpret_cast<const void*>(&extend_kernel<D, FP8, kScale | V>);
    }
}

template <int D, bool FP8>
const void* extend_kernel_ptr(int mode) {
    return (mode & kVScale) ? extend_kernel_mode<D, FP8, kVScale>(mode & ~kVScale)
                            : extend_kernel_mode<D, FP8, 0>(mode);
}

const void* extend_kernel_for(int head_dim, bool fp8, int mode) {
    if (head_dim == 128)
        return fp8 ? extend_kernel_ptr<128, true>(mode) : extend_kernel_ptr<128, false>(mode);
    return fp8 ? extend_kernel_ptr<64, true>(mode) : extend_kernel_ptr<64, false>(mode);
}

}  // namespace

int extend_rows_per_block() { return kExtRows; }
int extend_waves_per_block() { return kExtWaves; }

hipError_t launch_extend(const ExtendParams& p, int head_dim, bool fp8, int workers,
                         hipStream_t stream) {
    const int mode = (p.has_cap ? (p.alibi ? kCap | kAlibi : kCap)
                      : p.alibi ? kScale | kAlibi
                      : (p.qk_scale2 > 0.f && p.qk_scale2_ctx > 0.f) ? kFold : kScale) |
                     ((p.v_scale != 1.f || p.v_desc) ? kVScale : 0);
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
