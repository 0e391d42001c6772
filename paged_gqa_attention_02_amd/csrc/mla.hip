// mla.hip -- split pass of paged decode over a latent KV cache for gfx950:
// the query/key head dim DQK is larger than the value head dim DV, and the
// value of a token is the first DV entries of its row (Lk = 576 split as
// 512 + 64, Lv = 512, or 288 = 256 + 32 and 256: the `BLOCK_DMODEL` /
// `BLOCK_DPE` / `BLOCK_DV` choice of `_decode_grouped_att_m_fwd` on the
// decode page "vllm/attention/ops/triton_decode_attention.py").
//
// The value rows are read at the key rows' places with the key strides; a
// latent cache passes one pool as both, and then the value operands come from
// the key tile already in LDS (each row crosses HBM once).  The stream-K cut
// of the key ranges, the partial slots, the segment records and the merge are
// those of the decode split pass (decode_geom.h, merge.hip).
//
// Work: persistent blocks of NW waves walk the tiles of their range; wave wv
// owns query rows (the heads of the kv head) 16wv .. 16wv + 15, and the G
// heads share every staged byte.  Per 32-key tile, with
// v_mfma_f32_16x16x32_bf16:
//   S^T[32 keys x 16 rows] = K[32 x DQK] Q^T[DQK x 16]   K from LDS in the A
//                                                      layout, Q^T in registers
//   online softmax per row (one MFMA column: 4 lanes hold its keys)
//   O^T[DV x 16] += V^T[DV x 32] P^T[32 x 16]          P^T is the S^T
//                                                      accumulator; V^T from
//                                                      transposing LDS reads
// LDS tile: a main region (entries [0, DV) of 32 rows, 2*DV bytes a row) and a
// rope region (entries [DV, DQK)), each row's 16-byte slots XOR-swizzled so
// the operand reads of a quarter wave (K: 16 rows, one slot; V: 8 rows, 32
// bytes each) hit distinct banks.  Tiles are filled by direct global->LDS
// loads (lane i of a wave fills bytes 16i..16i+15 of a 1 KB run): a main run
// is whole rows, a rope run 8 (or 16) rows.  Two buffers: the next tile's
// loads are in flight while this tile is computed.
//
// One pool and at most 16 query heads (the common latent case): blocks of two
// waves, one computing and one staging the tiles through registers (plain
// 16-byte loads, then LDS stores) with one barrier per tile.  On MI355X the
// direct-to-LDS path streams at most about 5.2 TB/s, register loads about
// 6.9 TB/s.
#include <climits>

#include "decode_geom.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kMlaPages = 1024;        // page ids staged in LDS for one chunk

template <int DQK, int DV>
struct MlaTile {
    static constexpr int kMainPitch = 2 * DV;              // bytes per main row
    static constexpr int kMainSlots = kMainPitch / 16;
    static constexpr int kRopePitch = 2 * (DQK - DV);
    static constexpr int kRopeSlots = kRopePitch / 16;
    static constexpr int kMainBytes = kTile * kMainPitch;
    static constexpr int kKBytes = kMainBytes + kTile * kRopePitch;
    static constexpr int kMainRows = 1024 / kMainPitch;    // rows per 1 KB run
    static constexpr int kRopeRows = 1024 / kRopePitch;
    static constexpr int kMainRuns = kTile / kMainRows;
    static constexpr int kRopeRuns = kTile / kRopeRows;
    static_assert(kMainPitch % 256 == 0 && kMainPitch <= 1024 && kMainSlots >= 16,
                  "main rows start on bank 0 and hold at least 16 slots");
    static_assert(kRopeSlots == 8 || kRopeSlots == 4, "rope rows of 128 or 64 bytes");
    // Main region: slot s of row r sits at slot s ^ mswz(r) (< 16, so inside
    // the row).  K reads: 16 rows, one slot -> 16 distinct values of the
    // swizzle = 16 bank groups.  V reads: 8 consecutive rows (4 per 16
    // lanes), 32 bytes each -> mswz(r) >> 1 = r & 7 puts them on 8 distinct
    // 32-byte groups.
    static __device__ __forceinline__ int mswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
    // Rope region (rows of 128 / 64 bytes, two / four rows per 256 bytes):
    // (row parity, swizzle) resp. (row mod 4, swizzle) distinct over 16 rows.
    static __device__ __forceinline__ int rswz(int r) {
        return kRopeSlots == 8 ? (r >> 1) & 7 : (r >> 2) & 3;
    }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16 lanes, lane i receives element e of the
// 8 bytes lane 4e + i/4 addressed, element i % 4.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Wait for this wave's direct-to-LDS loads (vmcnt 0; expcnt and lgkmcnt at
// their maxima).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Where the rows of a chunk of tiles come from.
struct MlaChunk {
    const uint8_t* kbase;     // k_pool + kv head offset (bytes)
    const uint8_t* vbase;
    int64_t page_bytes;
    int tok_bytes;
    int page_shift, first_page;
    int t_begin, t_end;       // keys of the chunk inside the key range
    const int* pages;         // LDS: block_table[b][first_page ...]
};

// Stage the K rows (and, without ALIAS, the V rows) of the tile at t0 into
// LDS.  Runs: K main, K rope, then V main; wave wv issues runs wv, wv + NW,
// ...  Rows outside [t_begin, t_end) load a row inside it (finite data; the
// softmax masks them).
template <int DQK, int DV, int NW, bool ALIAS>
__device__ __forceinline__ void mla_stage(const MlaChunk& ch, int t0, bool uniform,
                                          uint8_t* kt, uint8_t* vt, int wv, int lane) {
    using T = MlaTile<DQK, DV>;
    constexpr int kRuns = T::kMainRuns + T::kRopeRuns + (ALIAS ? 0 : T::kMainRuns);
    constexpr int kPer = (kRuns + NW - 1) / NW;
    const int pmask = (1 << ch.page_shift) - 1;
    // page_size >= 32: the whole tile lies in one page
    const int64_t tile_page = uniform ? ch.pages[(t0 >> ch.page_shift) - ch.first_page] : 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int run = wv + k * NW;
        if (run >= kRuns) break;
        int row, off;
        const uint8_t* base;
        uint8_t* dst;
        if (run < T::kMainRuns) {
            row = run * T::kMainRows + lane / T::kMainSlots;
            off = 16 * ((lane % T::kMainSlots) ^ T::mswz(row));
            base = ch.kbase;
            dst = kt + run * 1024;
        } else if (run < T::kMainRuns + T::kRopeRuns) {
            const int rr = run - T::kMainRuns;
            row = rr * T::kRopeRows + lane / T::kRopeSlots;
            off = 2 * DV + 16 * ((lane % T::kRopeSlots) ^ T::rswz(row));
            base = ch.kbase;
            dst = kt + T::kMainBytes + rr * 1024;
        } else {
            const int rr = run - T::kMainRuns - T::kRopeRuns;
            row = rr * T::kMainRows + lane / T::kMainSlots;
            off = 16 * ((lane % T::kMainSlots) ^ T::mswz(row));
            base = ch.vbase;
            dst = vt + rr * 1024;
        }
        const int t = min(max(t0 + row, ch.t_begin), ch.t_end - 1);
        const int64_t page =
            uniform ? tile_page : (int64_t)ch.pages[(t >> ch.page_shift) - ch.first_page];
        const uint8_t* src =
            base + page * ch.page_bytes + (uint32_t)((t & pmask) * ch.tok_bytes + off);
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)(src),
            (void __attribute__((address_space(3)))*)(dst), 16, 0, 0);
    }
}

// Producer wave of a two-wave block (latent cache, at most 16 query heads):
// stages the chunk's tiles through registers, tile i into buffer i & 1, with
// one barrier per tile after the tile is in LDS; the consumer wave passes the
// same barrier before it reads the tile.  Two tiles are in flight.  Every
// step issues the same loads -- the last steps re-read the chunk's last tile,
// which the cache still holds -- so the load counts the compiler waits on are
// the same on every path.
template <int DQK, int DV>
__device__ __forceinline__ void mla_produce(const MlaChunk& ch, int tile0, int ct, bool uniform,
                                            uint8_t* b0, uint8_t* b1, int lane) {
    using T = MlaTile<DQK, DV>;
    constexpr int kRuns = T::kMainRuns + T::kRopeRuns;
    const int pmask = (1 << ch.page_shift) - 1;
    // (row, byte offset) of this lane's 16 bytes in run `run` of a tile
    auto slot_of = [&](int run, int& row, int& off) {
        if (run < T::kMainRuns) {
            row = run * T::kMainRows + lane / T::kMainSlots;
            off = 16 * ((lane % T::kMainSlots) ^ T::mswz(row));
        } else {
            const int rr = run - T::kMainRuns;
            row = rr * T::kRopeRows + lane / T::kRopeSlots;
            off = 2 * DV + 16 * ((lane % T::kRopeSlots) ^ T::rswz(row));
        }
    };
    // Straight-line loads into r (a branch per load would make the compiler
    // land each load in a temporary and wait for it before the copy).
    auto load = [&](u32x4 (&r)[kRuns], int i) {
        const int t0 = tile0 + i * kTile;
        if (uniform) {
            // page_size >= 32: the whole tile lies in one page
            const uint8_t* base =
                ch.kbase + (int64_t)ch.pages[(t0 >> ch.page_shift) - ch.first_page] * ch.page_bytes;
#pragma unroll
            for (int run = 0; run < kRuns; ++run) {
                int row, off;
                slot_of(run, row, off);
                const int t = min(max(t0 + row, ch.t_begin), ch.t_end - 1);
                r[run] = *reinterpret_cast<const u32x4*>(
                    base + (uint32_t)((t & pmask) * ch.tok_bytes + off));
            }
        } else {
#pragma unroll
            for (int run = 0; run < kRuns; ++run) {
                int row, off;
                slot_of(run, row, off);
                const int t = min(max(t0 + row, ch.t_begin), ch.t_end - 1);
                const int64_t page = ch.pages[(t >> ch.page_shift) - ch.first_page];
                r[run] = *reinterpret_cast<const u32x4*>(
                    ch.kbase + page * ch.page_bytes +
                    (uint32_t)((t & pmask) * ch.tok_bytes + off));
            }
        }
    };
    auto store = [&](const u32x4 (&r)[kRuns], uint8_t* buf) {
#pragma unroll
        for (int run = 0; run < kRuns; ++run) {
            uint8_t* dst = run < T::kMainRuns ? buf + run * 1024
                                              : buf + T::kMainBytes + (run - T::kMainRuns) * 1024;
            *reinterpret_cast<u32x4*>(dst + 16 * lane) = r[run];
        }
    };
    const int last = ct - 1;
    u32x4 ra[kRuns], rb[kRuns];
    load(ra, 0);
    load(rb, min(1, last));
    for (int i = 0; i < ct; i += 2) {
        store(ra, b0);
        load(ra, min(i + 2, last));
        __syncthreads();                       // tile i is in buffer 0
        if (i + 1 >= ct) break;
        store(rb, b1);
        load(rb, min(i + 3, last));
        __syncthreads();                       // tile i + 1 is in buffer 1
    }
}

// Per-lane byte offsets of the operand reads inside a tile (rows 16kb + c
// and 16h + 4grp + e share the swizzle of c and 4grp + e).
//   K main, MFMA step ds (entries 32ds + 8grp ..): kmain[ds & 3] + 256 (ds >> 2)
//   K rope, step ds: krope[ds]
//   V^T block dblk (entries 16dblk ..): vtr[dblk & 7] + 256 (dblk >> 3)
template <int DQK, int DV>
struct MlaOffs {
    static constexpr int kRopeSteps = (DQK - DV) / 32;
    int kmain[4];
    int krope[kRopeSteps];
    int vtr[8];
    __device__ __forceinline__ void init(int c, int grp, int lane) {
        using T = MlaTile<DQK, DV>;
        const int m = T::mswz(c);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            kmain[v] = c * T::kMainPitch + 64 * (v ^ (m >> 2)) + 16 * (grp ^ (m & 3));
        const int r = T::rswz(c);
#pragma unroll
        for (int ds = 0; ds < kRopeSteps; ++ds)
            krope[ds] = T::kMainBytes + c * T::kRopePitch + 16 * ((4 * ds + grp) ^ r);
        // transposing reads: lane (grp, 4e + q) reads row 4grp + e, entries
        // 16dblk + 4q .. +3 (logical slot 2dblk + q/2, byte 8(q % 2) in it)
        const int e = (lane & 15) >> 2, q = lane & 3;
        const int row = 4 * grp + e;
        const int mv = T::mswz(row);
#pragma unroll
        for (int v = 0; v < 8; ++v)
            vtr[v] = row * T::kMainPitch + 32 * (v ^ (mv >> 1)) + 16 * ((q >> 1) ^ (mv & 1)) +
                     8 * (q & 1);
    }
};

// ---------------------------------------------------------------------------
// Split pass
// ---------------------------------------------------------------------------
// PC: two-wave blocks over one pool with at most 16 query heads; wave 0
// computes and wave 1 stages the tiles through registers (mla_produce).
// Otherwise the NW waves stage each tile with direct-to-LDS loads and each
// computes its 16 query heads.
template <int DQK, int DV, int NW, bool ALIAS, bool PC>
__global__ __launch_bounds__(64 * NW) void mla_split_kernel(DecodeParams p) {
    static_assert(!PC || (NW == 2 && ALIAS), "producer/consumer blocks: two waves, one pool");
    using T = MlaTile<DQK, DV>;
    constexpr int KM = DV / 32;                // QK steps over the main entries
    constexpr int KR = (DQK - DV) / 32;        // QK steps over the rope entries
    constexpr int VE = DV / 16;                // PV MFMAs per tile

    const int lane = threadIdx.x & 63;
    const int wv = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, grp = lane >> 4;
    const int cg = 16 * wv + c;                // this lane's query row (head of the kv head)
    const int G = p.group;
    // Block h*Wg + j takes virtual head h over range j of that head's stream
    // (the plan makes the block count a multiple of the virtual heads), so
    // the blocks of the heads of one token range, which read the same rows,
    // run side by side.
    const int64_t W = gridDim.x;
    const int64_t w = blockIdx.x;
    const int HG = split_head_groups(p.num_kv_heads);
    const int hm = p.num_kv_heads / HG;
    const int64_t Wg = W / HG;
    const int head0 = (int)(w / Wg);
    if (head0 >= HG) return;                    // (no range: never merged)

    __shared__ int sm_pages[kMlaPages];
    // Two buffers, each its own LDS object: the compiler then knows that the
    // next tile's direct-to-LDS loads do not write the buffer being read, and
    // issues no wait for them before this tile's operand reads.
    __shared__ __attribute__((aligned(1024))) uint8_t sm_k0[T::kKBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_k1[T::kKBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_v0[ALIAS ? 16 : T::kMainBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sm_v1[ALIAS ? 16 : T::kMainBytes];

    const RangeStart rs = locate_range<false>(p, hm, w % Wg, Wg);
    const int64_t N = rs.N, r0 = rs.r0, r1 = rs.r1;
    if (r0 >= r1) {
        // an empty range (N < W): the merge may read this block's slot 0
        for (int i = threadIdx.x; i < p.rows; i += 64 * NW)
            p.part_lse[part_row(p, w, 0) + i] = -INFINITY;
        return;
    }

    int b = rs.b;
    int64_t seq_start = rs.seq_start;
    SeqRange sr = rs.sr;

    const int chunk_tiles = ((kMlaPages - 2) << p.page_shift) / kTile;
    const bool uniform = p.page_shift >= 5;

    MlaOffs<DQK, DV> lo;
    lo.init(c, grp, lane);

    // (stream units: a segment of n tiles is piece_cost units, then one a
    // tile)
    const int A = p.piece_cost;
    int64_t pos = r0;
    int slot = 0;
    while (pos < r1) {
        const int n = sr.tiles;                               // > 0 here
        const int nu = n + A;                                 // units of a segment
        const int kvh = head0 + (int)((pos - seq_start) / nu);
        const int64_t seg_end = seq_start + (int64_t)(kvh - head0 + 1) * nu;
        const int64_t u0 = seg_end - n;                       // unit of the first tile
        // the segment's tiles whose units are in [pos, r1); none when the
        // range ends in front of its first tile
        const int i0 = (int)max(pos - u0, (int64_t)0);
        const int cnt = (int)(min(r1, seg_end) - u0) - i0;
        if (cnt <= 0) break;
        const bool complete = (i0 == 0) && (cnt == n);
        if (i0 == 0 && threadIdx.x == 0) {
            // this block owns the segment's first tile: tell the merge which
            // blocks cover it
            const int64_t w_last =
                complete ? w : (int64_t)head0 * Wg + tile_owner(seg_end - 1, N, Wg);
            *reinterpret_cast<int4*>(p.seg_rec + 4 * ((int64_t)b * p.num_kv_heads + kvh)) =
                int4{(int)w, (int)w_last, slot, 0};
        }

        MlaChunk ch;
        ch.kbase = static_cast<const uint8_t*>(p.k_pool) + (int64_t)kvh * p.s_head * 2;
        ch.vbase = static_cast<const uint8_t*>(p.v_pool) + (int64_t)kvh * p.s_head * 2;
        ch.page_bytes = p.s_page * 2;
        ch.tok_bytes = (int)(p.s_tok * 2);
        ch.page_shift = p.page_shift;
        ch.pages = sm_pages;

        // Chunk c0 of the piece: its key range, and its page ids staged in LDS
        // between two barriers that every wave of the block takes.
        auto begin_chunk = [&](int c0) {
            const int ct = min(cnt - c0, chunk_tiles);
            const int tile0 = sr.base + (i0 + c0) * kTile;
            ch.t_begin = max(tile0, sr.lo);
            ch.t_end = min(tile0 + ct * kTile, sr.L);
            ch.first_page = ch.t_begin >> p.page_shift;
            const int n_pages = ((ch.t_end - 1) >> p.page_shift) - ch.first_page + 1;
            __syncthreads();     // the previous chunk's readers are done with the list
            const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride + ch.first_page;
            copy_ids_to_lds<8>(sm_pages, bt, n_pages, threadIdx.x, 64 * NW);
            __syncthreads();
        };
        auto next_piece = [&]() {
            pos = min(r1, seg_end);
            slot = 1;
            if (pos < r1 && pos == seq_start + (int64_t)nu * hm) {
                seq_start = pos;
                do {
                    ++b;
                    sr = seq_range(p, b);
                } while (sr.tiles == 0);
            }
        };
        if constexpr (PC) {
            if (wv == 1) {
                // the producer wave: stage the piece's tiles, chunk by chunk
                for (int c0 = 0; c0 < cnt; c0 += chunk_tiles) {
                    begin_chunk(c0);
                    mla_produce<DQK, DV>(ch, sr.base + (i0 + c0) * kTile,
                                         min(cnt - c0, chunk_tiles), uniform, sm_k0, sm_k1, lane);
                }
                next_piece();
                continue;
            }
        }

        // ---- Q^T as B operands: column c is head kvh*G + cg; step ds covers
        // entries 32ds + 8grp + j (main), DV + 32ds + 8grp + j (rope) ----
        u32x4 qop[KM + KR];
        {
            const int cc = cg < p.rows ? cg : 0;
            const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                                   (int64_t)b * p.q_stride_b + (int64_t)(kvh * G + cc) * DQK;
#pragma unroll
            for (int ds = 0; ds < KM + KR; ++ds) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * ds + 8 * grp);
                qop[ds] = cg < p.rows ? v : u32x4{0, 0, 0, 0};
            }
        }

        // per-request cache descales of sequence b (uniform loads)
        float vsc = p.v_scale, qk2 = p.qk_scale2, c1 = p.cap_c1;
        if (p.k_desc) {
            const float kd = p.k_desc[p.desc_per_seq ? b : 0];
            qk2 *= kd;
            c1 *= kd;
        }
        if (p.v_desc) vsc *= p.v_desc[p.desc_per_seq ? b : 0];
        const float al2 = p.alibi ? p.alibi[kvh * G + (cg < p.rows ? cg : 0)] * kLog2e : 0.f;
        const int qpos = sr.L - 1;                            // the query token's position

        f32x4 o[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = -INFINITY, l = 0.f;

        // ---- the piece's tiles, chunk by chunk (page list staged in LDS) ----
        for (int c0 = 0; c0 < cnt; c0 += chunk_tiles) {
            const int ct = min(cnt - c0, chunk_tiles);
            const int tile0 = sr.base + (i0 + c0) * kTile;
            begin_chunk(c0);

            // one tile of the chunk, staged in kt (vt: its value rows)
            auto compute = [&](int i, const uint8_t* kt, const uint8_t* vt) {
                const int t0 = tile0 + i * kTile;
                // ---- S^T = K Q^T: s[kb][j] = score of key t0 + 16kb + 4grp + j.
                // A wave is alone on its SIMD (the LDS tiles allow two blocks
                // per compute unit), so nothing hides LDS latency but this
                // wave's own queue: all operand reads of the tile are issued
                // before the MFMAs, and the two key halves' accumulation
                // chains alternate. ----
                f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
                // (batched reads where the registers allow: two-wave blocks
                // over one pool; larger blocks are held to fewer registers and
                // read each operand right before its MFMA)
                constexpr bool kBatch = NW <= 2 && ALIAS;
                if constexpr (kBatch) {
                    constexpr int kKB = (KM + KR) % 6 == 0 ? 6 : 3;   // contraction steps per batch
                    static_assert((KM + KR) % kKB == 0, "whole batches");
#pragma unroll
                    for (int d0 = 0; d0 < KM + KR; d0 += kKB) {
                        u32x4 ka[2][kKB];
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int u = 0; u < kKB; ++u) {
                                const int ds = d0 + u;
                                ka[kb][u] = *reinterpret_cast<const u32x4*>(
                                    ds < KM ? kt + kb * 16 * T::kMainPitch + lo.kmain[ds & 3] +
                                                  256 * (ds >> 2)
                                            : kt + kb * 16 * T::kRopePitch + lo.krope[ds - KM]);
                            }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int u = 0; u < kKB; ++u)
#pragma unroll
                            for (int kb = 0; kb < 2; ++kb)
                                s[kb] = mfma_bf16_16x16x32(ka[kb][u], qop[d0 + u], s[kb]);
                    }
                } else {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                        for (int ds = 0; ds < KM + KR; ++ds) {
                            const u32x4 a = *reinterpret_cast<const u32x4*>(
                                ds < KM ? kt + kb * 16 * T::kMainPitch + lo.kmain[ds & 3] +
                                              256 * (ds >> 2)
                                        : kt + kb * 16 * T::kRopePitch + lo.krope[ds - KM]);
                            s[kb] = mfma_bf16_16x16x32(a, qop[ds], s[kb]);
                        }
                    }
                }

                // ---- scale / cap, ALiBi, mask; online softmax (log2 units) ----
                const bool full = t0 >= ch.t_begin && t0 + kTile <= ch.t_end;
                float tmax = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = t0 + 16 * kb + 4 * grp + j;
                        float v = s[kb][j];
                        v = p.has_cap ? p.cap_c2 - 2.f * p.cap_c2 * fast_rcp(fast_exp2(v * c1) + 1.f)
                                      : v * qk2;
                        if (p.alibi) v += al2 * (float)(key - qpos);
                        if (!full) v = (key >= ch.t_begin && key < ch.t_end) ? v : -INFINITY;
                        s[kb][j] = v;
                        tmax = fmaxf(tmax, v);
                    }
                tmax = col4_max(tmax);
                // Lazy rescale: the reference max moves only when a score
                // exceeds it by more than kSlack (log2 units), so p <= 2^kSlack.
                constexpr float kSlack = 8.f;
                const bool move = __any(tmax > m + kSlack);
                const float m_new = move ? fmaxf(m, tmax) : m;
                const float ms = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = fast_exp2(m - ms);
                float psum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float pr = fast_exp2(s[kb][j] - ms);
                        psum += pr;
                        s[kb][j] = pr;
                    }
                l = l * alpha + psum;
                m = m_new;
                if (move) {
#pragma unroll
                    for (int e = 0; e < VE; ++e) o[e] *= alpha;
                }
                // P^T as the B operand: contraction slot (grp, jj) is key
                // 4grp + jj (jj < 4) or 16 + 4grp + jj - 4
                const u32x4 pop = {pack_bf16x2(s[0][0], s[0][1]), pack_bf16x2(s[0][2], s[0][3]),
                                   pack_bf16x2(s[1][0], s[1][1]), pack_bf16x2(s[1][2], s[1][3])};

                // ---- O^T += V^T P^T: two transposing reads per 16 entries ----
                if constexpr (kBatch) {
                    constexpr int kVB = 8;
#pragma unroll
                    for (int d0 = 0; d0 < VE; d0 += kVB) {
                        u32x4 va[kVB];
#pragma unroll
                        for (int u = 0; u < kVB; ++u) {
                            const int dblk = d0 + u;
                            const int off = lo.vtr[dblk & 7] + 256 * (dblk >> 3);
                            const u32x2 v0 = lds_read_tr16(vt + off);
                            const u32x2 v1 = lds_read_tr16(vt + 16 * T::kMainPitch + off);
                            va[u] = u32x4{v0.x, v0.y, v1.x, v1.y};
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int u = 0; u < kVB; ++u) o[d0 + u] = mfma_bf16_16x16x32(va[u], pop, o[d0 + u]);
                    }
                } else {
#pragma unroll
                    for (int dblk = 0; dblk < VE; ++dblk) {
                        const int off = lo.vtr[dblk & 7] + 256 * (dblk >> 3);
                        const u32x2 v0 = lds_read_tr16(vt + off);
                        const u32x2 v1 = lds_read_tr16(vt + 16 * T::kMainPitch + off);
                        o[dblk] = mfma_bf16_16x16x32(u32x4{v0.x, v0.y, v1.x, v1.y}, pop, o[dblk]);
                    }
                }
            };
            if constexpr (PC) {
                // the consumer wave (the producer took its own path above)
                for (int i = 0; i < ct; ++i) {
                    __syncthreads();                  // tile i is in buffer i & 1
                    const uint8_t* kt = (i & 1) ? sm_k1 : sm_k0;
                    compute(i, kt, kt);
                }
            } else {
                mla_stage<DQK, DV, NW, ALIAS>(ch, tile0, uniform, sm_k0, sm_v0, wv, lane);
                wait_vm0();
                __syncthreads();
                for (int i = 0; i < ct; ++i) {
                    const uint8_t* kt = (i & 1) ? sm_k1 : sm_k0;
                    const uint8_t* vt = ALIAS ? kt : ((i & 1) ? sm_v1 : sm_v0);
                    if (i + 1 < ct)
                        mla_stage<DQK, DV, NW, ALIAS>(ch, tile0 + (i + 1) * kTile, uniform,
                                                      (i & 1) ? sm_k0 : sm_k1,
                                                      (i & 1) ? sm_v0 : sm_v1, wv, lane);
                    compute(i, kt, vt);
                    wait_vm0();
                    __syncthreads();
                }
            }
        }

        // ---- finish the piece: row cg, entries 16dblk + 4grp + j ----
        const float lt = col4_sum(l);
        if (cg < p.rows) {
            if (complete) {
                // a sink logit joins the normaliser (no value row)
                float den = lt;
                if (p.sinks) den += fast_exp2(p.sinks[kvh * G + cg] * kLog2e - m);
                const float inv = lt > 0.f ? vsc / den : 0.f;
                uint16_t* orow = static_cast<uint16_t*>(p.out) + (int64_t)b * p.out_stride_b +
                                 (int64_t)(kvh * G + cg) * DV;
#pragma unroll
                for (int dblk = 0; dblk < VE; ++dblk)
                    *reinterpret_cast<u32x2*>(orow + 16 * dblk + 4 * grp) =
                        u32x2{pack_bf16x2(o[dblk][0] * inv, o[dblk][1] * inv),
                              pack_bf16x2(o[dblk][2] * inv, o[dblk][3] * inv)};
            } else {
                const int64_t row = part_row(p, w, slot) + cg;
                const float inv = lt > 0.f ? vsc / lt : 0.f;
                float* po = p.part_o + row * DV;
#pragma unroll
                for (int dblk = 0; dblk < VE; ++dblk)
                    *reinterpret_cast<f32x4*>(po + 16 * dblk + 4 * grp) = o[dblk] * inv;
                if (grp == 0) p.part_lse[row] = lt > 0.f ? m + __log2f(lt) : -INFINITY;
            }
        }

        next_piece();
    }
}

using MlaFn = void (*)(DecodeParams);

template <int DQK, int DV, bool ALIAS>
MlaFn mla_by_waves(int nw, bool pc) {
    if (pc) return ALIAS && nw == 2 ? mla_split_kernel<DQK, DV, 2, true, true> : nullptr;
    switch (nw) {
        case 2: return mla_split_kernel<DQK, DV, 2, ALIAS, false>;
        case 4: return mla_split_kernel<DQK, DV, 4, ALIAS, false>;
        case 8: return mla_split_kernel<DQK, DV, 8, ALIAS, false>;
        default: return nullptr;
    }
}

// rows: query rows per kv head.  Two-wave blocks over one pool with at most
// 16 rows are producer/consumer blocks.
MlaFn mla_kernel(int dqk, int dv, bool alias, int nw, int rows) {
    const bool pc = alias && nw == 2 && rows <= 16;
    if (dqk == 576 && dv == 512)
        return alias ? mla_by_waves<576, 512, true>(nw, pc)
                     : mla_by_waves<576, 512, false>(nw, pc);
    if (dqk == 288 && dv == 256)
        return alias ? mla_by_waves<288, 256, true>(nw, pc)
                     : mla_by_waves<288, 256, false>(nw, pc);
    return nullptr;
}

}  // namespace

hipError_t launch_mla_decode(const DecodeParams& p, int head_dim, int head_dim_v, bool alias,
                             int waves_per_block, int workers, hipStream_t stream) {
    const MlaFn f = mla_kernel(head_dim, head_dim_v, alias, waves_per_block, p.rows);
    if (!f) return hipErrorInvalidValue;
    hipLaunchKernelGGL(f, dim3(workers), dim3(64 * waves_per_block), 0, stream, p);
    return hipGetLastError();
}

hipError_t mla_blocks_per_cu(int head_dim, int head_dim_v, bool alias, int waves_per_block,
                             int rows, int* out) {
    const MlaFn f = mla_kernel(head_dim, head_dim_v, alias, waves_per_block, rows);
    if (!f) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, reinterpret_cast<const void*>(f),
                                                        64 * waves_per_block, 0);
}

}  // namespace pa
