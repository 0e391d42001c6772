// decode.hip -- split-KV paged GQA decode for gfx950.
//
// The computation is the split-KV scheme of `_fwd_grouped_kernel_stage1`
// (partial softmax-weighted sums with their log-sum-exp over contiguous
// pieces of a sequence's key range) and `_fwd_kernel_stage2` (merge of the
// pieces) on the page "vllm/attention/ops/triton_decode_attention.py".  Any
// contiguous partition of the key range gives the same result, so the
// partition here is chosen for the machine (stream-K):
//
//   * a segment is one (sequence b, kv head g): the 32-token tiles covering
//     the key range [lo, L) (lo = L - W under a sliding window, tiles start at
//     lo rounded down to 32);
//   * all segments are laid end to end (sequence-major, kv head minor) and
//     the resulting list of N tiles is cut into W equal contiguous ranges, W
//     = the persistent waves the chip holds; wave w owns tiles
//     [floor(w*N/W), floor((w+1)*N/W));
//   * a wave walks its range; a segment it covers completely is normalised
//     and written to the output directly, the (at most two) segments it
//     covers in part leave a partial (normalised sum + log2-sum-exp) in the
//     wave's two workspace slots;
//   * a second kernel merges the partials of every segment that spans
//     several waves (the merge of `_fwd_kernel_stage2`) and writes zero rows
//     for sequences with no keys.
//
// Every wave gets the same number of tiles whatever the length mix, and no
// wave waits for another.
//
// Per tile one wave computes, for all G query heads of the kv head at once
// (every K/V byte is read once for the whole group):
//   S^T[32 x 16] = K[32 x D] * Q^T[D x 16]       (v_mfma_f32_16x16x32_bf16;
//                                                 K rows are loaded whole and
//                                                 re-read from a per-wave LDS
//                                                 tile in the A layout)
//   online softmax in the log2 domain (scores of one head live in the 4 lanes
//   of one MFMA column; max by two cross-lane exchanges)
//   O[16 x D] += P[16 x 32] * V[32 x D]          (P is the S^T accumulator
//                                                 re-read as the A operand; V
//                                                 rows are loaded 16 bytes per
//                                                 lane and transposed in
//                                                 registers with v_perm)
// Rows of Q^T beyond G are zero; their results are never stored.
//
// Memory: every lane load is 16 bytes (8 bytes for fp8 V / D=64 bf16 V) of a
// K or V row, nontemporal; one wave load instruction covers whole rows (4 of
// K or V for bf16 D=128).  A wave keeps the next tile's K and V in flight
// while it computes the current one.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// Position (0..31) inside a tile of the token that MFMA contraction slot
// (grp, j) stands for in the P*V product.  Tokens 4*grp + j (j < 4) come from
// the first 16-token half of S^T, 16 + 4*grp + (j - 4) from the second half;
// with this choice the S^T accumulator is already the P operand.
__device__ __forceinline__ int tile_token(int grp, int j) {
    return (j < 4) ? 4 * grp + j : 16 + 4 * grp + (j - 4);
}

template <bool FP8>
__device__ __forceinline__ const uint8_t* row_ptr(const void* pool, int64_t page, int row,
                                                  int head, int64_t s_page, int64_t s_tok,
                                                  int64_t s_head) {
    constexpr int64_t kElem = FP8 ? 1 : 2;
    return static_cast<const uint8_t*>(pool) +
           (page * s_page + (int64_t)row * s_tok + (int64_t)head * s_head) * kElem;
}

// V bytes per lane per token: D/16 elements.
template <int BYTES>
struct VChunk;
template <>
struct VChunk<16> {
    using T = u32x4;
    static __device__ __forceinline__ T zero() { return T{0, 0, 0, 0}; }
};
template <>
struct VChunk<8> {
    using T = u32x2;
    static __device__ __forceinline__ T zero() { return T{0, 0}; }
};
template <>
struct VChunk<4> {
    using T = uint32_t;
    static __device__ __forceinline__ T zero() { return 0u; }
};

// dword `i` of a V chunk after conversion to bf16 pairs.
template <int D, bool FP8>
struct VRow {
    static constexpr int kVE = D / 16;                 // elements per lane per token
    static constexpr int kBytes = kVE * (FP8 ? 1 : 2);
    using Raw = typename VChunk<kBytes>::T;
    uint32_t w[kVE / 2];                               // bf16 pairs

    __device__ __forceinline__ void from_raw(Raw r) {
        if constexpr (!FP8) {
            if constexpr (kVE == 8) { w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w; }
            else { w[0] = r.x; w[1] = r.y; }
        } else {
            if constexpr (kVE == 8) {
                u32x2 a = e4m3x4_to_bf16x4(r.x), b = e4m3x4_to_bf16x4(r.y);
                w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y;
            } else {
                u32x2 a = e4m3x4_to_bf16x4(r);
                w[0] = a.x; w[1] = a.y;
            }
        }
    }
};

// Addressing of one split.  Page ids come from the split's page list in LDS
// (pages[i] = block_table[b][first_page + i]); the list index is clamped into
// the list, so every address lies inside a page of the split whatever the
// token: rows outside [t_begin, t_end) are read but their scores are masked
// and their V rows zeroed by the consumer.  Per-lane parts of the addresses
// that do not change from tile to tile are precomputed (bytes).
struct TileCtx {
    const int* pages;
    int first_page, last_idx, t_begin, t_end, c, grp;
    int64_t page_bytes;        // s_page * elem
    int tok_bytes;             // s_tok * elem
    int k_lane;                // kvh*s_head*elem + 16*grp (+ c*tok_bytes when UNIFORM)
    int k_row;                 // whole-row K loads: the lane's row within a load
    int k_row_lane;            // kvh*s_head*elem + 16*column (+ k_row*tok_bytes when UNIFORM)
    int v_lane[4];             // kvh*s_head*elem + VBYTES*c (+ (4*grp + r)*tok_bytes when UNIFORM)
};

template <bool UNIFORM>
__device__ __forceinline__ int64_t page_of(const TileCtx& x, int pshift, int t) {
    const int idx = min(max((t >> pshift) - x.first_page, 0), x.last_idx);
    if constexpr (UNIFORM)   // one page for the whole wave: keep it scalar
        return (int64_t)__builtin_amdgcn_readfirstlane(x.pages[idx]);
    return (int64_t)x.pages[idx];
}

// Streaming loads of K/V rows: every byte is read once, so they bypass
// cache retention (nontemporal).
template <typename T>
__device__ __forceinline__ T load_stream(const uint8_t* ptr) {
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(ptr));
}

// K rows of a tile as S^T A operands: tokens 16h + c, h = 0, 1.  Load i of a
// half reads the 16 bytes at 64*i of the lane's slice of the row.
template <int D, bool FP8>
struct KRegs {
    static constexpr int N = FP8 ? D / 64 : D / 32;   // 16-byte loads per half
    u32x4 w[2][N];
};

template <int D, bool FP8, bool UNIFORM>
__device__ __forceinline__ void issue_k(KRegs<D, FP8>& R, const DecodeParams& p,
                                        const TileCtx& x, int t0) {
    const uint8_t* pool = static_cast<const uint8_t*>(p.k_pool);
    const int pmask = (1 << p.page_shift) - 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint8_t* ptr;
        if constexpr (UNIFORM) {
            // page_size is a multiple of 16: the half sits in one page
            const int th = t0 + 16 * h;
            const uint8_t* base = pool + page_of<true>(x, p.page_shift, th) * x.page_bytes +
                                  (int64_t)((th & pmask) * x.tok_bytes);
            ptr = base + x.k_lane;
        } else {
            const int t = t0 + 16 * h + x.c;
            ptr = pool + page_of<false>(x, p.page_shift, t) * x.page_bytes +
                  (int64_t)((t & pmask) * x.tok_bytes + x.k_lane);
        }
        // (plain loads: each 128-byte line of a row is read by two
        // consecutive instructions, and the second must find it cached)
#pragma unroll
        for (int i = 0; i < KRegs<D, FP8>::N; ++i)
            R.w[h][i] = *reinterpret_cast<const u32x4*>(ptr + 64 * i);
    }
}

// K rows of a tile loaded whole (every wave load instruction reads complete
// rows, rows_per_load of them), to be transposed through LDS into the S^T A
// operands.  Row `rows_per_load*i + lane/lanes_per_row` of the tile, 16 bytes
// at 16*(lane % lanes_per_row).
template <int D, bool FP8>
struct KRowRegs {
    static constexpr int kRowBytes = D * (FP8 ? 1 : 2);
    static constexpr int kLanesPerRow = kRowBytes / 16;
    static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
    static constexpr int N = kTile / kRowsPerLoad;          // loads per tile
    static constexpr int kLdsStride = kRowBytes + 16;       // padded LDS row
    u32x4 w[N];
};

template <int D, bool FP8, bool UNIFORM>
__device__ __forceinline__ void issue_k_rows(KRowRegs<D, FP8>& R, const DecodeParams& p,
                                             const TileCtx& x, int t0) {
    using KR = KRowRegs<D, FP8>;
    const uint8_t* pool = static_cast<const uint8_t*>(p.k_pool);
    const int pmask = (1 << p.page_shift) - 1;
#pragma unroll
    for (int i = 0; i < KR::N; ++i) {
        const int row0 = KR::kRowsPerLoad * i;              // first row of this load
        const uint8_t* ptr;
        if constexpr (UNIFORM) {
            const int th = t0 + (row0 & 16);               // the half holding the rows
            ptr = pool + page_of<true>(x, p.page_shift, th) * x.page_bytes +
                  (int64_t)(((th & pmask) + (row0 & 15)) * x.tok_bytes) + x.k_row_lane;
        } else {
            const int t = t0 + row0 + x.k_row;
            ptr = pool + page_of<false>(x, p.page_shift, t) * x.page_bytes +
                  (int64_t)((t & pmask) * x.tok_bytes + x.k_row_lane);
        }
        R.w[i] = load_stream<u32x4>(ptr);
    }
}

// Registers -> LDS tile [32 rows][kLdsStride bytes].
template <int D, bool FP8>
__device__ __forceinline__ void stage_k(const KRowRegs<D, FP8>& R, uint8_t* lds, int lane) {
    using KR = KRowRegs<D, FP8>;
    const int row = lane / KR::kLanesPerRow, col = lane % KR::kLanesPerRow;
#pragma unroll
    for (int i = 0; i < KR::N; ++i)
        *reinterpret_cast<u32x4*>(lds + (KR::kRowsPerLoad * i + row) * KR::kLdsStride + 16 * col) =
            R.w[i];
}

// S^T = K Q^T with the K rows read back from the LDS tile in the A layout
// (row 16h + c, the lane's slice as in issue_k).
template <int D, bool FP8>
__device__ __forceinline__ void tile_scores_lds(f32x4 s[2], const uint8_t* lds,
                                                const u32x4* qop, int c, int grp) {
    using KR = KRowRegs<D, FP8>;
    constexpr int NL = FP8 ? D / 64 : D / 32;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint8_t* rowp = lds + (16 * h + c) * KR::kLdsStride + 16 * grp;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(rowp + 64 * i);
            if constexpr (FP8) {
                const u32x2 a = e4m3x4_to_bf16x4(w.x), bb = e4m3x4_to_bf16x4(w.y);
                const u32x2 cc = e4m3x4_to_bf16x4(w.z), dd = e4m3x4_to_bf16x4(w.w);
                s[h] = mfma_bf16_16x16x32(u32x4{a.x, a.y, bb.x, bb.y}, qop[2 * i], s[h]);
                s[h] = mfma_bf16_16x16x32(u32x4{cc.x, cc.y, dd.x, dd.y}, qop[2 * i + 1], s[h]);
            } else {
                s[h] = mfma_bf16_16x16x32(w, qop[i], s[h]);
            }
        }
    }
}

// V chunks of the 8 tokens this lane transposes for P*V.
template <int D, bool FP8>
struct VRegs {
    typename VRow<D, FP8>::Raw w[8];
};

template <int D, bool FP8, bool UNIFORM>
__device__ __forceinline__ void issue_v(VRegs<D, FP8>& R, const DecodeParams& p,
                                        const TileCtx& x, int t0) {
    using Raw = typename VRow<D, FP8>::Raw;
    const uint8_t* pool = static_cast<const uint8_t*>(p.v_pool);
    const int pmask = (1 << p.page_shift) - 1;
    if constexpr (UNIFORM) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int th = t0 + 16 * h;
            const uint8_t* base = pool + page_of<true>(x, p.page_shift, th) * x.page_bytes +
                                  (int64_t)((th & pmask) * x.tok_bytes);
#pragma unroll
            for (int r = 0; r < 4; ++r) R.w[4 * h + r] = load_stream<Raw>(base + x.v_lane[r]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = t0 + tile_token(x.grp, i);
            const uint8_t* ptr = pool + page_of<false>(x, p.page_shift, t) * x.page_bytes +
                                 (int64_t)((t & pmask) * x.tok_bytes + x.v_lane[0]);
            R.w[i] = load_stream<Raw>(ptr);
        }
    }
}

// S^T = K Q^T for one tile: s[h][j] is the score of token 16h + 4*grp + j for
// the head of this lane's column.
template <int D, bool FP8>
__device__ __forceinline__ void tile_scores(f32x4 s[2], const KRegs<D, FP8>& R,
                                            const u32x4* qop) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KRegs<D, FP8>::N; ++i) {
            const u32x4 w = R.w[h][i];
            if constexpr (FP8) {
                const u32x2 a = e4m3x4_to_bf16x4(w.x), bb = e4m3x4_to_bf16x4(w.y);
                const u32x2 cc = e4m3x4_to_bf16x4(w.z), dd = e4m3x4_to_bf16x4(w.w);
                s[h] = mfma_bf16_16x16x32(u32x4{a.x, a.y, bb.x, bb.y}, qop[2 * i], s[h]);
                s[h] = mfma_bf16_16x16x32(u32x4{cc.x, cc.y, dd.x, dd.y}, qop[2 * i + 1], s[h]);
            } else {
                s[h] = mfma_bf16_16x16x32(w, qop[i], s[h]);
            }
        }
    }
}

// Online-softmax state of one wave: running max / partial sum of the head in
// this lane's MFMA column, and O rows 4*grp..4*grp+3 at d = VE*c + e.
template <int D>
struct Acc {
    float m = -INFINITY;
    float l = 0.f;
    f32x4 o[D / 16];
};

// Scores -> probabilities (log2 domain), running max/sum, O rescale.
// Returns the P operand (bf16) of P*V.
template <int D, bool CAP>
__device__ __forceinline__ u32x4 tile_softmax(Acc<D>& A, const f32x4 s[2],
                                              const DecodeParams& p, const TileCtx& x, int t0,
                                              bool full) {
    constexpr int VE = D / 16;
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float v = (j < 4) ? s[0][j] : s[1][j - 4];
        if constexpr (CAP) {
            // c*tanh(y/c) = c - 2c / (exp(2y/c) + 1), times log2(e)
            v = p.cap_c2 - 2.f * p.cap_c2 * fast_rcp(fast_exp2(v * p.cap_c1) + 1.f);
        } else {
            v *= p.qk_scale2;
        }
        sc[j] = v;
    }
    if (!full) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = t0 + tile_token(x.grp, j);
            sc[j] = (t >= x.t_begin && t < x.t_end) ? sc[j] : -INFINITY;
        }
    }
    float tmax = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float m_new = fmaxf(A.m, tmax);
    const float alpha = fast_exp2(A.m - m_new);
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        pr[j] = fast_exp2(sc[j] - m_new);
        psum += pr[j];
    }
    A.l = A.l * alpha + psum;
    A.m = m_new;
    // rescale O: row 4*grp + j belongs to head column 4*grp + j
    float arow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) arow[j] = __shfl(alpha, 4 * x.grp + j, 64);
#pragma unroll
    for (int e = 0; e < VE; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) A.o[e][j] *= arow[j];
    return u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                 pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
}

// O += P V, V rows transposed in registers (v_perm) into B operands.
template <int D, bool FP8>
__device__ __forceinline__ void tile_pv(Acc<D>& A, VRegs<D, FP8>& R, u32x4 pop,
                                        const TileCtx& x, int t0, bool full) {
    constexpr int VE = D / 16;
    using VR = VRow<D, FP8>;
    if (!full) {
        // rows outside the key range may hold anything (NaN included): zero
        // them in place (the buffer is refilled right after)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = t0 + tile_token(x.grp, i);
            R.w[i] = (t >= x.t_begin && t < x.t_end) ? R.w[i] : VChunk<VR::kBytes>::zero();
        }
    }
    VR vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vr[i].from_raw(R.w[i]);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        const bool hi = e & 1;
        const int wd = e >> 1;
        const u32x4 bop = {pick_halves(vr[0].w[wd], vr[1].w[wd], hi),
                           pick_halves(vr[2].w[wd], vr[3].w[wd], hi),
                           pick_halves(vr[4].w[wd], vr[5].w[wd], hi),
                           pick_halves(vr[6].w[wd], vr[7].w[wd], hi)};
        A.o[e] = mfma_bf16_16x16x32(pop, bop, A.o[e]);
        // build each B operand right before its MFMA (keeps 4 registers live,
        // not 4*VE)
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// Segment geometry (shared by the split pass and the merge)
// ---------------------------------------------------------------------------
struct SeqRange {
    int L, lo, base, tiles;   // tiles: 32-token tiles from base covering [lo, L)
};

__device__ __forceinline__ SeqRange seq_range(const DecodeParams& p, int b) {
    SeqRange r;
    r.L = p.seq_lens[b];
    r.lo = (p.window > 0 && r.L > p.window) ? r.L - p.window : 0;
    r.base = r.lo & ~(kTile - 1);
    r.tiles = r.L > r.lo ? (r.L - r.base + kTile - 1) / kTile : 0;
    return r;
}

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k, 64);
    return v;
}

// Total tiles N over all segments (every lane gets the sum).
__device__ __forceinline__ int64_t total_tiles(const DecodeParams& p) {
    const int lane = __lane_id();
    int64_t n = 0;
    for (int b0 = 0; b0 < p.num_seqs; b0 += 64) {
        const int b = b0 + lane;
        n += b < p.num_seqs ? (int64_t)seq_range(p, b).tiles : 0;
    }
    return wave_sum64(n) * p.num_kv_heads;
}

// Sequence whose segments contain global tile `pos` (< N), and the global
// index of its first tile.  Sequences without tiles are skipped.
__device__ __forceinline__ void find_seq(const DecodeParams& p, int64_t pos, int& b_out,
                                         int64_t& start_out) {
    const int lane = __lane_id();
    int64_t carry = 0;
    for (int b0 = 0; b0 < p.num_seqs; b0 += 64) {
        const int b = b0 + lane;
        int64_t n = b < p.num_seqs ? (int64_t)seq_range(p, b).tiles * p.num_kv_heads : 0;
        // inclusive scan across the wave
        int64_t incl = n;
#pragma unroll
        for (int k = 1; k < 64; k <<= 1) {
            const int64_t t = __shfl_up(incl, k, 64);
            if (lane >= k) incl += t;
        }
        const int64_t total = __shfl(incl, 63, 64);
        if (carry + total > pos) {
            const uint64_t hit = __ballot(carry + incl > pos);
            const int j = __builtin_ctzll(hit);
            b_out = b0 + j;
            start_out = carry + __shfl(incl - n, j, 64);
            return;
        }
        carry += total;
    }
    b_out = p.num_seqs;
    start_out = carry;
}

// First tile of wave w's range.
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t N, int64_t W) {
    return w * N / W;
}

// Partial slots of wave w: slot 0 holds its first segment when incomplete,
// slot 1 its last one when incomplete (a middle segment is always complete).
__device__ __forceinline__ int64_t part_row(const DecodeParams& p, int64_t w, int slot) {
    return (w * 2 + slot) * p.group;
}

// Wave holding global tile t: the largest w with floor(w*N/W) <= t.
__device__ __forceinline__ int64_t tile_owner(int64_t t, int64_t N, int64_t W) {
    return ((t + 1) * W + N - 1) / N - 1;
}

// Partial row of wave wv's piece of the segment starting at global tile
// seg0, whose first tile wave w0 owns, or -1 when wv's range is empty
// (possible only when N < W).  The owner's range may start before the
// segment (its piece is then the range's last one: slot 1); a later wave's
// range starts inside the segment (slot 0).
__device__ __forceinline__ int piece_row(const DecodeParams& p, int64_t wv, int64_t w0,
                                         int64_t seg0, int64_t N, int64_t W) {
    if (wv == w0) return (int)part_row(p, wv, range_start(wv, N, W) >= seg0 ? 0 : 1);
    if (N < W && range_start(wv, N, W) == range_start(wv + 1, N, W)) return -1;
    return (int)part_row(p, wv, 0);
}

// ---------------------------------------------------------------------------
// Split pass: persistent waves, one contiguous range of tiles each
// ---------------------------------------------------------------------------
template <int D, bool FP8, bool UNIFORM, bool CAP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kDecodeOccupancy)))
void decode_split_kernel(DecodeParams p) {
    constexpr int KK = D / 32;                  // QK MFMAs per 16-token half
    constexpr int VE = D / 16;                  // PV MFMAs per tile
#if !PA_DECODE_KLDS
    constexpr int SUB = kDecodeSub;
#endif

    const int lane = threadIdx.x;
    const int c = lane & 15;
    const int grp = lane >> 4;
    const int G = p.group;
    const int64_t W = gridDim.x;
    const int64_t w = blockIdx.x;

    __shared__ int sm_pages[kMaxSplitPages];
#if PA_DECODE_KLDS
    __shared__ __attribute__((aligned(16))) uint8_t sm_k[kTile * KRowRegs<D, FP8>::kLdsStride];
#endif

    const int64_t N = total_tiles(p);
    if (w == 0 && lane == 0) p.seq_tile0[p.num_seqs] = N;

    const int64_t r0 = range_start(w, N, W);
    const int64_t r1 = range_start(w + 1, N, W);
    if (r0 >= r1) return;

    int b;
    int64_t seq_start;
    find_seq(p, r0, b, seq_start);
    SeqRange sr = seq_range(p, b);

    // tiles of one chunk whose pages fit the LDS page list
    const int chunk_tiles = ((kMaxSplitPages - 2) << p.page_shift) / kTile;
    constexpr int kElem = FP8 ? 1 : 2;
    constexpr int kVBytes = VRow<D, FP8>::kBytes;

    int64_t pos = r0;
    int slot = 0;
    while (pos < r1) {
        const int n = sr.tiles;                               // > 0 here
        const int kvh = (int)((pos - seq_start) / n);
        const int i0 = (int)((pos - seq_start) % n);
        const int64_t seg_end = seq_start + (int64_t)(kvh + 1) * n;
        const int cnt = (int)(min(r1, seg_end) - pos);
        const bool complete = (i0 == 0) && (cnt == n);
        if (kvh == 0 && i0 == 0 && lane == 0) p.seq_tile0[b] = seq_start;

        // ---- Q^T as the B operand: column c = query head kvh*G + c ----
        // The contraction index (grp, j) of MFMA kk stands for d = dq(kk, grp)
        // + j; for fp8 K one 16-byte load feeds two consecutive MFMAs.
        u32x4 qop[KK];
        {
            const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                                   (int64_t)b * p.q_stride_b +
                                   (int64_t)(kvh * G + (c < G ? c : 0)) * D;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int d0 = FP8 ? 64 * (kk / 2) + 16 * grp + 8 * (kk % 2) : 32 * kk + 8 * grp;
                const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + d0);
                qop[kk] = (c < G) ? v : u32x4{0, 0, 0, 0};
            }
        }

        Acc<D> acc;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc.o[e] = f32x4{0.f, 0.f, 0.f, 0.f};

        TileCtx x;
        x.c = c;
        x.grp = grp;
        x.page_bytes = p.s_page * kElem;
        x.tok_bytes = (int)(p.s_tok * kElem);
        {
            const int head = (int)(kvh * p.s_head * kElem);
            x.k_lane = head + 16 * grp + (UNIFORM ? c * x.tok_bytes : 0);
            using KR = KRowRegs<D, FP8>;
            x.k_row = lane / KR::kLanesPerRow;
            x.k_row_lane = head + 16 * (lane % KR::kLanesPerRow) +
                           (UNIFORM ? x.k_row * x.tok_bytes : 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x.v_lane[r] = head + kVBytes * c + (UNIFORM ? (4 * grp + r) * x.tok_bytes : 0);
        }
        x.pages = sm_pages;

        // ---- the piece's tiles, chunk by chunk (page list staged in LDS) ----
        for (int c0 = 0; c0 < cnt; c0 += chunk_tiles) {
            const int ct = min(cnt - c0, chunk_tiles);
            const int tile0 = sr.base + (i0 + c0) * kTile;
            x.t_begin = max(tile0, sr.lo);
            x.t_end = min(tile0 + ct * kTile, sr.L);
            x.first_page = x.t_begin >> p.page_shift;
            const int n_pages = ((x.t_end - 1) >> p.page_shift) - x.first_page + 1;
            x.last_idx = n_pages - 1;
            __syncthreads();     // previous chunk's readers are done with the list
            {
                const int32_t* bt_row =
                    p.block_table + (int64_t)b * p.bt_stride + x.first_page;
                for (int i = lane; i < n_pages; i += 64) sm_pages[i] = bt_row[i];
            }
            __syncthreads();

#if PA_DECODE_KLDS
            // K rows are loaded whole (nontemporal) and transposed through the
            // wave's LDS tile; the registers are free for the next tile's K as
            // soon as they are staged, V rotates as below.  The last tile is
            // peeled off so the steady loop issues its loads unconditionally.
            {
                KRowRegs<D, FP8> kr;
                VRegs<D, FP8> vr;
                auto tile_t0 = [&](int i) { return tile0 + min(i, ct - 1) * kTile; };
                issue_k_rows<D, FP8, UNIFORM>(kr, p, x, tile_t0(0));
                issue_v<D, FP8, UNIFORM>(vr, p, x, tile_t0(0));
                for (int i = 0; i + 1 < ct; ++i) {
                    const int t0 = tile_t0(i);
                    const bool full = (t0 >= x.t_begin) && (t0 + kTile <= x.t_end);
                    stage_k<D, FP8>(kr, sm_k, lane);
                    __syncthreads();
                    issue_k_rows<D, FP8, UNIFORM>(kr, p, x, tile_t0(i + 1));
                    f32x4 s[2];
                    tile_scores_lds<D, FP8>(s, sm_k, qop, c, grp);
                    const u32x4 pop = tile_softmax<D, CAP>(acc, s, p, x, t0, full);
                    tile_pv<D, FP8>(acc, vr, pop, x, t0, full);
                    __syncthreads();
                    issue_v<D, FP8, UNIFORM>(vr, p, x, tile_t0(i + 1));
                }
                const int t0 = tile_t0(ct - 1);
                const bool full = (t0 >= x.t_begin) && (t0 + kTile <= x.t_end);
                stage_k<D, FP8>(kr, sm_k, lane);
                __syncthreads();
                f32x4 s[2];
                tile_scores_lds<D, FP8>(s, sm_k, qop, c, grp);
                const u32x4 pop = tile_softmax<D, CAP>(acc, s, p, x, t0, full);
                tile_pv<D, FP8>(acc, vr, pop, x, t0, full);
                __syncthreads();
            }
#else
            // K and V rotate through one register set each, holding SUB
            // consecutive tiles: the next step's K rows are requested as soon
            // as this step's scores are formed and its V rows as soon as this
            // step's P*V is done.  The last step is peeled off so that the
            // steady-state loop issues its loads unconditionally (exact load
            // counters); a missing tile of the last step is loaded as a repeat
            // of the chunk's last tile and not consumed.
            KRegs<D, FP8> kr[SUB];
            VRegs<D, FP8> vr[SUB];
            const int steps = (ct + SUB - 1) / SUB;
            auto tile_t0 = [&](int i) { return tile0 + min(i, ct - 1) * kTile; };
#pragma unroll
            for (int u = 0; u < SUB; ++u) issue_k<D, FP8, UNIFORM>(kr[u], p, x, tile_t0(u));
#pragma unroll
            for (int u = 0; u < SUB; ++u) issue_v<D, FP8, UNIFORM>(vr[u], p, x, tile_t0(u));
            for (int st = 0; st + 1 < steps; ++st) {
                f32x4 s[SUB][2];
#pragma unroll
                for (int u = 0; u < SUB; ++u) tile_scores<D, FP8>(s[u], kr[u], qop);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < SUB; ++u)
                    issue_k<D, FP8, UNIFORM>(kr[u], p, x, tile_t0((st + 1) * SUB + u));
#pragma unroll
                for (int u = 0; u < SUB; ++u) {
                    const int t0 = tile_t0(st * SUB + u);
                    const bool full = (t0 >= x.t_begin) && (t0 + kTile <= x.t_end);
                    const u32x4 pop = tile_softmax<D, CAP>(acc, s[u], p, x, t0, full);
                    tile_pv<D, FP8>(acc, vr[u], pop, x, t0, full);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < SUB; ++u)
                    issue_v<D, FP8, UNIFORM>(vr[u], p, x, tile_t0((st + 1) * SUB + u));
            }
            {
                const int st = steps - 1;
#pragma unroll
                for (int u = 0; u < SUB; ++u) {
                    if (st * SUB + u < ct) {
                        const int t0 = tile_t0(st * SUB + u);
                        const bool full = (t0 >= x.t_begin) && (t0 + kTile <= x.t_end);
                        f32x4 s[2];
                        tile_scores<D, FP8>(s, kr[u], qop);
                        const u32x4 pop = tile_softmax<D, CAP>(acc, s, p, x, t0, full);
                        tile_pv<D, FP8>(acc, vr[u], pop, x, t0, full);
                    }
                }
            }
#endif
        }

        // ---- finish the piece: sum over the 4 lanes of each column, then
        // row r = 4*grp + j of O (head of column r) is normalised and stored ----
        float l_tot = acc.l + shfl_xor(acc.l, 16);
        l_tot += shfl_xor(l_tot, 32);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            const float lr = __shfl(l_tot, r, 64);
            const float mr = __shfl(acc.m, r, 64);
            if (r < G) {
                const float inv = p.v_scale / lr;
                if (complete) {
                    uint16_t* o16 = static_cast<uint16_t*>(p.out) +
                                    (int64_t)b * p.out_stride_b +
                                    (int64_t)(kvh * G + r) * D + VE * c;
                    uint32_t wv[VE / 2];
#pragma unroll
                    for (int e = 0; e < VE; e += 2)
                        wv[e / 2] = pack_bf16x2(acc.o[e][j] * inv, acc.o[e + 1][j] * inv);
                    if constexpr (VE == 8)
                        *reinterpret_cast<u32x4*>(o16) = u32x4{wv[0], wv[1], wv[2], wv[3]};
                    else
                        *reinterpret_cast<u32x2*>(o16) = u32x2{wv[0], wv[1]};
                } else {
                    const int64_t row = part_row(p, w, slot) + r;
                    float* po = p.part_o + row * D + VE * c;
#pragma unroll
                    for (int e = 0; e < VE; e += 4)
                        *reinterpret_cast<f32x4*>(po + e) =
                            f32x4{acc.o[e][j] * inv, acc.o[e + 1][j] * inv,
                                  acc.o[e + 2][j] * inv, acc.o[e + 3][j] * inv};
                    if (c == 0) p.part_lse[row] = mr + __log2f(lr);
                }
            }
        }

        // ---- next piece ----
        pos += cnt;
        slot = 1;
        if (pos < r1 && pos == seq_start + (int64_t)n * p.num_kv_heads) {
            seq_start = pos;
            do {
                ++b;
                sr = seq_range(p, b);
            } while (sr.tiles == 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Merge: one block per (segment, query-head row r).  Segments inside one
// wave's range were written by the split pass; the others are combined here
// from the partials of the waves that cover them,
//   out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M)    (`_fwd_kernel_stage2`).
// Threads are (column quad q, piece lane pl): each folds the pieces
// pl, pl + kR, ... of its four columns into a running (max, sum, acc) --
// the log-sum-exp values and the partial rows are loaded in the same round --
// and the kR piece lanes are then combined through LDS.  Sequences with no
// keys get zero rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int num_workers) {
    constexpr int kQ = D / 4;                // threads per row, 4 columns each
    constexpr int kR = 256 / kQ;             // piece lanes
    constexpr int kBatch = 4;                // pieces in flight per thread
    const int G = p.group;
    const int r = blockIdx.x % G;
    const int seg = blockIdx.x / G;
    const int kvh = seg % p.num_kv_heads;
    const int b = seg / p.num_kv_heads;
    const int q = threadIdx.x % kQ, pl = threadIdx.x / kQ;
    const SeqRange sr = seq_range(p, b);
    uint16_t* out = static_cast<uint16_t*>(p.out) + (int64_t)b * p.out_stride_b +
                    (int64_t)(kvh * G + r) * D + 4 * q;
    if (sr.tiles == 0) {
        if (pl == 0) *reinterpret_cast<u32x2*>(out) = u32x2{0u, 0u};
        return;
    }
    // N tiles in all and the first global tile of this segment, as the split
    // pass found them
    const int64_t N = p.seq_tile0[p.num_seqs];
    const int64_t seg0 = p.seq_tile0[b] + (int64_t)kvh * sr.tiles;
    const int64_t W = num_workers;
    const int64_t w0 = tile_owner(seg0, N, W), w1 = tile_owner(seg0 + sr.tiles - 1, N, W);
    if (w0 == w1) return;                    // written whole by one wave
    const int64_t npieces = w1 - w0 + 1;

    float m = -INFINITY, sum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i0 = pl; i0 < npieces; i0 += kR * kBatch) {
        float lse[kBatch];
        f32x4 o[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t i = i0 + (int64_t)kR * u;
            const int row = i < npieces ? piece_row(p, w0 + i, w0, seg0, N, W) : -1;
            lse[u] = -INFINITY;
            o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (row >= 0) {
                lse[u] = p.part_lse[row + r];
                o[u] = *reinterpret_cast<const f32x4*>(p.part_o + (int64_t)(row + r) * D + 4 * q);
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
            const float w = lse[u] == -INFINITY ? 0.f : fast_exp2(lse[u] - mn);
            sum += w;
            acc += w * o[u];
        }
        m = mn;
    }

    __shared__ float sm_m[kR], sm_s[kR];
    __shared__ f32x4 sm_acc[kR][kQ];
    if (q == 0) {
        sm_m[pl] = m;
        sm_s[pl] = sum;
    }
    sm_acc[pl][q] = acc;
    __syncthreads();
    if (pl == 0) {
        float M = sm_m[0];
#pragma unroll
        for (int j = 1; j < kR; ++j) M = fmaxf(M, sm_m[j]);
        float S = 0.f;
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kR; ++j) {
            const float f = sm_m[j] == -INFINITY ? 0.f : fast_exp2(sm_m[j] - M);
            S += f * sm_s[j];
            a += f * sm_acc[j][q];
        }
        const float inv = 1.f / S;
        *reinterpret_cast<u32x2*>(out) =
            u32x2{pack_bf16x2(a.x * inv, a.y * inv), pack_bf16x2(a.z * inv, a.w * inv)};
    }
}

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

template <int D, bool FP8, bool UNIFORM>
hipError_t launch_decode_t(const DecodeParams& p, int workers, hipStream_t stream) {
    dim3 grid(workers);
    if (p.has_cap)
        hipLaunchKernelGGL((decode_split_kernel<D, FP8, UNIFORM, true>), grid, dim3(64), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, FP8, UNIFORM, false>), grid, dim3(64), 0,
                           stream, p);
    return hipGetLastError();
}

template <int D, bool FP8, bool UNIFORM>
const void* split_kernel_ptr() {
    return reinterpret_cast<const void*>(&decode_split_kernel<D, FP8, UNIFORM, false>);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, bool fp8, bool uniform_pages,
                         int workers, hipStream_t stream) {
    if (head_dim == 128) {
        if (fp8) return uniform_pages ? launch_decode_t<128, true, true>(p, workers, stream)
                                      : launch_decode_t<128, true, false>(p, workers, stream);
        return uniform_pages ? launch_decode_t<128, false, true>(p, workers, stream)
                             : launch_decode_t<128, false, false>(p, workers, stream);
    }
    if (fp8) return uniform_pages ? launch_decode_t<64, true, true>(p, workers, stream)
                                  : launch_decode_t<64, true, false>(p, workers, stream);
    return uniform_pages ? launch_decode_t<64, false, true>(p, workers, stream)
                         : launch_decode_t<64, false, false>(p, workers, stream);
}

hipError_t decode_waves_per_cu(int head_dim, bool fp8, bool uniform_pages, int* out) {
    const void* f;
    if (head_dim == 128)
        f = fp8 ? (uniform_pages ? split_kernel_ptr<128, true, true>()
                                 : split_kernel_ptr<128, true, false>())
                : (uniform_pages ? split_kernel_ptr<128, false, true>()
                                 : split_kernel_ptr<128, false, false>());
    else
        f = fp8 ? (uniform_pages ? split_kernel_ptr<64, true, true>()
                                 : split_kernel_ptr<64, true, false>())
                : (uniform_pages ? split_kernel_ptr<64, false, true>()
                                 : split_kernel_ptr<64, false, false>());
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, f, 64, 0);
}

hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, int workers, int B,
                               int Hkv, hipStream_t stream) {
    dim3 grid((unsigned)B * Hkv * p.group);
    if (head_dim == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(256), 0, stream, p, workers);
    else
        hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(256), 0, stream, p, workers);
    return hipGetLastError();
}

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
