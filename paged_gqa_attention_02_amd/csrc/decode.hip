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
#include <climits>

#include "decode_geom.h"
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
    int lim, wlo;              // this lane's column: keys t with wlo <= t <= lim (verify)
    float qk2, c1;             // the segment's score scale (or soft-cap factor), log2 units
    float al2;                 // this lane's column: ALiBi slope, log2 units per position
    int full_lo, full_hi;      // tiles inside [full_lo, full_hi) are valid for every column
    int64_t page_bytes;        // s_page * elem
    int tok_bytes;             // s_tok * elem
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

// Loads of K/V rows.  With one wave per block every byte is read once, so
// they bypass cache retention (nontemporal, NT); the waves of a larger block
// read the same rows, and plain loads let the later ones hit in L2.
template <typename T, bool NT>
__device__ __forceinline__ T load_stream(const uint8_t* ptr) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const T*>(ptr));
    else return *reinterpret_cast<const T*>(ptr);
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

template <int D, bool FP8, bool UNIFORM, bool NT>
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
        R.w[i] = load_stream<u32x4, NT>(ptr);
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

// Blocks of NW > 1 waves share each tile: wave wv loads the row groups
// i = wv, wv + NW, ... (kRowsPerLoad rows each) of K and of V and stages them
// into the block's K and V tiles in LDS; every wave then reads its operands
// from those tiles.
template <int D, bool FP8, int NW>
struct SharedRows {
    using KR = KRowRegs<D, FP8>;
    static constexpr int M = (KR::N + NW - 1) / NW;        // row groups per wave
    u32x4 k[M], v[M];
};

template <int D, bool FP8, bool UNIFORM, int NW>
__device__ __forceinline__ void issue_shared(SharedRows<D, FP8, NW>& R, const DecodeParams& p,
                                             const TileCtx& x, int t0, int wv) {
    using KR = KRowRegs<D, FP8>;
    const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
    const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
    const int pmask = (1 << p.page_shift) - 1;
#pragma unroll
    for (int m = 0; m < SharedRows<D, FP8, NW>::M; ++m) {
        const int i = wv + NW * m;
        if (i >= KR::N) break;                              // (uniform per wave)
        const int row0 = KR::kRowsPerLoad * i;
        int64_t off;
        if constexpr (UNIFORM) {
            const int th = t0 + (row0 & 16);
            off = page_of<true>(x, p.page_shift, th) * x.page_bytes +
                  (int64_t)(((th & pmask) + (row0 & 15)) * x.tok_bytes) + x.k_row_lane;
        } else {
            const int t = t0 + row0 + x.k_row;
            off = page_of<false>(x, p.page_shift, t) * x.page_bytes +
                  (int64_t)((t & pmask) * x.tok_bytes + x.k_row_lane);
        }
        R.k[m] = load_stream<u32x4, true>(kpool + off);
        R.v[m] = load_stream<u32x4, true>(vpool + off);
    }
}

template <int D, bool FP8, int NW>
__device__ __forceinline__ void stage_shared(const SharedRows<D, FP8, NW>& R, uint8_t* kl,
                                             uint8_t* vl, int lane, int wv) {
    using KR = KRowRegs<D, FP8>;
    const int row = lane / KR::kLanesPerRow, col = lane % KR::kLanesPerRow;
#pragma unroll
    for (int m = 0; m < SharedRows<D, FP8, NW>::M; ++m) {
        const int i = wv + NW * m;
        if (i >= KR::N) break;
        const int o = (KR::kRowsPerLoad * i + row) * KR::kLdsStride + 16 * col;
        *reinterpret_cast<u32x4*>(kl + o) = R.k[m];
        *reinterpret_cast<u32x4*>(vl + o) = R.v[m];
    }
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

template <int D, bool FP8, bool UNIFORM, bool NT>
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
            for (int r = 0; r < 4; ++r) R.w[4 * h + r] = load_stream<Raw, NT>(base + x.v_lane[r]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = t0 + tile_token(x.grp, i);
            const uint8_t* ptr = pool + page_of<false>(x, p.page_shift, t) * x.page_bytes +
                                 (int64_t)((t & pmask) * x.tok_bytes + x.v_lane[0]);
            R.w[i] = load_stream<Raw, NT>(ptr);
        }
    }
}

// V chunks of the lane's 8 tokens (as issue_v) read from the block's V tile.
template <int D, bool FP8>
__device__ __forceinline__ void read_v_lds(VRegs<D, FP8>& R, const uint8_t* vl, int c,
                                           int grp) {
    using Raw = typename VRow<D, FP8>::Raw;
    using KR = KRowRegs<D, FP8>;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        R.w[i] = *reinterpret_cast<const Raw*>(vl + tile_token(grp, i) * KR::kLdsStride +
                                               VRow<D, FP8>::kBytes * c);
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
// Score modes of the split pass (template flags).
enum SplitScore { kScoreCap = 1, kScoreAlibi = 2 };

template <int D, int SCORE>
__device__ __forceinline__ u32x4 tile_softmax(Acc<D>& A, const f32x4 s[2],
                                              const DecodeParams& p, const TileCtx& x, int t0,
                                              bool full) {
    constexpr int VE = D / 16;
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float v = (j < 4) ? s[0][j] : s[1][j - 4];
        if constexpr ((SCORE & kScoreCap) != 0) {
            // c*tanh(y/c) = c - 2c / (exp(2y/c) + 1), times log2(e)
            v = p.cap_c2 - 2.f * p.cap_c2 * fast_rcp(fast_exp2(v * x.c1) + 1.f);
        } else {
            v *= x.qk2;
        }
        sc[j] = v;
    }
    if constexpr ((SCORE & kScoreAlibi) != 0) {
        // ALiBi: slope * (key - query position), the query sitting at lim
#pragma unroll
        for (int j = 0; j < 8; ++j)
            sc[j] += x.al2 * (float)(t0 + tile_token(x.grp, j) - x.lim);
    }
    if (!full) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = t0 + tile_token(x.grp, j);
            const bool keep = t >= x.t_begin && t < x.t_end && t <= x.lim && t >= x.wlo;
            sc[j] = keep ? sc[j] : -INFINITY;
        }
    }
    float tmax = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
    tmax = col4_max(tmax);
    // Lazy rescale: a head's reference max m moves only when a score exceeds
    // it by more than kSlack (log2 units), so p <= 2^kSlack and O is rescaled
    // on few tiles (every tile has a valid key, so the first one moves m).
    constexpr float kSlack = 8.f;
    const bool move = __any(tmax > A.m + kSlack);
    const float m_new = move ? fmaxf(A.m, tmax) : A.m;
    // (a column with no key yet keeps m = -inf: exponents are taken against 0)
    const float ms = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(A.m - ms);
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        pr[j] = fast_exp2(sc[j] - ms);
        psum += pr[j];
    }
    A.l = A.l * alpha + psum;
    A.m = m_new;
    if (move) {
        // rescale O: row 4*grp + j belongs to head column 4*grp + j
        float arow[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) arow[j] = __shfl(alpha, 4 * x.grp + j, 64);
#pragma unroll
        for (int e = 0; e < VE; ++e)
#pragma unroll
            for (int j = 0; j < 4; ++j) A.o[e][j] *= arow[j];
    }
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
// Split pass: persistent waves, one contiguous range of tiles each
// ---------------------------------------------------------------------------
template <int D, bool FP8, bool UNIFORM, int SCORE, int NW>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(split_waves_per_simd(D, FP8, NW))))
void decode_split_kernel(DecodeParams p) {
    constexpr int KK = D / 32;                  // QK MFMAs per 16-token half
    constexpr int VE = D / 16;                  // PV MFMAs per tile

    // NW waves per block walk the same tiles; wave wv owns the 16 MFMA
    // columns (query rows) 16*wv .. 16*wv + 15 of the segment.
    const int lane = threadIdx.x & 63;
    const int wv = NW == 1 ? 0 : (int)(threadIdx.x >> 6);
    const int c = lane & 15;
    const int grp = lane >> 4;
    const int cg = 16 * wv + c;                 // this lane's query row
    const int G = p.group;
    // With per-head streams (HG = Hkv), block h*Wg + j takes kv head h over
    // range j of that head's stream (the plan makes the block count a
    // multiple of HG), so the blocks of the heads of one token range run side
    // by side; otherwise (HG = 1) one stream holds hm = Hkv segments per
    // sequence.
    const int64_t W = gridDim.x;
    const int64_t w = blockIdx.x;
    const int HG = split_head_groups(p.num_kv_heads);
    const int hm = p.num_kv_heads / HG;
    const int64_t Wg = W / HG;
    const int head0 = (int)(w / Wg);
    if (head0 >= HG) return;                    // (no range: never merged)

    __shared__ int sm_pages[kMaxSplitPages];
    // one wave: its own K tile; several: the block's shared K and V tiles
    __shared__ __attribute__((aligned(16)))
    uint8_t sm_kv[NW == 1 ? 1 : 2][kTile * KRowRegs<D, FP8>::kLdsStride];
    uint8_t* const sm_k = sm_kv[0];
    uint8_t* const sm_v = sm_kv[NW == 1 ? 0 : 1];

    const RangeStart rs = locate_range<FP8>(p, hm, w % Wg, Wg);
    const int64_t N = rs.N, r0 = rs.r0, r1 = rs.r1;
    if (r0 >= r1) {
        // an empty range (N < W): the merge may read this wave's slot 0
        for (int i = threadIdx.x; i < p.rows; i += 64 * NW)
            p.part_lse[part_row(p, w, 0) + i] = -INFINITY;
        return;
    }

    int b = rs.b;
    int64_t seq_start = rs.seq_start;
    SeqRange sr = rs.sr;

    // tiles of one chunk whose pages fit the LDS page list
    const int chunk_tiles = ((kMaxSplitPages - 2) << p.page_shift) / kTile;
    constexpr int kElem = FP8 ? 1 : 2;
    constexpr int kVBytes = VRow<D, FP8>::kBytes;

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
            // this wave owns the segment's first tile: tell the merge which
            // waves cover it
            const int64_t w_last =
                complete ? w : (int64_t)head0 * Wg + tile_owner(seg_end - 1, N, Wg);
            *reinterpret_cast<int4*>(p.seg_rec + 4 * ((int64_t)b * p.num_kv_heads + kvh)) =
                int4{(int)w, (int)w_last, slot, 0};
        }

        // ---- Q^T as the B operand: column c is query row cg = 16*wv + c,
        // token cg / G, head kvh*G + cg % G.  The contraction index (grp, j) of
        // MFMA kk stands for d = dq(kk, grp) + j; for fp8 K one 16-byte load
        // feeds two MFMAs.
        u32x4 qop[KK];
        {
            const int cc = cg < p.rows ? cg : 0;
            const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                                   (int64_t)b * p.q_stride_b + (int64_t)(cc / G) * p.q_stride_t +
                                   (int64_t)(kvh * G + cc % G) * D;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int d0 = FP8 ? 64 * (kk / 2) + 16 * grp + 8 * (kk % 2) : 32 * kk + 8 * grp;
                const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + d0);
                qop[kk] = (cg < p.rows) ? v : u32x4{0, 0, 0, 0};
            }
        }

        Acc<D> acc;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc.o[e] = f32x4{0.f, 0.f, 0.f, 0.f};

        TileCtx x;
        x.c = c;
        x.grp = grp;
        // per-request cache descales of sequence b (uniform loads)
        float vsc = p.v_scale;
        x.qk2 = p.qk_scale2;
        x.c1 = p.cap_c1;
        if (p.k_desc) {
            const float kd = p.k_desc[p.desc_per_seq ? b : 0];
            x.qk2 *= kd;
            x.c1 *= kd;
        }
        if (p.v_desc) vsc *= p.v_desc[p.desc_per_seq ? b : 0];
        x.page_bytes = p.s_page * kElem;
        x.tok_bytes = (int)(p.s_tok * kElem);
        {
            const int head = (int)(kvh * p.s_head * kElem);
            using KR = KRowRegs<D, FP8>;
            x.k_row = lane / KR::kLanesPerRow;
            x.k_row_lane = head + 16 * (lane % KR::kLanesPerRow) +
                           (UNIFORM ? x.k_row * x.tok_bytes : 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x.v_lane[r] = head + kVBytes * c + (UNIFORM ? (4 * grp + r) * x.tok_bytes : 0);
        }
        x.pages = sm_pages;
        // causal limit and window start of this lane's column (query token
        // cg / G at position L - q_len + cg / G); for decode these never bind
        x.lim = sr.L - p.q_len + (cg < p.rows ? cg / G : 0);
        x.al2 = p.alibi ? p.alibi[kvh * G + (cg < p.rows ? cg : 0) % G] * kLog2e : 0.f;
        x.wlo = p.window > 0 ? x.lim - p.window + 1 : INT_MIN;

        // ---- the piece's tiles, chunk by chunk (page list staged in LDS) ----
        for (int c0 = 0; c0 < cnt; c0 += chunk_tiles) {
            const int ct = min(cnt - c0, chunk_tiles);
            const int tile0 = sr.base + (i0 + c0) * kTile;
            x.t_begin = max(tile0, sr.lo);
            x.t_end = min(tile0 + ct * kTile, sr.L);
            x.full_lo = max(x.t_begin, p.window > 0 ? sr.L - p.window : 0);
            x.full_hi = min(x.t_end, sr.L - p.q_len + 1);
            x.first_page = x.t_begin >> p.page_shift;
            const int n_pages = ((x.t_end - 1) >> p.page_shift) - x.first_page + 1;
            x.last_idx = n_pages - 1;
            __syncthreads();     // previous chunk's readers are done with the list
            {
                const int32_t* bt_row =
                    p.block_table + (int64_t)b * p.bt_stride + x.first_page;
                copy_ids_to_lds<8>(sm_pages, bt_row, n_pages, threadIdx.x, 64 * NW);
            }
            __syncthreads();

            // K rows are loaded whole (nontemporal) and transposed through the
            // wave's LDS tile, so their registers take the next tile's K as
            // soon as they are staged; V's registers take the next tile's V
            // once P*V is done.  The last tile is peeled off so the steady
            // loop issues its loads unconditionally (exact load counters).
            if constexpr (NW == 1) {
                KRowRegs<D, FP8> kr;
                VRegs<D, FP8> vr;
                auto tile_t0 = [&](int i) { return tile0 + min(i, ct - 1) * kTile; };
                issue_k_rows<D, FP8, UNIFORM, NW == 1>(kr, p, x, tile_t0(0));
                issue_v<D, FP8, UNIFORM, NW == 1>(vr, p, x, tile_t0(0));
                for (int i = 0; i + 1 < ct; ++i) {
                    const int t0 = tile_t0(i);
                    const bool full = (t0 >= x.full_lo) && (t0 + kTile <= x.full_hi);
                    stage_k<D, FP8>(kr, sm_k, lane);
                    __syncthreads();
                    issue_k_rows<D, FP8, UNIFORM, NW == 1>(kr, p, x, tile_t0(i + 1));
                    f32x4 s[2];
                    tile_scores_lds<D, FP8>(s, sm_k, qop, c, grp);
                    const u32x4 pop = tile_softmax<D, SCORE>(acc, s, p, x, t0, full);
                    tile_pv<D, FP8>(acc, vr, pop, x, t0, full);
                    __syncthreads();
                    issue_v<D, FP8, UNIFORM, NW == 1>(vr, p, x, tile_t0(i + 1));
                }
                const int t0 = tile_t0(ct - 1);
                const bool full = (t0 >= x.full_lo) && (t0 + kTile <= x.full_hi);
                stage_k<D, FP8>(kr, sm_k, lane);
                __syncthreads();
                f32x4 s[2];
                tile_scores_lds<D, FP8>(s, sm_k, qop, c, grp);
                const u32x4 pop = tile_softmax<D, SCORE>(acc, s, p, x, t0, full);
                tile_pv<D, FP8>(acc, vr, pop, x, t0, full);
                __syncthreads();
            } else {
                // NW > 1: each wave loads and stages its share of K and V
                SharedRows<D, FP8, NW> R;
                auto tile_t0 = [&](int i) { return tile0 + min(i, ct - 1) * kTile; };
                issue_shared<D, FP8, UNIFORM, NW>(R, p, x, tile_t0(0), wv);
                for (int i = 0; i < ct; ++i) {
                    const int t0 = tile_t0(i);
                    const bool full = (t0 >= x.full_lo) && (t0 + kTile <= x.full_hi);
                    stage_shared<D, FP8, NW>(R, sm_k, sm_v, lane, wv);
                    __syncthreads();
                    if (i + 1 < ct) issue_shared<D, FP8, UNIFORM, NW>(R, p, x, tile_t0(i + 1), wv);
                    f32x4 s[2];
                    tile_scores_lds<D, FP8>(s, sm_k, qop, c, grp);
                    const u32x4 pop = tile_softmax<D, SCORE>(acc, s, p, x, t0, full);
                    VRegs<D, FP8> vr;
                    read_v_lds<D, FP8>(vr, sm_v, c, grp);
                    tile_pv<D, FP8>(acc, vr, pop, x, t0, full);
                    __syncthreads();
                }
            }
        }

        // ---- finish the piece: sum over the 4 lanes of each column, then
        // row r = 4*grp + j of O (query row rg = 16*wv + r) is normalised and
        // stored ----
        const float l_tot = col4_sum(acc.l);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            const int rg = 16 * wv + r;
            const float lr = __shfl(l_tot, r, 64);
            const float mr = __shfl(acc.m, r, 64);
            if (rg < p.rows) {
                // (a column with no key: zero row, lse = -inf for the merge)
                if (complete) {
                    // a sink logit joins the normaliser (no value row)
                    float den = lr;
                    if (p.sinks)
                        den += fast_exp2(p.sinks[kvh * G + rg % G] * kLog2e - mr);
                    const float inv = lr > 0.f ? vsc / den : 0.f;
                    uint16_t* o16 = static_cast<uint16_t*>(p.out) +
                                    (int64_t)b * p.out_stride_b +
                                    (int64_t)(rg / G) * p.out_stride_t +
                                    (int64_t)(kvh * G + rg % G) * D + VE * c;
                    uint32_t ov[VE / 2];
#pragma unroll
                    for (int e = 0; e < VE; e += 2)
                        ov[e / 2] = pack_bf16x2(acc.o[e][j] * inv, acc.o[e + 1][j] * inv);
                    if constexpr (VE == 8)
                        *reinterpret_cast<u32x4*>(o16) = u32x4{ov[0], ov[1], ov[2], ov[3]};
                    else
                        *reinterpret_cast<u32x2*>(o16) = u32x2{ov[0], ov[1]};
                } else {
                    const float inv = lr > 0.f ? vsc / lr : 0.f;
                    const int64_t row = part_row(p, w, slot) + rg;
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
        pos = min(r1, seg_end);
        slot = 1;
        if (pos < r1 && pos == seq_start + (int64_t)nu * hm) {
            seq_start = pos;
            do {
                ++b;
                sr = seq_range(p, b);
            } while (sr.tiles == 0);
        }
    }
}

using SplitFn = void (*)(DecodeParams);

template <int D, bool FP8, bool UNIFORM, int SCORE>
SplitFn split_by_waves(int nw) {
    switch (nw) {
        case 1: return decode_split_kernel<D, FP8, UNIFORM, SCORE, 1>;
        case 2: return decode_split_kernel<D, FP8, UNIFORM, SCORE, 2>;
        case 3: return decode_split_kernel<D, FP8, UNIFORM, SCORE, 3>;
        case 4: return decode_split_kernel<D, FP8, UNIFORM, SCORE, 4>;
        default: return nullptr;
    }
}

template <int D, bool FP8, bool UNIFORM>
SplitFn split_by_score(int score, int nw) {
    switch (score) {
        case 0: return split_by_waves<D, FP8, UNIFORM, 0>(nw);
        case kScoreCap: return split_by_waves<D, FP8, UNIFORM, kScoreCap>(nw);
        case kScoreAlibi: return split_by_waves<D, FP8, UNIFORM, kScoreAlibi>(nw);
        default: return split_by_waves<D, FP8, UNIFORM, kScoreCap | kScoreAlibi>(nw);
    }
}

template <int D, bool FP8>
SplitFn split_by_pages(bool uniform, int score, int nw) {
    return uniform ? split_by_score<D, FP8, true>(score, nw)
                   : split_by_score<D, FP8, false>(score, nw);
}

SplitFn split_kernel(int head_dim, bool fp8, bool uniform, int score, int nw) {
    if (head_dim == 128)
        return fp8 ? split_by_pages<128, true>(uniform, score, nw)
                   : split_by_pages<128, false>(uniform, score, nw);
    if (head_dim == 64)
        return fp8 ? split_by_pages<64, true>(uniform, score, nw)
                   : split_by_pages<64, false>(uniform, score, nw);
    return nullptr;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, bool fp8, bool uniform_pages,
                         int waves_per_block, int workers, hipStream_t stream) {
    const int score = (p.has_cap ? kScoreCap : 0) | (p.alibi ? kScoreAlibi : 0);
    const SplitFn f = split_kernel(head_dim, fp8, uniform_pages, score, waves_per_block);
    if (!f) return hipErrorInvalidValue;
    hipLaunchKernelGGL(f, dim3(workers), dim3(64 * waves_per_block), 0, stream, p);
    return hipGetLastError();
}

hipError_t decode_blocks_per_cu(int head_dim, bool fp8, bool uniform_pages, int waves_per_block,
                                int* out) {
    const SplitFn f = split_kernel(head_dim, fp8, uniform_pages, 0, waves_per_block);
    if (!f) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, reinterpret_cast<const void*>(f),
                                                        64 * waves_per_block, 0);
}

}  // namespace pa
