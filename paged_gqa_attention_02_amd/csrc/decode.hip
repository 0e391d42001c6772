// decode.hip -- split-KV paged GQA decode for gfx950.
//
// One work item is (sequence b, kv head g, split s): the tokens
// [base + s*T, base + (s+1)*T) of the key range [lo, L), where lo = L - W
// under a sliding window, base = lo rounded down to 32 and T the plan's
// tokens_per_split.  This is the split-KV scheme of `_fwd_grouped_kernel_stage1`
// (partial softmax-weighted sum plus its log-sum-exp per split) and
// `_fwd_kernel_stage2` (merge of the splits) on the page
// "vllm/attention/ops/triton_decode_attention.py"; the splits here have a
// fixed token count instead of an equal share of each sequence, so long and
// short sequences produce equally sized work items.
//
// A work item is one block of kDecodeWaves waves; wave w takes the 32-token
// tiles w, w + kDecodeWaves, ... of the split and the waves combine through
// LDS at the end.  Per tile one wave computes, for all G query heads of the
// kv head at once (every K/V byte is read once for the whole group):
//   S^T[32 x 16] = K[32 x D] * Q^T[D x 16]       (v_mfma_f32_16x16x32_bf16,
//                                                 K rows read from HBM straight
//                                                 into the A operand)
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
// K or V row; one wave load instruction for V covers four whole rows.
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
#pragma unroll
        // (plain loads: each 128-byte line of a row is read by two
        // consecutive instructions, and the second must find it cached)
        for (int i = 0; i < KRegs<D, FP8>::N; ++i)
            R.w[h][i] = *reinterpret_cast<const u32x4*>(ptr + 64 * i);
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

template <int D, bool FP8, bool UNIFORM, bool CAP, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kDecodeOccupancy)))
void decode_partial_kernel(DecodeParams p) {
    constexpr int KK = D / 32;                  // QK MFMAs per 16-token half
    constexpr int VE = D / 16;                  // PV MFMAs per tile

    const int lane = threadIdx.x & 63;
    const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15;
    const int grp = lane >> 4;
    // Work items are numbered kv-head fastest, then sequence, then split:
    // blocks are dealt to the 8 XCDs by block id modulo 8, so this keeps the
    // split index (whose upper values exist only for long sequences) out of
    // the XCD choice and gives every XCD an even share of the work.
    const int kvh = blockIdx.x % p.num_kv_heads;
    const int b = (blockIdx.x / p.num_kv_heads) % p.num_seqs;
    const int split = blockIdx.x / (p.num_kv_heads * p.num_seqs);
    const int G = p.group;

    const int L = p.seq_lens[b];
    const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
    const int base = lo & ~(kTile - 1);
    const int T = p.tokens_per_split;
    // (min with the grid: lengths beyond the planned bound cannot index past
    // the partials)
    const int n_splits = L > lo ? min((L - base + T - 1) / T, p.num_splits) : 0;

    __shared__ int sm_pages[kMaxSplitPages];

    if (split >= n_splits) {
        if (split == 0) {   // nothing to attend: zero rows
            for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
                const int r = idx / D, d = idx % D;
                uint16_t* o = static_cast<uint16_t*>(p.out) + (int64_t)b * p.out_stride_b +
                              (int64_t)(kvh * G + r) * D + d;
                *o = 0;
            }
        }
        return;
    }

    const int chunk0 = base + split * T;
    const int t_begin = max(chunk0, lo);
    const int t_end = min(chunk0 + T, L);
    const int n_tiles = (t_end - chunk0 + kTile - 1) / kTile;

    // The split's page list, once, into LDS: every later page lookup is an
    // LDS read instead of a dependent global load.
    const int first_page = t_begin >> p.page_shift;
    const int n_pages = ((t_end - 1) >> p.page_shift) - first_page + 1;
    {
        const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride + first_page;
        for (int i = threadIdx.x; i < n_pages; i += NW * 64) sm_pages[i] = bt_row[i];
    }

    // Q^T as the B operand: column c = query head kvh*G + c.  The contraction
    // index (grp, j) of MFMA kk stands for d = dq(kk, grp) + j; for fp8 K one
    // 16-byte load feeds two consecutive MFMAs, hence the different order.
    u32x4 qop[KK];
    {
        const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_stride_b +
                               (int64_t)(kvh * G + (c < G ? c : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int d0 = FP8 ? 64 * (kk / 2) + 16 * grp + 8 * (kk % 2) : 32 * kk + 8 * grp;
            u32x4 v = *reinterpret_cast<const u32x4*>(qrow + d0);
            qop[kk] = (c < G) ? v : u32x4{0, 0, 0, 0};
        }
    }
    __syncthreads();

    Acc<D> acc;
#pragma unroll
    for (int e = 0; e < VE; ++e) acc.o[e] = f32x4{0.f, 0.f, 0.f, 0.f};

    TileCtx x;
    {
        constexpr int kElem = FP8 ? 1 : 2;
        constexpr int kVBytes = VRow<D, FP8>::kBytes;
        x.pages = sm_pages;
        x.first_page = first_page;
        x.last_idx = n_pages - 1;
        x.t_begin = t_begin;
        x.t_end = t_end;
        x.c = c;
        x.grp = grp;
        x.page_bytes = p.s_page * kElem;
        x.tok_bytes = (int)(p.s_tok * kElem);
        const int head = (int)(kvh * p.s_head * kElem);
        x.k_lane = head + 16 * grp + (UNIFORM ? c * x.tok_bytes : 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            x.v_lane[r] = head + kVBytes * c + (UNIFORM ? (4 * grp + r) * x.tok_bytes : 0);
    }

    // K and V rotate through one register set each, holding SUB consecutive
    // tiles of this wave: the next step's K rows are requested as soon as
    // this step's scores are formed and its V rows as soon as this step's P*V
    // is done, so about SUB tiles per wave are always in flight.  The last
    // step is peeled off so that the steady-state loop issues its loads
    // unconditionally (exact load counters); a missing tile of the last step
    // is loaded as a repeat of the wave's last tile and not consumed.  This
    // wave's tiles are wave, wave + NW, ...
    constexpr int SUB = kDecodeSub;
    KRegs<D, FP8> kr[SUB];
    VRegs<D, FP8> vr[SUB];
    const int my_tiles = wave < n_tiles ? (n_tiles - wave + NW - 1) / NW : 0;
    const int my_steps = (my_tiles + SUB - 1) / SUB;
    auto tile_t0 = [&](int i) { return chunk0 + (wave + min(i, my_tiles - 1) * NW) * kTile; };
    if (my_tiles > 0) {
#pragma unroll
        for (int u = 0; u < SUB; ++u) issue_k<D, FP8, UNIFORM>(kr[u], p, x, tile_t0(u));
#pragma unroll
        for (int u = 0; u < SUB; ++u) issue_v<D, FP8, UNIFORM>(vr[u], p, x, tile_t0(u));
        for (int st = 0; st + 1 < my_steps; ++st) {
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
                const bool full = (t0 >= t_begin) && (t0 + kTile <= t_end);
                const u32x4 pop = tile_softmax<D, CAP>(acc, s[u], p, x, t0, full);
                tile_pv<D, FP8>(acc, vr[u], pop, x, t0, full);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < SUB; ++u)
                issue_v<D, FP8, UNIFORM>(vr[u], p, x, tile_t0((st + 1) * SUB + u));
        }
        const int st = my_steps - 1;
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
            if (st * SUB + u < my_tiles) {
                const int t0 = tile_t0(st * SUB + u);
                const bool full = (t0 >= t_begin) && (t0 + kTile <= t_end);
                f32x4 s[2];
                tile_scores<D, FP8>(s, kr[u], qop);
                const u32x4 pop = tile_softmax<D, CAP>(acc, s, p, x, t0, full);
                tile_pv<D, FP8>(acc, vr[u], pop, x, t0, full);
            }
        }
    }

    // ---- finish: softmax sum over the 4 lanes of each column ----
    float l_tot = acc.l + shfl_xor(acc.l, 16);
    l_tot += shfl_xor(l_tot, 32);
    const bool direct = (n_splits == 1);
    if constexpr (NW == 1) {
        // Row r = 4*grp + j of O belongs to the head of column r: fetch that
        // column's max and sum, normalise and store this lane's VE values.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            const float lr = __shfl(l_tot, r, 64);
            const float mr = __shfl(acc.m, r, 64);
            if (r < G) {
                const float inv = p.v_scale / lr;
                const int h = kvh * G + r;
                if (direct) {
                    uint16_t* o16 = static_cast<uint16_t*>(p.out) +
                                    (int64_t)b * p.out_stride_b + (int64_t)h * D + VE * c;
                    uint32_t w[VE / 2];
#pragma unroll
                    for (int e = 0; e < VE; e += 2)
                        w[e / 2] = pack_bf16x2(acc.o[e][j] * inv, acc.o[e + 1][j] * inv);
                    if constexpr (VE == 8)
                        *reinterpret_cast<u32x4*>(o16) = u32x4{w[0], w[1], w[2], w[3]};
                    else
                        *reinterpret_cast<u32x2*>(o16) = u32x2{w[0], w[1]};
                } else {
                    const int64_t row = ((int64_t)b * p.num_q_heads + h) * p.num_splits + split;
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
    } else {
        // combine the waves of this block through LDS
        __shared__ float sm_m[NW][16];
        __shared__ float sm_l[NW][16];
        __shared__ float sm_o[NW][16][D];
        if (grp == 0) {
            sm_m[wave][c] = acc.m;
            sm_l[wave][c] = l_tot;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            if (r < G) {
#pragma unroll
                for (int e = 0; e < VE; ++e) sm_o[wave][r][VE * c + e] = acc.o[e][j];
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
            const int r = idx / D, d = idx % D;
            float M = sm_m[0][r];
#pragma unroll
            for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][r]);
            float num = 0.f, lsum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = fast_exp2(sm_m[w][r] - M);
                num += f * sm_o[w][r][d];
                lsum += f * sm_l[w][r];
            }
            const float val = num / lsum * p.v_scale;
            const int h = kvh * G + r;
            if (direct) {
                uint16_t* o16 = static_cast<uint16_t*>(p.out) + (int64_t)b * p.out_stride_b +
                                (int64_t)h * D + d;
                *o16 = (uint16_t)(pack_bf16x2(val, 0.f) & 0xffffu);
            } else {
                const int64_t row = ((int64_t)b * p.num_q_heads + h) * p.num_splits + split;
                p.part_o[row * D + d] = val;
                if (d == 0) p.part_lse[row] = M + __log2f(lsum);
            }
        }
    }
}

// Merge of the split partials of one (sequence, kv head): for each query head,
// out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M)  (`_fwd_kernel_stage2`).
// The per-split weights are formed once per head in LDS.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    const int G = p.group;
    const int L = p.seq_lens[b];
    const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
    const int base = lo & ~(kTile - 1);
    const int T = p.tokens_per_split;
    const int n = L > lo ? min((L - base + T - 1) / T, p.num_splits) : 0;
    if (n <= 1) return;

    __shared__ float wts[16][kMaxSplits];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t row0 = ((int64_t)b * p.num_q_heads + kvh * G) * p.num_splits;

    for (int idx = threadIdx.x; idx < G * n; idx += 256) {
        const int r = idx / n, s = idx % n;
        wts[r][s] = p.part_lse[row0 + (int64_t)r * p.num_splits + s];
    }
    __syncthreads();
    for (int r = wave; r < G; r += 4) {
        float mx = -INFINITY;
        for (int s = lane; s < n; s += 64) mx = fmaxf(mx, wts[r][s]);
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1) mx = fmaxf(mx, shfl_xor(mx, k));
        float sum = 0.f;
        for (int s = lane; s < n; s += 64) {
            const float e = fast_exp2(wts[r][s] - mx);
            wts[r][s] = e;
            sum += e;
        }
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1) sum += shfl_xor(sum, k);
        const float inv = 1.f / sum;
        for (int s = lane; s < n; s += 64) wts[r][s] *= inv;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int r = idx / D, d = idx % D;
        const float* po = p.part_o + (row0 + (int64_t)r * p.num_splits) * D + d;
        float acc = 0.f;
        for (int s = 0; s < n; ++s) acc += wts[r][s] * po[(int64_t)s * D];
        uint16_t* o16 = static_cast<uint16_t*>(p.out) + (int64_t)b * p.out_stride_b +
                        (int64_t)(kvh * G + r) * D + d;
        *o16 = (uint16_t)(pack_bf16x2(acc, 0.f) & 0xffffu);
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
hipError_t launch_decode_t(const DecodeParams& p, int B, int Hkv, hipStream_t stream) {
    dim3 grid(p.num_splits * Hkv * B);
    if (p.has_cap)
        hipLaunchKernelGGL((decode_partial_kernel<D, FP8, UNIFORM, true, kDecodeWaves>),
                           grid, dim3(kDecodeWaves * 64), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_partial_kernel<D, FP8, UNIFORM, false, kDecodeWaves>),
                           grid, dim3(kDecodeWaves * 64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int head_dim, bool fp8, bool uniform_pages,
                         int B, int Hkv, hipStream_t stream) {
    if (head_dim == 128) {
        if (fp8) return uniform_pages ? launch_decode_t<128, true, true>(p, B, Hkv, stream)
                                      : launch_decode_t<128, true, false>(p, B, Hkv, stream);
        return uniform_pages ? launch_decode_t<128, false, true>(p, B, Hkv, stream)
                             : launch_decode_t<128, false, false>(p, B, Hkv, stream);
    }
    if (fp8) return uniform_pages ? launch_decode_t<64, true, true>(p, B, Hkv, stream)
                                  : launch_decode_t<64, true, false>(p, B, Hkv, stream);
    return uniform_pages ? launch_decode_t<64, false, true>(p, B, Hkv, stream)
                         : launch_decode_t<64, false, false>(p, B, Hkv, stream);
}

hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, int B, int Hkv,
                               hipStream_t stream) {
    dim3 grid(Hkv, B);
    if (head_dim == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(256), 0, stream, p);
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
