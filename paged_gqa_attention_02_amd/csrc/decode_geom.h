// decode_geom.h -- where the decode kernels find things: the address of a
// cached row, and the stream-K cut of all (sequence, kv head) key ranges
// into the split pass's per-wave tile ranges.  Shared by the split pass, the
// merge and the gather.
//
// A segment is one (sequence b, kv head g): the 32-token tiles from
// base = lo rounded down to 32 that cover the key range [lo, L), lo = L - W
// under a sliding window W.  Segments are laid end to end into streams of N
// units, a segment with n tiles taking A + n of them (A = piece_cost: what
// starting a piece costs, in tiles' worth of work, put in front of its first
// tile), and worker w of W owns the tiles whose units fall in
// [floor(w*N/W), floor((w+1)*N/W)) of its stream.  The GQA split pass with
// at most kAlignedHeadsMax kv heads keeps one stream per kv head (its
// sequences' segments in order, hm = 1) and Hkv groups of W/Hkv blocks,
// block h*W/Hkv + j taking kv head h of range j: the blocks reading the
// heads of one token range run at the same time, so the heads' rows of a
// token, which sit together in the pool, are fetched together.  With more kv
// heads, and in the latent split pass, one stream holds all segments,
// sequence-major and (virtual) head minor (hm = heads).
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Address of (page, row, head) of a pool, strides in elements.
template <bool FP8>
__device__ __forceinline__ const uint8_t* row_ptr(const void* pool, int64_t page, int row,
                                                  int head, int64_t s_page, int64_t s_tok,
                                                  int64_t s_head) {
    constexpr int64_t kElem = FP8 ? 1 : 2;
    return static_cast<const uint8_t*>(pool) +
           (page * s_page + (int64_t)row * s_tok + (int64_t)head * s_head) * kElem;
}

struct SeqRange {
    int L, lo, base, tiles;   // tiles: 32-token tiles from base covering [lo, L)
};

// Stream units of one segment with n tiles (none without tiles).
__device__ __forceinline__ int seg_units(const DecodeParams& p, int n) {
    return n > 0 ? n + p.piece_cost : 0;
}

__device__ __forceinline__ SeqRange seq_range(const DecodeParams& p, int b) {
    SeqRange r;
    r.L = p.seq_lens[b];
    // the first query token (position L - q_len) has the earliest window
    r.lo = (p.window > 0 && r.L - p.q_len + 1 > p.window) ? r.L - p.q_len + 1 - p.window : 0;
    r.base = r.lo & ~(kTile - 1);
    r.tiles = r.L > r.lo ? (r.L - r.base + kTile - 1) / kTile : 0;
    return r;
}

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k, 64);
    return v;
}

// Total units N of a stream holding hm segments per sequence (every lane
// gets the sum).
__device__ __forceinline__ int64_t total_tiles(const DecodeParams& p, int hm) {
    const int lane = __lane_id();
    int64_t n = 0;
    for (int b0 = 0; b0 < p.num_seqs; b0 += 64) {
        const int b = b0 + lane;
        n += b < p.num_seqs ? (int64_t)seg_units(p, seq_range(p, b).tiles) : 0;
    }
    return wave_sum64(n) * hm;
}

// Sequence whose segments contain stream unit `pos` (< N), and the stream
// index of its first unit.  Sequences without tiles are skipped.
__device__ __forceinline__ void find_seq(const DecodeParams& p, int hm, int64_t pos, int& b_out,
                                         int64_t& start_out) {
    const int lane = __lane_id();
    int64_t carry = 0;
    for (int b0 = 0; b0 < p.num_seqs; b0 += 64) {
        const int b = b0 + lane;
        int64_t n = b < p.num_seqs ? (int64_t)seg_units(p, seq_range(p, b).tiles) * hm : 0;
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

// First unit of wave w's range.
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t N, int64_t W) {
    return w * N / W;
}

// Where wave (or block) w of W starts: the total N, its range [r0, r1) (in
// stream units), and, when the range is not empty, the sequence b holding
// unit r0, the stream index of b's first unit and b's key range.
struct RangeStart {
    int64_t N, r0, r1, seq_start;
    int b;
    SeqRange sr;
};

// One round of reads for at most 64*E sequences: lane i holds sequences
// E*i .. E*i + E - 1, read together; the lane sums are scanned across the
// wave.
template <int E>
__device__ __forceinline__ RangeStart locate_range_wave(const DecodeParams& p, int hm,
                                                        int64_t w, int64_t W) {
    RangeStart rs;
    const int lane = __lane_id();
    SeqRange mine[E];
    int64_t n[E], lsum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int bb = E * lane + e;
        mine[e] = bb < p.num_seqs ? seq_range(p, bb) : SeqRange{0, 0, 0, 0};
        n[e] = (int64_t)seg_units(p, mine[e].tiles) * hm;
        lsum += n[e];
    }
    int64_t incl = lsum;                      // inclusive scan of the lane sums
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        const int64_t t = __shfl_up(incl, k, 64);
        if (lane >= k) incl += t;
    }
    rs.N = __shfl(incl, 63, 64);
    rs.r0 = range_start(w, rs.N, W);
    rs.r1 = range_start(w + 1, rs.N, W);
    if (rs.r0 >= rs.r1) return rs;
    // the first lane whose sequences end past r0, then the first of its
    // sequences that does (it has tiles)
    const int j = __builtin_ctzll(__ballot(incl > rs.r0));
    int64_t start = __shfl(incl - lsum, j, 64);
    rs.b = E * j + E - 1;
    rs.seq_start = start;
    bool found = false;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t nj = __shfl(n[e], j, 64);
        if (!found && start + nj > rs.r0) {
            found = true;
            rs.b = E * j + e;
            rs.seq_start = start;
            rs.sr = SeqRange{__shfl(mine[e].L, j, 64), __shfl(mine[e].lo, j, 64),
                             __shfl(mine[e].base, j, 64), __shfl(mine[e].tiles, j, 64)};
        }
        start += nj;
    }
    return rs;
}

// Up to 64 sequences (WIDE: up to 256, four a lane): one round of reads;
// more: the lengths are scanned twice (total_tiles, find_seq).  WIDE is for
// the kernels that meet large batches (the fp8 ones); it measured slower for
// the bf16 kernel at 64 sequences although that path does not run there.
template <bool WIDE>
__device__ __forceinline__ RangeStart locate_range(const DecodeParams& p, int hm, int64_t w,
                                                   int64_t W) {
    if (p.num_seqs <= 64) return locate_range_wave<1>(p, hm, w, W);
    if constexpr (WIDE) {
        if (p.num_seqs <= 256) return locate_range_wave<4>(p, hm, w, W);
    }
    RangeStart rs;
    rs.N = total_tiles(p, hm);
    rs.r0 = range_start(w, rs.N, W);
    rs.r1 = range_start(w + 1, rs.N, W);
    if (rs.r0 >= rs.r1) return rs;
    find_seq(p, hm, rs.r0, rs.b, rs.seq_start);
    rs.sr = seq_range(p, rs.b);
    return rs;
}

// Partial slots of wave w: slot 0 holds its first segment when incomplete,
// slot 1 its last one when incomplete (a middle segment is always complete).
__device__ __forceinline__ int64_t part_row(const DecodeParams& p, int64_t w, int slot) {
    return (w * 2 + slot) * p.rows;
}

// Wave holding stream unit t: the largest w with floor(w*N/W) <= t.
__device__ __forceinline__ int64_t tile_owner(int64_t t, int64_t N, int64_t W) {
    return ((t + 1) * W + N - 1) / N - 1;
}

}  // namespace pa
