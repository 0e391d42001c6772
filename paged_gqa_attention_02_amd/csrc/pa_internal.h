// pa_internal.h -- argument blocks shared by the host API and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paged_attn.h"

namespace pa {

// Decode works on tiles of 32 consecutive token positions; every split starts
// on a multiple of 32.
constexpr int kTile = 32;
// Upper bound on the persistent split-pass waves (a forced count included).
constexpr int kMaxWorkers = 1 << 20;
#ifndef PA_DECODE_OCCUPANCY
#define PA_DECODE_OCCUPANCY 2
#endif
constexpr int kDecodeOccupancy = PA_DECODE_OCCUPANCY;   // waves per SIMD the kernel must allow
// Waves per SIMD a split-pass variant is compiled for.  The bf16 D = 128
// one-wave-block variant gets the SIMD's registers to itself (1024 persistent
// waves on 256 compute units): it streams as fast with half the waves, and
// half as many range boundaries leave fewer partials to merge.  The plan asks
// the runtime for the occupancy of the variant it launches.
constexpr int split_waves_per_simd(int head_dim, bool fp8, int waves_per_block) {
    return (head_dim == 128 && !fp8 && waves_per_block == 1) ? 1 : kDecodeOccupancy;
}
// Page-table entries staged in LDS for one chunk of a wave's range: a chunk
// of T tokens touches at most T/page_size + 2 pages.
constexpr int kMaxSplitPages = 2080;
// What starting a piece of a segment costs the split pass, in tiles' worth
// of work (the stream-K cut charges it to every segment).
#ifndef PA_FP8_PIECE_COST
#define PA_FP8_PIECE_COST 4
#endif
#ifndef PA_BF16_PIECE_COST
#define PA_BF16_PIECE_COST 1
#endif
#ifndef PA_LATENT_PIECE_COST
#define PA_LATENT_PIECE_COST 3
#endif
constexpr int kFp8PieceCost = PA_FP8_PIECE_COST;
constexpr int kBf16PieceCost = PA_BF16_PIECE_COST;
constexpr int kLatentPieceCost = PA_LATENT_PIECE_COST;
#ifndef PA_EXTEND_PIECE_COST
#define PA_EXTEND_PIECE_COST 6
#endif
constexpr int kExtendPieceCost = PA_EXTEND_PIECE_COST;
// Decode with at most this many (virtual) kv heads: one key-tile stream per
// head, and the split-pass blocks of one token range take its heads side by
// side (GQA: a token's rows of all heads are adjacent in the pool, so they
// are fetched together; latent cache: the two virtual heads read the same
// rows, the second from L2).  With more heads (whose rows of a token span
// more memory than benefits from it) one stream holds all (sequence, kv
// head) ranges.
constexpr int kAlignedHeadsMax = 8;
__host__ __device__ inline int split_head_groups(int num_kv_heads) {
    return num_kv_heads <= kAlignedHeadsMax ? num_kv_heads : 1;
}

struct DecodeParams {
    const void* q;            // bf16 [B, Hq, D], row stride q_stride_b
    int64_t q_stride_b;       // elements
    const void* k_pool;       // bf16 | e4m3fn
    const void* v_pool;
    int64_t s_page, s_tok, s_head;   // pool strides in elements
    const int32_t* block_table;
    int64_t bt_stride;
    const int32_t* seq_lens;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;            // G = Hq / Hkv (1..16; latent cache: 1..128)
    int32_t q_len;            // query rows per sequence (1: decode; > 1: verify)
    int32_t rows;             // MFMA columns used: G * q_len <= 16; column c is query
                              // token c / G, head c % G of the kv head
    int64_t q_stride_t, out_stride_t;   // elements between a sequence's query tokens
    int32_t page_shift;       // log2(page_size)
    int32_t window;           // <= 0: off
    int32_t has_cap;
    float qk_scale2;          // scale * k_scale * log2(e)           (no cap)
    float cap_c1;             // 2 * scale * k_scale * log2(e) / c   (cap)
    float cap_c2;             // c * log2(e)                         (cap)
    float v_scale;
    const float* sinks;       // [Hq] sink logits (natural-log units) or null
    const float* alibi;       // [Hq] ALiBi slopes (natural-log units per position) or null
    const float* k_desc;      // per-request cache descales or null; request b
    const float* v_desc;      //   uses entry desc_per_seq ? b : 0
    int32_t desc_per_seq;
    void* out;                // bf16 [B, Hq, D], row stride out_stride_b
    int64_t out_stride_b;
    float* part_o;            // [workers, 2, rows, Dv]: partial of a segment a wave covers in part
    float* part_lse;          // [workers, 2, rows] (log2 domain)
    int32_t* seg_rec;         // [B * Hkv][4]: for a segment with keys, the waves owning its
                              // first and last tile and the first one's slot (written by
                              // the owner of the first tile).  Split pass -> merge.
    int32_t piece_cost;       // tiles' worth of work a piece costs beyond its tiles: the
                              // stream-K cut gives every segment this much extra length
                              // in front of its first tile (0: tiles only)
};

struct GatherParams {
    const void* k_pool;
    const void* v_pool;
    int64_t s_page, s_tok, s_head;
    const int32_t* block_table;
    int64_t bt_stride;
    const int32_t* seq_lens;
    int32_t num_seqs, num_kv_heads, page_shift;
    void* k_out;
    void* v_out;
};

struct ExtendParams {
    const void* q;            // bf16 [total_q, Hq, D]
    const void* k_new;        // bf16 [total_q, Hkv, D]
    const void* v_new;
    const int32_t* cu_seqlens_q;
    const int32_t* ctx_lens;
    const void* k_pool;
    const void* v_pool;
    int64_t s_page, s_tok, s_head;
    const int32_t* block_table;
    int64_t bt_stride;
    int32_t num_seqs, num_q_heads, num_kv_heads, group;
    int32_t page_shift;
    int32_t window;
    int32_t q_tiles;          // row tiles per (sequence, kv head): ceil(max_q_len * G / rows)
    int32_t has_cap;
    float qk_scale2;          // scale * log2(e), for new (bf16) keys
    float qk_scale2_ctx;      // scale * k_scale * log2(e), for cached keys
    float cap_c1, cap_c1_ctx, cap_c2;
    float v_scale;            // applied to the cached-value part of the sum
    const float* sinks;       // [Hq] sink logits (natural-log units) or null
    const float* alibi;       // [Hq] ALiBi slopes or null
    const float* k_desc;      // per-request cache descales or null (as decode)
    const float* v_desc;
    int32_t desc_per_seq;
    void* out;                // bf16 [total_q, Hq, D]
    // persistent-block split of the key tiles (workspace)
    int64_t* pfx;             // [items + 1]: stream units of items 0..i-1
    int32_t* rec;             // [items][4]: blocks covering an item, first block's slot
    float* part_lse;          // [workers][2][rows per block] (log2 domain)
    float* part_o;            // [workers][2][rows per block][D]
    int32_t piece_cost;       // units an item with tiles takes in front of its first tile
};

struct AppendParams {
    const void* key;          // bf16 [num_tokens, Hkv, D], token stride row_stride
    const void* value;
    int64_t row_stride;       // elements
    void* k_pool;             // bf16 | e4m3fn, strides in elements
    void* v_pool;
    int64_t s_page, s_tok, s_head;
    const int64_t* slot_mapping;
    int64_t num_tokens;
    int32_t num_kv_heads, head_dim, page_shift;
    float k_scale, v_scale;   // e4m3fn caches: stored value = enc(x / scale)
};

hipError_t launch_cache_append(const AppendParams& p, bool fp8, hipStream_t stream);
// Split pass: `workers` persistent blocks of waves_per_block (1..4) waves; wave
// i of a block serves query rows 16i..16i+15 of every segment.
hipError_t launch_decode(const DecodeParams& p, int head_dim, bool fp8, bool uniform_pages,
                         int waves_per_block, int workers, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, int num_seqs,
                               int num_kv_heads, hipStream_t stream);
// Resident split-pass blocks per compute unit (occupancy of the kernel variant).
hipError_t decode_blocks_per_cu(int head_dim, bool fp8, bool uniform_pages, int waves_per_block,
                                int* out);
constexpr int kMaxDecodeRows = 64;   // query rows per kv head: 16 per wave, 4 waves
// Latent-cache decode (head_dim_v < head_dim, bf16): the split pass; the
// merge is launch_decode_merge with head_dim_v.  alias: v_pool == k_pool.
hipError_t launch_mla_decode(const DecodeParams& p, int head_dim, int head_dim_v, bool alias,
                             int waves_per_block, int workers, hipStream_t stream);
// rows: query rows per kv head (the variant depends on it).
hipError_t mla_blocks_per_cu(int head_dim, int head_dim_v, bool alias, int waves_per_block,
                             int rows, int* out);
constexpr int kMaxLatentGroup = 128;   // query heads per kv head: 16 per wave, 8 waves
hipError_t launch_gather(const GatherParams& p, int head_dim, bool fp8, hipStream_t stream);
// Extend: a scan of the items' tile counts, `workers` persistent blocks, and a
// merge of the items several blocks cover.
hipError_t launch_extend(const ExtendParams& p, int head_dim, bool fp8, int workers,
                         hipStream_t stream);
// Resident extend blocks per compute unit.
hipError_t extend_blocks_per_cu(int head_dim, bool fp8, int* out);
constexpr int64_t kMaxExtendItems = (int64_t)1 << 24;   // (sequence, kv head, row tile)
// Rows (new token, query head) one extend block covers.
int extend_rows_per_block();
int extend_waves_per_block();

// Passes of a decode call: the split pass, the merge, or both in order.
enum DecodePasses { kDecodeSplitPass = 1, kDecodeMergePass = 2, kDecodeBothPasses = 3 };
// Checks a decode/verify call (mode PA_MODE_DECODE or PA_MODE_VERIFY) with a
// workspace of workspace_bytes bytes and fills *p but for its workspace
// pointers.  *empty: the call is valid and launches nothing.  The workspace
// pointer itself is the caller's to check.
pa_status decode_prepare(int mode, const pa_plan* plan, const void* q, int64_t q_stride_b,
                         const void* k_pool, const void* v_pool, int64_t kv_stride_page,
                         int64_t kv_stride_tok, int64_t kv_stride_head, int64_t num_pages,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                         int32_t page_size, float scale, float softcap, int32_t window,
                         float k_scale, float v_scale, void* out, int64_t out_stride_b,
                         uint64_t workspace_bytes, const pa_extras* extras, DecodeParams* p,
                         bool* empty);
// Lays the plan's workspace out at `workspace` (16-byte aligned, at least
// plan.workspace_bytes) and enqueues the passes.
pa_status decode_launch(int passes, const pa_plan& pl, DecodeParams& p, void* workspace,
                        hipStream_t stream);

}  // namespace pa
