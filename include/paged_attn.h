/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged GQA attention library.
 *
 * The library computes attention of a batch of queries against a paged,
 * block-table-indexed K/V cache with grouped-query heads, in two modes:
 *
 *   decode   one query token per sequence (the token at position L-1, whose
 *            own key/value is already in the cache): split-KV partial
 *            attention with log-sum-exp, then a merge of the splits.  This is
 *            the computation of `decode_attention_fwd` and its kernels
 *            `_fwd_grouped_kernel_stage1` / `_fwd_kernel_stage2` on the page
 *            "vllm/attention/ops/triton_decode_attention.py".
 *   verify   q_len query tokens per sequence (the speculative verify step of
 *            the b12x page: `1 + num_speculative_tokens` rows for every
 *            request, whose keys/values are already in the cache): token i
 *            at position L - q_len + i attends causally to the cached tokens
 *            up to and including itself, through the same split/merge kernels
 *            as decode.
 *   extend   prefix-prefill: new query tokens attend to the sequence's cached
 *            context through the pages (no mask) and causally to each other
 *            (contiguous new K/V rows), as `context_attention_fwd` and
 *            `_fwd_kernel` on the page "vllm/attention/ops/prefix_prefill.py".
 *
 * Problem parameters follow the statement of the problem on those pages and on
 * the vLLM "b12x" backend page (`B12xPagedAttentionImpl.__init__`/`forward`):
 * Q, the K/V page pools, the block table, per-sequence lengths, scale,
 * soft-cap, sliding window, page size and the fp8 k/v descales.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - G = num_q_heads / num_kv_heads; query head h reads key/value head h / G.
 * - K/V pools: element (page, row, kv_head, d) sits at
 *     pool + page*kv_stride_page + row*kv_stride_tok + kv_head*kv_stride_head + d
 *   (strides in elements; d is contiguous).  The dense layout
 *   [num_pages, page_size, num_kv_heads, head_dim] is the `_kv_cache_views`
 *   view of the b12x page; a [num_pages, num_kv_heads, page_size, head_dim]
 *   layout is expressed by its strides.
 * - Token t of sequence b sits in page block_table[b*bt_stride + t/page_size],
 *   row t % page_size.  Only entries t/page_size < ceil(L_b/page_size) are
 *   read; padding may hold anything (e.g. -1).
 * - Sliding window W > 0 keeps key position j for query position p iff
 *   p - j < W (the b12x page stores `window_left = W - 1`; prefix_prefill keeps
 *   `pos_q - pos_k < SLIDING_WINDOW`).  W <= 0 means no window.
 * - Soft-cap c > 0 replaces each scaled score s by c*tanh(s/c) (applied after
 *   the scale, as `logit_cap` in `_fwd_kernel_stage1`); c <= 0 means off.
 * - fp8 caches are OCP e4m3fn; a cached key is dec(K)*k_scale and a cached
 *   value dec(V)*v_scale (per-tensor descales).  For bf16 caches pass 1.0.
 * - Q, new K/V and the output are bf16 (round-to-nearest-even on output).
 * - Every device pointer must be 16-byte aligned; every row stride must keep
 *   16-byte alignment.
 *
 * Ownership and errors
 * --------------------
 * The caller owns every buffer, including the workspace; the library never
 * allocates device memory, never synchronises, and keeps no state between
 * calls (the one exception is paged_attn_decode_noalloc, whose scratch is a
 * fixed array inside the library).  Compute calls enqueue kernels on `hip_stream` (a hipStream_t, NULL =
 * the null stream) and return; buffers must stay valid until the stream
 * reaches that point.  All host-visible arguments are validated before
 * anything is enqueued: on error nothing is launched and the output is
 * untouched.  Contents of device buffers (lengths within the stated bounds,
 * page ids within [0, num_pages), monotone cu_seqlens_q) are the caller's
 * contract and are not checked.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAGED_ATTN_ABI_VERSION 4

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
    PA_ERR_INVALID_SHAPE = 2,      /* inconsistent sizes (b12x: ValueError) */
    PA_ERR_UNSUPPORTED = 3,        /* valid but not built (b12x: NotImplementedError/TypeError) */
    PA_ERR_WORKSPACE_TOO_SMALL = 4,/* workspace below plan->workspace_bytes (b12x: RuntimeError) */
    PA_ERR_MISALIGNED = 5,         /* pointer or stride breaks 16-byte alignment */
    PA_ERR_PLAN_MISMATCH = 6,      /* call arguments disagree with the plan */
    PA_ERR_HIP = 7,                /* a HIP runtime call or launch failed */
    PA_STATUS_MAX_ENUM = 0x7fffffff /* not a status: gives the type every int32 value */
} pa_status;

typedef enum { PA_KV_BF16 = 0, PA_KV_FP8_E4M3 = 1 } pa_kv_dtype;
typedef enum { PA_MODE_DECODE = 0, PA_MODE_EXTEND = 1, PA_MODE_VERIFY = 2 } pa_mode;

/*
 * Optional inputs of a compute call (the `attention_sink_bias`, `k_descale`
 * and `v_descale` that the vLLM "b12x" backend page hands to its kernel's
 * `bind`, and ALiBi slopes).  Pass NULL for none, or leave members NULL.  Device pointers,
 * 4-byte aligned; contents are read by the kernels and not checked.
 *
 *   sinks         fp32 [Hq]: one logit per query head that joins the softmax
 *                 normaliser and carries no value:
 *                   out = sum_j e^{s_j} v_j / (e^{sink[h]} + sum_j e^{s_j}),
 *                 s_j the scaled (and soft-capped) scores; the sink itself is
 *                 neither scaled nor capped.  A row with no key stays zero.
 *   k_descale,    fp32 per-request cache descales (finite, > 0): a cached key
 *   v_descale     of request b is dec(K) * k_scale * k_descale[b'] (values
 *                 alike), b' = b when num_descales > 1, else 0.  New extend
 *                 rows are not cache elements and take no descale.
 *   alibi_slopes  fp32 [Hq]: ALiBi slope a[h] of each query head (the
 *                 `Alibi_slopes` of `_fwd_kernel_alibi` on the prefix_prefill
 *                 page): a key at position j seen from a query at position p
 *                 gets a[h] * (j - p) added to its scaled (and capped) score;
 *                 causal limit, window and sinks apply as without it.
 *   num_descales  entries behind k_descale/v_descale: 1 (shared by every
 *                 request) or >= B; anything else is PA_ERR_INVALID_SHAPE
 *                 (the b12x `_prepare_fp8_descales` expands a single value,
 *                 slices a longer tensor and rejects a shorter one).
 */
typedef struct {
    const float* sinks;
    const float* k_descale;
    const float* v_descale;
    const float* alibi_slopes;
    int32_t num_descales;
    int32_t reserved;
} pa_extras;

/* Host-side description of one call shape (plain values, no pointers). */
typedef struct {
    int32_t mode;              /* pa_mode */
    int32_t num_seqs;          /* B >= 0 */
    int32_t num_q_heads;       /* Hq, a multiple of num_kv_heads */
    int32_t num_kv_heads;      /* Hkv >= 1; G = Hq/Hkv must be 1, 2, 4, 8 or 16
                                  (latent cache: 1 .. 128) */
    int32_t head_dim;          /* D: 64 or 128 (q/k and v alike); latent cache:
                                  576 or 288 (q/k) */
    int32_t page_size;         /* P >= 1 */
    int32_t kv_dtype;          /* pa_kv_dtype */
    int32_t window;            /* sliding window W (<= 0: off) */
    int32_t max_pages_per_seq; /* block-table row width in entries */
    int32_t max_kv_len;        /* bound on cached tokens per sequence
                                  (decode/verify: seq_lens, incl. the query
                                   tokens; extend: ctx_lens) */
    int32_t total_q;           /* extend: rows of q/k_new/v_new/out */
    int32_t max_q_len;         /* extend: bound on new tokens per sequence;
                                  verify: the query tokens per sequence
                                  (q_len >= 1, G * q_len <= 64) */
    int32_t num_splits;        /* decode: 0 = plan chooses; > 0 forces the
                                  number of split-pass pieces (blocks),
                                  rounded up to a multiple of num_kv_heads
                                  when that is at most 8 (a latent cache
                                  with over 64 query heads: of 2) */
    int32_t head_dim_v;        /* value head dim: 0 (or head_dim) = head_dim;
                                  head_dim_v < head_dim selects a latent cache
                                  (decode, bf16, (576, 512) or (288, 256)):
                                  the value of a token is the first
                                  head_dim_v entries of the value pool's row,
                                  read with the key strides; pass v_pool =
                                  k_pool for a latent cache whose value is the
                                  key row's prefix (`_fwd_grouped_kernel_stage1`
                                  with Lk = 576 = 512 + 64, Lv = 512) */
} pa_problem;

/* The plan: a plain value the caller owns (nothing to free).  Planning reads
 * no device data, so it never depends on live lengths (the b12x page plans
 * fixed capacities the same way). */
typedef struct {
    pa_problem prob;
    int32_t num_splits;        /* decode/verify: split-pass pieces = persistent
                                  blocks */
    int32_t tokens_per_split;  /* tile granularity of the pieces: 32 keys
                                  (decode/verify), 64 keys (extend) */
    int32_t waves_per_block;   /* decode/verify: waves per block, one per 16
                                  query rows (token, head) of a kv head
                                  (latent cache: rounded up to 2, 4 or 8);
                                  extend: waves per block, one per 32 rows */
    int32_t num_cus;           /* compute units the plan was made for */
    uint64_t workspace_bytes;  /* device scratch the compute call needs */
    int32_t reserved[8];
} pa_plan;

/*
 * paged_attn_plan -- choose the split-KV decomposition and size the workspace.
 *
 * Decode with Hkv <= 8 kv heads: for each kv head h, the 32-token tiles of
 * its key ranges [lo, L) (lo = max(0, L-W) with a window) over all
 * sequences, laid end to end, are cut into out->num_splits / Hkv contiguous
 * pieces of equal weight, a key range weighing its tiles plus a fixed number
 * of tiles' worth (what starting a piece costs a block: 1 at bf16, 4 at fp8,
 * 3 for a latent cache); block h * (num_splits / Hkv) + j of the split pass
 * takes piece j of head h, so the blocks reading the kv heads of one token range
 * run side by side (a token's heads are adjacent in the pool).  A latent
 * cache with more than 64 query heads runs as two virtual kv heads over the
 * same rows, laid out the same way (the two blocks of a token range read the
 * same rows together).  With more kv heads all (sequence, head) ranges laid
 * end to end are cut into num_splits pieces.  The plan takes as many blocks
 * as the device keeps resident (compute units x resident blocks per unit,
 * rounded down to a multiple of the heads laid out so), or prob->num_splits
 * (rounded up to one) when that is > 0.
 * A block has one wave per 16 query rows of a kv head (G for decode,
 * G * q_len for verify); its waves walk the same tiles.  Latent cache: the
 * count is rounded up to 2, 4 or 8; with at most 16 query heads over one pool
 * the second wave stages the tiles for the first.  The resident count per
 * unit is the runtime's occupancy for the kernel variant (one fewer of eight
 * for fp8 caches, which stream faster so).
 * Pieces of one key range are merged by log-sum-exp (the split partition
 * and merge of `_fwd_kernel_stage1/2`; any partition gives the same result).
 * Verify: as decode, with lo = max(0, L - q_len + 1 - W), the window start of
 * the first query token.
 * Extend: the key tiles (64 keys) of every item -- a sequence, a kv head and
 * one block's worth of its new (token, query head) rows -- laid end to end,
 * are cut into out->num_splits contiguous pieces of equal weight (an item
 * weighing its tiles plus 6), one per persistent block (as many as the
 * device keeps resident, or prob->num_splits when > 0).  The workspace holds
 * the items' weight prefix sums, the blocks covering each item, and two
 * partial slots per block.
 *
 * hip_device >= 0 queries that device's compute-unit count; hip_device < 0
 * plans for an MI355X (256 compute units) without touching any device.
 * Host only: no allocation, no launch.
 */
pa_status paged_attn_plan(const pa_problem* prob, int hip_device, pa_plan* out);

/*
 * paged_attn_decode -- one query token per sequence.
 *
 *   q             bf16 [B, Hq, D], sequence stride q_stride_b (elements),
 *                 heads contiguous (latent cache: D = head_dim, the value
 *                 rows and out have Dv = head_dim_v entries)
 *   k_pool,v_pool bf16 or e4m3fn pools (layout above), num_pages pages
 *   block_table   int32 [B, >= ceil(L_b/P)] with row stride bt_stride
 *   seq_lens      int32 [B]: L_b cached tokens including the query token
 *                 (0 <= L_b <= prob.max_kv_len); L_b = 0 gives a zero row
 *   page_size, window   must equal the plan's
 *   scale         multiplies q.k (e.g. 1/sqrt(D))
 *   softcap       c > 0 enables c*tanh(s/c)
 *   k_scale,v_scale  fp8 descales (1.0 for bf16)
 *   out           bf16 [B, Hq, D], sequence stride out_stride_b
 *   workspace     >= plan->workspace_bytes of device memory (split partials
 *                 and each sequence's tile offset, written by the split pass
 *                 and read by the merge; no initial contents needed);
 *                 calls that share a workspace must not overlap
 *   extras        optional sinks and per-request descales (see pa_extras),
 *                 or NULL
 *
 * Two kernels run: the key ranges of all (sequence, kv head) pairs, laid end
 * to end, are cut into plan->num_splits pieces of equal weight (see
 * paged_attn_plan), one per persistent block of the split pass; a second
 * kernel merges by log-sum-exp every pair that spans several pieces (the
 * split/merge of `_fwd_grouped_kernel_stage1` / `_fwd_kernel_stage2`).
 */
pa_status paged_attn_decode(const pa_plan* plan,
                            const void* q, int64_t q_stride_b,
                            const void* k_pool, const void* v_pool,
                            int64_t kv_stride_page, int64_t kv_stride_tok,
                            int64_t kv_stride_head, int64_t num_pages,
                            const int32_t* block_table, int64_t bt_stride,
                            const int32_t* seq_lens,
                            int32_t page_size, float scale, float softcap,
                            int32_t window, float k_scale, float v_scale,
                            void* out, int64_t out_stride_b,
                            void* workspace, uint64_t workspace_bytes,
                            const pa_extras* extras,
                            void* hip_stream);

/*
 * Latent cache (prob.head_dim_v < prob.head_dim): the same call with
 * q [B, Hq, D] and out [B, Hq, Dv]; v_pool's rows are read at the key rows'
 * places with the key strides and their first Dv entries are the values.
 * When v_pool == k_pool each row is read once (the values come from the key
 * rows already loaded).  bf16 caches only; G up to 128.
 */

/*
 * paged_attn_decode_split, paged_attn_decode_merge -- the two kernels of
 * paged_attn_decode enqueued one call at a time, with the same arguments and
 * checks.  split followed by merge on one stream, with one workspace and
 * nothing writing that workspace in between, is paged_attn_decode (bit for
 * bit).  For callers that time or schedule the two passes separately.
 */
pa_status paged_attn_decode_split(const pa_plan* plan,
                                  const void* q, int64_t q_stride_b,
                                  const void* k_pool, const void* v_pool,
                                  int64_t kv_stride_page, int64_t kv_stride_tok,
                                  int64_t kv_stride_head, int64_t num_pages,
                                  const int32_t* block_table, int64_t bt_stride,
                                  const int32_t* seq_lens,
                                  int32_t page_size, float scale, float softcap,
                                  int32_t window, float k_scale, float v_scale,
                                  void* out, int64_t out_stride_b,
                                  void* workspace, uint64_t workspace_bytes,
                                  const pa_extras* extras,
                                  void* hip_stream);
pa_status paged_attn_decode_merge(const pa_plan* plan,
                                  const void* q, int64_t q_stride_b,
                                  const void* k_pool, const void* v_pool,
                                  int64_t kv_stride_page, int64_t kv_stride_tok,
                                  int64_t kv_stride_head, int64_t num_pages,
                                  const int32_t* block_table, int64_t bt_stride,
                                  const int32_t* seq_lens,
                                  int32_t page_size, float scale, float softcap,
                                  int32_t window, float k_scale, float v_scale,
                                  void* out, int64_t out_stride_b,
                                  void* workspace, uint64_t workspace_bytes,
                                  const pa_extras* extras,
                                  void* hip_stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc): the same arguments and kernels, without
 * the workspace.  The scratch is a fixed array of
 * PAGED_ATTN_NOALLOC_SCRATCH_BYTES inside this library, one copy per GPU,
 * held from the library's first use on that GPU until the process ends.
 *
 * - A plan whose workspace_bytes exceeds PAGED_ATTN_NOALLOC_SCRATCH_BYTES is
 *   rejected with PA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued
 *   (a decode plan needs about 4 to 14 MiB for 64 to 256 sequences of
 *   Llama-3-8B-like heads; a latent cache with 16 heads per kv head at 512
 *   splits needs 32 MiB).
 * - The call allocates nothing: no hipMalloc, no hipFree.  Its first call on
 *   a device looks up that device's copy of the array (hipGetSymbolAddress)
 *   and keeps the address; the kernels run on hip_stream's device.
 * - Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (other streams, or other threads) race and give wrong results.  Calls
 *   in order on one stream are safe.  Nothing in the array needs initial
 *   contents (the split pass writes what the merge reads).
 * - Decode mode only (plans made with PA_MODE_DECODE, latent caches
 *   included); errors otherwise as paged_attn_decode.
 */
#define PAGED_ATTN_NOALLOC_SCRATCH_BYTES (48ull << 20)
pa_status paged_attn_decode_noalloc(const pa_plan* plan,
                                    const void* q, int64_t q_stride_b,
                                    const void* k_pool, const void* v_pool,
                                    int64_t kv_stride_page, int64_t kv_stride_tok,
                                    int64_t kv_stride_head, int64_t num_pages,
                                    const int32_t* block_table, int64_t bt_stride,
                                    const int32_t* seq_lens,
                                    int32_t page_size, float scale, float softcap,
                                    int32_t window, float k_scale, float v_scale,
                                    void* out, int64_t out_stride_b,
                                    const pa_extras* extras,
                                    void* hip_stream);

/*
 * paged_attn_verify -- q_len query tokens per sequence against the cache
 * (speculative verification; q_len = plan->prob.max_q_len, the plan made
 * with mode PA_MODE_VERIFY).  The arguments are paged_attn_decode's, except:
 *
 *   q             bf16 [B, q_len, Hq, D]: token i of sequence b at
 *                 q + b*q_stride_b + i*Hq*D (q_stride_b >= q_len*Hq*D)
 *   seq_lens      L_b cached tokens including all q_len query tokens; token i
 *                 sits at position L_b - q_len + i and attends to the keys
 *                 j <= L_b - q_len + i (and, with a window, j > that - W);
 *                 a token with no such key (L_b - q_len + i < 0) gets a zero row
 *   out           bf16 [B, q_len, Hq, D], sequence stride out_stride_b
 *                 (>= q_len*Hq*D)
 *
 * The G*q_len (token, head) rows of a kv head are served by one block (a
 * wave per 16 rows) walking each K/V tile once from HBM: one pass over the
 * cache serves all q_len tokens.  Same kernels, workspace rules and errors as
 * paged_attn_decode.
 */
pa_status paged_attn_verify(const pa_plan* plan,
                            const void* q, int64_t q_stride_b,
                            const void* k_pool, const void* v_pool,
                            int64_t kv_stride_page, int64_t kv_stride_tok,
                            int64_t kv_stride_head, int64_t num_pages,
                            const int32_t* block_table, int64_t bt_stride,
                            const int32_t* seq_lens,
                            int32_t page_size, float scale, float softcap,
                            int32_t window, float k_scale, float v_scale,
                            void* out, int64_t out_stride_b,
                            void* workspace, uint64_t workspace_bytes,
                            const pa_extras* extras,
                            void* hip_stream);

/*
 * paged_attn_extend -- prefix-prefill of new tokens on top of a paged context.
 *
 *   q             bf16 [total_q, Hq, D] (rows of all sequences, concatenated)
 *   k_new,v_new   bf16 [total_q, Hkv, D]: keys/values of the new tokens
 *   cu_seqlens_q  int32 [B+1]: sequence b owns rows [cu[b], cu[b+1]),
 *                 cu[0] = 0, cu[B] = total_q, cu[b+1]-cu[b] <= max_q_len
 *   ctx_lens      int32 [B]: C_b cached tokens (<= prob.max_kv_len); new row
 *                 i of sequence b sits at position C_b + i
 *   k_pool...bt_stride  the cached context, as for decode
 *   out           bf16 [total_q, Hq, D]
 *   workspace     >= plan->workspace_bytes of device memory, 16-byte
 *                 aligned (required: extend always has one); no initial
 *                 contents needed; calls that share a workspace must not
 *                 overlap
 *   extras        optional sinks and per-request descales (see pa_extras),
 *                 or NULL; descales apply to the cached context only
 *
 * Three kernels run on hip_stream: a scan of the items' key-tile counts, the
 * persistent blocks (each walks its piece of the tiles with online softmax,
 * writing items it covers whole to out and the ends of the others to the
 * workspace), and a merge by log-sum-exp of the items several blocks share.
 */
pa_status paged_attn_extend(const pa_plan* plan,
                            const void* q, const void* k_new, const void* v_new,
                            const int32_t* cu_seqlens_q, const int32_t* ctx_lens,
                            const void* k_pool, const void* v_pool,
                            int64_t kv_stride_page, int64_t kv_stride_tok,
                            int64_t kv_stride_head, int64_t num_pages,
                            const int32_t* block_table, int64_t bt_stride,
                            int32_t page_size, float scale, float softcap,
                            int32_t window, float k_scale, float v_scale,
                            void* out, void* workspace, uint64_t workspace_bytes,
                            const pa_extras* extras,
                            void* hip_stream);

/*
 * paged_attn_cache_append -- write new tokens' keys and values into the
 * paged caches (the `do_kv_cache_update` step on the vLLM "b12x" backend
 * page, which passes key, value, the caches, `slot_mapping` and the k/v
 * scales to `reshape_and_cache_flash`).
 *
 *   key, value    bf16 [num_tokens, num_kv_heads, head_dim], heads contiguous,
 *                 token stride kv_row_stride (elements)
 *   k_pool,v_pool the caches, layout and strides as for decode
 *   slot_mapping  int64 [num_tokens]: token i goes to page s / page_size, row
 *                 s % page_size (s = slot_mapping[i]) for every kv head;
 *                 s < 0 skips the token (padding).  0 <= s < num_pages *
 *                 page_size and distinct slots are the caller's contract.
 *   kv_dtype      PA_KV_BF16: the rows are copied unchanged.
 *                 PA_KV_FP8_E4M3: each element x is stored as e4m3fn(x / scale)
 *                 (k_scale for keys, v_scale for values; IEEE fp32 division,
 *                 round to nearest even, saturating at +-448, NaN kept);
 *                 scales must be finite and > 0.
 *
 * One kernel on hip_stream; no workspace.  head_dim 64 or 128, page_size a
 * power of two up to 4096, 16-byte aligned pointers and strides.
 */
pa_status paged_attn_cache_append(const void* key, const void* value, int64_t num_tokens,
                                  int64_t kv_row_stride, int32_t num_kv_heads,
                                  int32_t head_dim, void* k_pool, void* v_pool,
                                  int64_t kv_stride_page, int64_t kv_stride_tok,
                                  int64_t kv_stride_head, int64_t num_pages, int32_t page_size,
                                  int32_t kv_dtype, const int64_t* slot_mapping, float k_scale,
                                  float v_scale, void* hip_stream);

/*
 * paged_attn_gather -- test aid: copy every cached key/value row
 * (t in [0, L_b)) of every sequence, through the same address path the
 * attention kernels use, into k_out/v_out [sum_b L_b, Hkv, D] (sequence-major,
 * same element type as the pools).  A byte-exact check of the block-table
 * gather.  Uses the plan's problem (decode mode) for shapes.
 */
pa_status paged_attn_gather(const pa_plan* plan,
                            const void* k_pool, const void* v_pool,
                            int64_t kv_stride_page, int64_t kv_stride_tok,
                            int64_t kv_stride_head, int64_t num_pages,
                            const int32_t* block_table, int64_t bt_stride,
                            const int32_t* seq_lens,
                            void* k_out, void* v_out, void* hip_stream);

/*
 * paged_attn_check_inputs -- host-side check of the device-content contract
 * of a compute call, on host copies of its metadata (the b12x page's
 * `forward` validates its metadata on the host the same way).  For callers
 * and tests that want a wrong length, page id or offset reported instead of
 * read out of bounds on the GPU.  Host only: reads host memory, no HIP call.
 *
 *   plan          the plan of the call
 *   lens          int32 [B]: seq_lens (decode/verify) or ctx_lens (extend);
 *                 each must lie in [0, prob.max_kv_len]
 *   block_table   int32 [B, >= ceil(L_b/P)] with row stride bt_stride: every
 *                 entry t/P < ceil(L_b/P) must lie in [0, num_pages)
 *   cu_seqlens_q  extend: int32 [B+1] with cu[0] = 0, 0 <= cu[b+1] - cu[b] <=
 *                 prob.max_q_len, cu[B] = prob.total_q; NULL otherwise
 *   bad_array,    on PA_ERR_INVALID_SHAPE (either may be NULL): which array
 *   bad_index     broke the contract (1 lens, 2 block_table, 3 cu_seqlens_q)
 *                 and the element's index in it (block_table: b*bt_stride +
 *                 entry)
 *
 * Returns PA_OK, PA_ERR_INVALID_SHAPE for a broken contract, or the status
 * paged_attn_plan would give the plan's problem / PA_ERR_NULL_POINTER /
 * PA_ERR_INVALID_SHAPE (bt_stride below max_pages_per_seq, num_pages < 1).
 */
pa_status paged_attn_check_inputs(const pa_plan* plan, const int32_t* lens,
                                  const int32_t* block_table, int64_t bt_stride,
                                  int64_t num_pages, const int32_t* cu_seqlens_q,
                                  int32_t* bad_array, int64_t* bad_index);

/* Human-readable name of a status code (static storage). */
const char* paged_attn_status_str(pa_status status);

/* Writes a one-line summary of the plan into buf (always NUL-terminated);
 * returns the length it wanted. */
int paged_attn_plan_describe(const pa_plan* plan, char* buf, int buf_len);

/* PAGED_ATTN_ABI_VERSION of the built library. */
int paged_attn_abi_version(void);

/* Path of the HIP runtime library this library resolved its symbols from
 * (lets a host process check it shares one runtime with its allocator). */
const char* paged_attn_hip_runtime_path(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
