// api.cpp -- the C ABI: planning, argument validation, kernel launches.
//
// Validation mirrors the error conventions of the vLLM "b12x" backend page
// (`B12xPagedAttentionImpl.__init__` / `forward`): shape inconsistencies
// (its ValueError) -> PA_ERR_INVALID_SHAPE, unsupported features or dtypes
// (NotImplementedError / TypeError) -> PA_ERR_UNSUPPORTED, scratch too small
// (RuntimeError) -> PA_ERR_WORKSPACE_TOO_SMALL.  Everything is checked before
// anything is enqueued.
#include <dlfcn.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "paged_attn.h"
#include "pa_internal.h"

namespace {

using namespace pa;

constexpr int kDefaultCus = 256;        // MI355X
constexpr int kDefaultExtendBlocksPerCu = 2;   // extend occupancy when no device is queried

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t m) { return cdiv(a, m) * m; }
bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// A latent cache: values narrower than keys (the value is the first
// head_dim_v entries of the row).
bool is_latent(const pa_problem& pr) {
    return pr.head_dim_v != 0 && pr.head_dim_v != pr.head_dim;
}

// Entries of a value (and output) row.
int value_dim(const pa_problem& pr) { return is_latent(pr) ? pr.head_dim_v : pr.head_dim; }

// A latent cache with one kv head and more than 64 query heads is run as two
// virtual kv heads of half the heads each, over the same rows (head stride
// 0): blocks of four waves, which keep their registers, instead of eight,
// which are held to 256 VGPRs and spill.  Query head h stays head h: virtual
// kv head v serves heads [v*G/2, (v+1)*G/2).
int latent_head_split(const pa_problem& pr) {
    if (!is_latent(pr) || pr.num_kv_heads != 1) return 1;
    return (pr.num_q_heads > 64 && pr.num_q_heads % 2 == 0) ? 2 : 1;
}

pa_status check_problem(const pa_problem& pr) {
    if (pr.mode != PA_MODE_DECODE && pr.mode != PA_MODE_EXTEND && pr.mode != PA_MODE_VERIFY)
        return PA_ERR_UNSUPPORTED;
    if (pr.num_seqs < 0 || pr.num_q_heads <= 0 || pr.num_kv_heads <= 0 || pr.page_size <= 0 ||
        pr.max_kv_len < 0 || pr.max_pages_per_seq < 0 || pr.num_splits < 0 ||
        pr.head_dim_v < 0)
        return PA_ERR_INVALID_SHAPE;
    if (pr.num_q_heads % pr.num_kv_heads != 0) return PA_ERR_INVALID_SHAPE;
    // one merge block per (sequence, query head): the grid is 31-bit
    if ((int64_t)pr.num_seqs * pr.num_q_heads >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
    const int G = pr.num_q_heads / pr.num_kv_heads;
    if (is_latent(pr)) {
        // decode over a bf16 latent cache, (576, 512) or (288, 256), G <= 128
        if (pr.mode != PA_MODE_DECODE || pr.kv_dtype != PA_KV_BF16) return PA_ERR_UNSUPPORTED;
        if (!((pr.head_dim == 576 && pr.head_dim_v == 512) ||
              (pr.head_dim == 288 && pr.head_dim_v == 256)))
            return PA_ERR_UNSUPPORTED;
        if (G > kMaxLatentGroup) return PA_ERR_UNSUPPORTED;
    } else {
        if (G > 16 || !is_pow2(G)) return PA_ERR_UNSUPPORTED;
        if (pr.head_dim != 64 && pr.head_dim != 128) return PA_ERR_UNSUPPORTED;
    }
    if (pr.kv_dtype != PA_KV_BF16 && pr.kv_dtype != PA_KV_FP8_E4M3) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(pr.page_size) || pr.page_size > 4096) return PA_ERR_UNSUPPORTED;
    if ((int64_t)pr.max_pages_per_seq < cdiv(pr.max_kv_len, pr.page_size))
        return PA_ERR_INVALID_SHAPE;
    if (pr.mode == PA_MODE_VERIFY) {
        // max_q_len query rows per sequence: G * q_len MFMA columns, 16 per wave
        if (pr.max_q_len < 1) return PA_ERR_INVALID_SHAPE;
        if ((int64_t)G * pr.max_q_len > kMaxDecodeRows) return PA_ERR_UNSUPPORTED;
    }
    if (pr.mode == PA_MODE_EXTEND) {
        if (pr.total_q < 0 || pr.max_q_len < 0) return PA_ERR_INVALID_SHAPE;
        if (pr.num_seqs > 0 && pr.total_q > 0 && pr.max_q_len == 0) return PA_ERR_INVALID_SHAPE;
        // key positions are 32-bit; items are (sequence, kv head, row tile)
        if ((int64_t)pr.max_kv_len + pr.max_q_len >= ((int64_t)1 << 30)) return PA_ERR_UNSUPPORTED;
        const int64_t tiles = cdiv((int64_t)pr.max_q_len * (pr.num_q_heads / pr.num_kv_heads),
                                   extend_rows_per_block());
        if (tiles * pr.num_seqs * pr.num_kv_heads > kMaxExtendItems) return PA_ERR_UNSUPPORTED;
    }
    return PA_OK;
}

// Extend workspace: the items' tile prefix, their block records, and two
// partial slots (log2-sum-exp, rows) per persistent block.
struct ExtLayout {
    int64_t items, rec, lse, o, total;
};

ExtLayout extend_layout(const pa_problem& pr, int64_t workers) {
    ExtLayout L;
    const int64_t rows = extend_rows_per_block();
    L.items = cdiv((int64_t)pr.max_q_len * (pr.num_q_heads / pr.num_kv_heads), rows) *
              pr.num_seqs * pr.num_kv_heads;
    L.rec = round_up((L.items + 1) * 8, 256);
    L.lse = L.rec + round_up(L.items * 16, 256);
    L.o = L.lse + round_up(workers * 2 * rows * 4, 256);
    L.total = L.o + round_up(workers * 2 * rows * pr.head_dim * 4, 256);
    return L;
}

// Split-pass waves per block: one per 16 query rows of a kv head (latent
// cache: rounded up to 2, 4 or 8; with at most 16 rows the second wave stages
// the tiles for the first).
int decode_waves_per_block(const pa_problem& pr) {
    const int q_len = pr.mode == PA_MODE_VERIFY ? pr.max_q_len : 1;
    const int g = pr.num_q_heads / pr.num_kv_heads / latent_head_split(pr);
    const int nw = (g * q_len + 15) / 16;
    if (is_latent(pr)) {
        int p2 = 2;
        while (p2 < nw) p2 *= 2;
        return p2;
    }
    return nw;
}

int elem_bytes(int kv_dtype) { return kv_dtype == PA_KV_FP8_E4M3 ? 1 : 2; }

// Decode/verify workspace: two partial slots (rows of Dv floats and their
// log-sum-exp) per persistent block, and one record per segment.
struct DecLayout {
    int64_t lse, rec, total;
};

DecLayout decode_layout(const pa_problem& pr, int64_t workers) {
    DecLayout L;
    const int64_t q_len = pr.mode == PA_MODE_VERIFY ? pr.max_q_len : 1;
    const int split = latent_head_split(pr);
    const int64_t rows = workers * 2 * (pr.num_q_heads / pr.num_kv_heads / split) * q_len;
    L.lse = round_up(rows * value_dim(pr) * 4, 256);
    L.rec = L.lse + round_up(rows * 4, 256);
    L.total = L.rec + round_up(16 * (int64_t)pr.num_seqs * pr.num_kv_heads * split, 256);
    return L;
}

// Optional sinks and per-request descales (NULL extras: none).
struct Extras {
    const float* sinks = nullptr;
    const float* alibi = nullptr;
    const float* k_desc = nullptr;
    const float* v_desc = nullptr;
    int32_t per_seq = 0;
};

pa_status read_extras(const pa_extras* ex, int32_t num_seqs, Extras* out) {
    *out = Extras{};
    if (!ex) return PA_OK;
    const auto aligned4 = [](const void* ptr) {
        return (reinterpret_cast<uintptr_t>(ptr) & 3u) == 0;
    };
    if (!aligned4(ex->sinks) || !aligned4(ex->k_descale) || !aligned4(ex->v_descale) ||
        !aligned4(ex->alibi_slopes))
        return PA_ERR_MISALIGNED;
    if (ex->k_descale || ex->v_descale) {
        // one value for every request, or one per request (b12x
        // `_prepare_fp8_descales`: a single value is expanded, a longer
        // tensor is sliced, anything shorter is rejected)
        if (ex->num_descales < 1) return PA_ERR_INVALID_SHAPE;
        if (ex->num_descales > 1 && ex->num_descales < num_seqs) return PA_ERR_INVALID_SHAPE;
        out->per_seq = ex->num_descales > 1;
    }
    out->sinks = ex->sinks;
    out->alibi = ex->alibi_slopes;
    out->k_desc = ex->k_descale;
    out->v_desc = ex->v_descale;
    return PA_OK;
}

pa_status check_pools(const pa_plan& pl, const void* k_pool, const void* v_pool,
                      int64_t s_page, int64_t s_tok, int64_t s_head, int64_t num_pages,
                      const int32_t* block_table, int64_t bt_stride) {
    const pa_problem& pr = pl.prob;
    if (!k_pool || !v_pool || !block_table) return PA_ERR_NULL_POINTER;
    if (s_page < 0 || s_tok < 0 || s_head < 0 || num_pages < 1) return PA_ERR_INVALID_SHAPE;
    if (bt_stride < pr.max_pages_per_seq) return PA_ERR_INVALID_SHAPE;
    const int64_t eb = elem_bytes(pr.kv_dtype);
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_MISALIGNED;
    if ((s_page * eb) % 16 || (s_tok * eb) % 16 || (s_head * eb) % 16) return PA_ERR_MISALIGNED;
    // byte offsets inside one page are 32-bit in the kernels
    const int64_t in_page = ((int64_t)(pr.page_size - 1) * s_tok +
                             (int64_t)(pr.num_kv_heads - 1) * s_head + pr.head_dim) * eb;
    if (in_page >= ((int64_t)1 << 31)) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

}  // namespace

extern "C" {

const char* paged_attn_status_str(pa_status s) {
    switch (s) {
        case PA_OK: return "ok";
        case PA_ERR_NULL_POINTER: return "null pointer";
        case PA_ERR_INVALID_SHAPE: return "invalid shape";
        case PA_ERR_UNSUPPORTED: return "unsupported";
        case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case PA_ERR_MISALIGNED: return "misaligned pointer or stride";
        case PA_ERR_PLAN_MISMATCH: return "arguments do not match the plan";
        case PA_ERR_HIP: return "HIP runtime error";
        case PA_STATUS_MAX_ENUM: break;
    }
    return "unknown status";
}

int paged_attn_abi_version(void) { return PAGED_ATTN_ABI_VERSION; }

const char* paged_attn_hip_runtime_path(void) {
    static char path[4096];
    Dl_info info;
    void* sym = reinterpret_cast<void*>(&hipGetDeviceCount);
    if (dladdr(sym, &info) && info.dli_fname) {
        snprintf(path, sizeof path, "%s", info.dli_fname);
        return path;
    }
    return "";
}

pa_status paged_attn_plan(const pa_problem* prob, int hip_device, pa_plan* out) {
    if (!prob || !out) return PA_ERR_NULL_POINTER;
    const pa_problem pr = *prob;
    pa_status st = check_problem(pr);
    if (st != PA_OK) return st;

    int cus = kDefaultCus;
    if (hip_device >= 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, hip_device) != hipSuccess) return PA_ERR_HIP;
        cus = prop.multiProcessorCount;
    }

    pa_plan pl;
    memset(&pl, 0, sizeof pl);
    pl.prob = pr;
    pl.num_cus = cus;
    pl.waves_per_block = 1;
    pl.num_splits = 1;
    pl.tokens_per_split = kTile;

    if (pr.mode == PA_MODE_DECODE || pr.mode == PA_MODE_VERIFY) {
        // Split pass: persistent blocks, each owning an equal contiguous range
        // of the tiles of all segments, one wave per 16 query rows of a
        // segment.  By default as many blocks as the device keeps resident;
        // prob.num_splits > 0 forces the count.
        const int nw = decode_waves_per_block(pr);
        int64_t workers;
        if (pr.num_splits > 0) {
            workers = pr.num_splits;
        } else {
            // latent cache: two blocks of at most two waves share a compute
            // unit's LDS (the plan assumes v_pool == k_pool)
            int per_cu = is_latent(pr) ? (nw <= 2 ? 2 : 1)
                                       : 4 * split_waves_per_simd(pr.head_dim,
                                                                  pr.kv_dtype == PA_KV_FP8_E4M3,
                                                                  nw) / nw;
            if (hip_device >= 0) {
                int cur = -1;
                if (hipGetDevice(&cur) != hipSuccess) return PA_ERR_HIP;
                if (cur != hip_device && hipSetDevice(hip_device) != hipSuccess) return PA_ERR_HIP;
                const hipError_t e =
                    is_latent(pr)
                        ? mla_blocks_per_cu(pr.head_dim, pr.head_dim_v, true, nw,
                                            pr.num_q_heads / pr.num_kv_heads /
                                                latent_head_split(pr),
                                            &per_cu)
                        : decode_blocks_per_cu(pr.head_dim, pr.kv_dtype == PA_KV_FP8_E4M3,
                                               pr.page_size >= 16, nw, &per_cu);
                if (cur != hip_device) (void)hipSetDevice(cur);
                if (e != hipSuccess || per_cu < 1) return PA_ERR_HIP;
            }
            // fp8 K/V, one-wave blocks: seven of the eight resident waves per
            // compute unit stream faster than all eight (measured on MI355X:
            // 165 against 174 us at 256 sequences, G 8, window 4096)
            if (!is_latent(pr) && pr.kv_dtype == PA_KV_FP8_E4M3 && nw == 1 && per_cu == 8)
                per_cu = 7;
            workers = (int64_t)cus * per_cu;
        }
        {
            // a multiple of the per-head streams: block h*W/HG + j takes head
            // h over range j of that head's tiles (a forced count is rounded
            // up, the device count down)
            const int64_t H = split_head_groups(pr.num_kv_heads * latent_head_split(pr));
            workers = pr.num_splits > 0 ? (workers + H - 1) / H * H
                                        : std::max<int64_t>(H, workers / H * H);
        }
        if (workers > kMaxWorkers) return PA_ERR_UNSUPPORTED;
        pl.num_splits = (int32_t)workers;
        pl.tokens_per_split = kTile;
        pl.waves_per_block = nw;
        pl.workspace_bytes = (uint64_t)decode_layout(pr, workers).total;
    }
    if (pr.mode == PA_MODE_EXTEND) {
        // Persistent blocks, each owning an equal contiguous range of the key
        // tiles of all (sequence, kv head, row tile) items; as many as the
        // device keeps resident, or prob.num_splits when > 0.
        int64_t workers;
        if (pr.num_splits > 0) {
            workers = pr.num_splits;
        } else {
            int per_cu = kDefaultExtendBlocksPerCu;
            if (hip_device >= 0) {
                int cur = -1;
                if (hipGetDevice(&cur) != hipSuccess) return PA_ERR_HIP;
                if (cur != hip_device && hipSetDevice(hip_device) != hipSuccess) return PA_ERR_HIP;
                const hipError_t e =
                    extend_blocks_per_cu(pr.head_dim, pr.kv_dtype == PA_KV_FP8_E4M3, &per_cu);
                if (cur != hip_device) (void)hipSetDevice(cur);
                if (e != hipSuccess || per_cu < 1) return PA_ERR_HIP;
            }
            workers = (int64_t)cus * per_cu;
        }
        if (workers > kMaxWorkers) return PA_ERR_UNSUPPORTED;
        pl.num_splits = (int32_t)workers;
        pl.tokens_per_split = 64;
        pl.waves_per_block = extend_waves_per_block();
        pl.workspace_bytes = (uint64_t)extend_layout(pr, workers).total;
    }
    *out = pl;
    return PA_OK;
}

int paged_attn_plan_describe(const pa_plan* pl, char* buf, int buf_len) {
    char tmp[512];
    int n;
    if (!pl) {
        n = snprintf(tmp, sizeof tmp, "(null plan)");
    } else {
        const pa_problem& p = pl->prob;
        n = snprintf(tmp, sizeof tmp,
                     "%s B=%d Hq=%d Hkv=%d D=%d Dv=%d P=%d kv=%s window=%d max_kv_len=%d "
                     "splits=%d tokens_per_split=%d waves=%d cus=%d workspace=%llu",
                     p.mode == PA_MODE_DECODE ? "decode"
                     : p.mode == PA_MODE_VERIFY ? "verify" : "extend", p.num_seqs,
                     p.num_q_heads, p.num_kv_heads, p.head_dim, value_dim(p), p.page_size,
                     p.kv_dtype == PA_KV_FP8_E4M3 ? "fp8_e4m3" : "bf16", p.window,
                     p.max_kv_len, pl->num_splits, pl->tokens_per_split,
                     pl->waves_per_block, pl->num_cus,
                     (unsigned long long)pl->workspace_bytes);
    }
    if (buf && buf_len > 0) snprintf(buf, (size_t)buf_len, "%s", tmp);
    return n;
}

}  // extern "C"

namespace pa {

pa_status decode_prepare(int mode, const pa_plan* plan, const void* q, int64_t q_stride_b,
                         const void* k_pool, const void* v_pool, int64_t kv_stride_page,
                         int64_t kv_stride_tok, int64_t kv_stride_head, int64_t num_pages,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                         int32_t page_size, float scale, float softcap, int32_t window,
                         float k_scale, float v_scale, void* out, int64_t out_stride_b,
                         uint64_t workspace_bytes, const pa_extras* extras, DecodeParams* pp,
                         bool* empty) {
    *empty = false;
    if (!plan) return PA_ERR_NULL_POINTER;
    const pa_plan& pl = *plan;
    const pa_problem& pr = pl.prob;
    pa_status st = check_problem(pr);
    if (st != PA_OK) return st;
    if (pr.mode != mode) return PA_ERR_PLAN_MISMATCH;
    if (page_size != pr.page_size || window != pr.window) return PA_ERR_PLAN_MISMATCH;
    // the workspace layout follows from (num_splits, problem): a plan edited
    // after paged_attn_plan must not make the kernels write past it
    if (pl.tokens_per_split != kTile || pl.num_splits < 1 || pl.num_splits > kMaxWorkers ||
        pl.num_splits % split_head_groups(pr.num_kv_heads * latent_head_split(pr)) != 0 ||
        pl.waves_per_block != decode_waves_per_block(pr) ||
        pl.workspace_bytes != (uint64_t)decode_layout(pr, pl.num_splits).total)
        return PA_ERR_PLAN_MISMATCH;
    if (pr.num_seqs == 0) {
        *empty = true;
        return PA_OK;
    }
    if (!q || !seq_lens || !out) return PA_ERR_NULL_POINTER;
    st = check_pools(pl, k_pool, v_pool, kv_stride_page, kv_stride_tok, kv_stride_head,
                     num_pages, block_table, bt_stride);
    if (st != PA_OK) return st;
    // verify: q_len query rows per sequence, each Hq*D contiguous (out rows
    // Hq*Dv)
    const int32_t q_len = mode == PA_MODE_VERIFY ? pr.max_q_len : 1;
    const int64_t row = (int64_t)pr.num_q_heads * pr.head_dim;
    const int64_t orow = (int64_t)pr.num_q_heads * value_dim(pr);
    if (q_stride_b < q_len * row || out_stride_b < q_len * orow) return PA_ERR_INVALID_SHAPE;
    if (!aligned16(q) || !aligned16(out) || (q_stride_b * 2) % 16 || (out_stride_b * 2) % 16)
        return PA_ERR_MISALIGNED;
    if (!isfinite(scale) || !isfinite(softcap) || !isfinite(k_scale) || !isfinite(v_scale))
        return PA_ERR_INVALID_SHAPE;
    Extras ex;
    st = read_extras(extras, pr.num_seqs, &ex);
    if (st != PA_OK) return st;
    if (workspace_bytes < pl.workspace_bytes) return PA_ERR_WORKSPACE_TOO_SMALL;

    DecodeParams& p = *pp;
    memset(&p, 0, sizeof p);
    p.q = q;
    p.q_stride_b = q_stride_b;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.s_page = kv_stride_page;
    p.s_tok = kv_stride_tok;
    // (a split latent cache: virtual kv heads over the same rows)
    const int split = latent_head_split(pr);
    p.s_head = split > 1 ? 0 : kv_stride_head;
    p.block_table = block_table;
    p.bt_stride = bt_stride;
    p.seq_lens = seq_lens;
    p.num_seqs = pr.num_seqs;
    p.num_q_heads = pr.num_q_heads;
    p.num_kv_heads = pr.num_kv_heads * split;
    p.group = pr.num_q_heads / p.num_kv_heads;
    p.q_len = q_len;
    p.rows = p.group * q_len;
    p.q_stride_t = row;
    p.out_stride_t = orow;
    p.page_shift = ilog2(pr.page_size);
    p.window = pr.window;
    const float kl2e = 1.4426950408889634f;
    p.has_cap = softcap > 0.f;
    p.qk_scale2 = scale * k_scale * kl2e;
    if (p.has_cap) {
        p.cap_c1 = 2.f * scale * k_scale * kl2e / softcap;
        p.cap_c2 = softcap * kl2e;
    }
    p.v_scale = v_scale;
    p.sinks = ex.sinks;
    p.alibi = ex.alibi;
    p.k_desc = ex.k_desc;
    p.v_desc = ex.v_desc;
    p.desc_per_seq = ex.per_seq;
    p.out = out;
    p.out_stride_b = out_stride_b;
    // a piece costs its wave work beyond its tiles (the next sequence's page
    // list, Q rows and first tile are waited for); the ranges charge each
    // segment that much, in tiles' worth, so a range holding many short
    // sequences gets fewer tiles
    p.piece_cost = is_latent(pr) ? kLatentPieceCost
                   : pr.kv_dtype == PA_KV_FP8_E4M3 ? kFp8PieceCost : kBf16PieceCost;
    return PA_OK;
}

pa_status decode_launch(int passes, const pa_plan& pl, DecodeParams& p, void* workspace,
                        hipStream_t stream) {
    const pa_problem& pr = pl.prob;
    const DecLayout L = decode_layout(pr, pl.num_splits);
    char* ws = static_cast<char*>(workspace);
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(ws + L.lse);
    p.seg_rec = reinterpret_cast<int32_t*>(ws + L.rec);
    const bool uniform = pr.page_size >= 16;
    if (passes & kDecodeSplitPass) {
        const hipError_t e =
            is_latent(pr)
                ? launch_mla_decode(p, pr.head_dim, pr.head_dim_v, p.k_pool == p.v_pool,
                                    pl.waves_per_block, pl.num_splits, stream)
                : launch_decode(p, pr.head_dim, pr.kv_dtype == PA_KV_FP8_E4M3, uniform,
                                pl.waves_per_block, pl.num_splits, stream);
        if (e != hipSuccess) return PA_ERR_HIP;
    }
    if ((passes & kDecodeMergePass) &&
        launch_decode_merge(p, value_dim(pr), pr.num_seqs, p.num_kv_heads, stream) !=
            hipSuccess)
        return PA_ERR_HIP;
    return PA_OK;
}

}  // namespace pa

namespace {

pa_status decode_impl(int passes, int mode, const pa_plan* plan, const void* q, int64_t q_stride_b,
                      const void* k_pool, const void* v_pool, int64_t kv_stride_page,
                      int64_t kv_stride_tok, int64_t kv_stride_head, int64_t num_pages,
                      const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                      int32_t page_size, float scale, float softcap, int32_t window,
                      float k_scale, float v_scale, void* out, int64_t out_stride_b,
                      void* workspace, uint64_t workspace_bytes, const pa_extras* extras,
                      void* hip_stream) {
    DecodeParams p;
    bool empty = false;
    const pa_status st = decode_prepare(
        mode, plan, q, q_stride_b, k_pool, v_pool, kv_stride_page, kv_stride_tok,
        kv_stride_head, num_pages, block_table, bt_stride, seq_lens, page_size, scale, softcap,
        window, k_scale, v_scale, out, out_stride_b, workspace_bytes, extras, &p, &empty);
    if (st != PA_OK || empty) return st;
    if (!workspace) return PA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return PA_ERR_MISALIGNED;
    return decode_launch(passes, *plan, p, workspace, static_cast<hipStream_t>(hip_stream));
}

}  // namespace

extern "C" {

#define PA_DECODE_ARGS                                                                      \
    plan, q, q_stride_b, k_pool, v_pool, kv_stride_page, kv_stride_tok, kv_stride_head,     \
        num_pages, block_table, bt_stride, seq_lens, page_size, scale, softcap, window,     \
        k_scale, v_scale, out, out_stride_b, workspace, workspace_bytes, extras, hip_stream
#define PA_DECODE_PARAMS                                                                    \
    const pa_plan *plan, const void *q, int64_t q_stride_b, const void *k_pool,             \
        const void *v_pool, int64_t kv_stride_page, int64_t kv_stride_tok,                  \
        int64_t kv_stride_head, int64_t num_pages, const int32_t *block_table,              \
        int64_t bt_stride, const int32_t *seq_lens, int32_t page_size, float scale,         \
        float softcap, int32_t window, float k_scale, float v_scale, void *out,             \
        int64_t out_stride_b, void *workspace, uint64_t workspace_bytes,                   \
        const pa_extras *extras, void *hip_stream

pa_status paged_attn_decode(PA_DECODE_PARAMS) {
    return decode_impl(kDecodeBothPasses, PA_MODE_DECODE, PA_DECODE_ARGS);
}

pa_status paged_attn_decode_split(PA_DECODE_PARAMS) {
    return decode_impl(kDecodeSplitPass, PA_MODE_DECODE, PA_DECODE_ARGS);
}

pa_status paged_attn_decode_merge(PA_DECODE_PARAMS) {
    return decode_impl(kDecodeMergePass, PA_MODE_DECODE, PA_DECODE_ARGS);
}

pa_status paged_attn_verify(PA_DECODE_PARAMS) {
    return decode_impl(kDecodeBothPasses, PA_MODE_VERIFY, PA_DECODE_ARGS);
}

pa_status paged_attn_gather(const pa_plan* plan, const void* k_pool, const void* v_pool,
                            int64_t kv_stride_page, int64_t kv_stride_tok,
                            int64_t kv_stride_head, int64_t num_pages,
                            const int32_t* block_table, int64_t bt_stride,
                            const int32_t* seq_lens, void* k_out, void* v_out,
                            void* hip_stream) {
    if (!plan) return PA_ERR_NULL_POINTER;
    const pa_plan& pl = *plan;
    const pa_problem& pr = pl.prob;
    pa_status st = check_problem(pr);
    if (st != PA_OK) return st;
    if (is_latent(pr)) return PA_ERR_UNSUPPORTED;   // rows of 64 or 128 entries only
    if (pr.num_seqs == 0) return PA_OK;
    if (!seq_lens || !k_out || !v_out) return PA_ERR_NULL_POINTER;
    st = check_pools(pl, k_pool, v_pool, kv_stride_page, kv_stride_tok, kv_stride_head,
                     num_pages, block_table, bt_stride);
    if (st != PA_OK) return st;
    if (!aligned16(k_out) || !aligned16(v_out)) return PA_ERR_MISALIGNED;
    GatherParams p;
    memset(&p, 0, sizeof p);
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.s_page = kv_stride_page;
    p.s_tok = kv_stride_tok;
    p.s_head = kv_stride_head;
    p.block_table = block_table;
    p.bt_stride = bt_stride;
    p.seq_lens = seq_lens;
    p.num_seqs = pr.num_seqs;
    p.num_kv_heads = pr.num_kv_heads;
    p.page_shift = ilog2(pr.page_size);
    p.k_out = k_out;
    p.v_out = v_out;
    if (launch_gather(p, pr.head_dim, pr.kv_dtype == PA_KV_FP8_E4M3,
                      static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return PA_ERR_HIP;
    return PA_OK;
}

pa_status paged_attn_cache_append(const void* key, const void* value, int64_t num_tokens,
                                  int64_t kv_row_stride, int32_t num_kv_heads,
                                  int32_t head_dim, void* k_pool, void* v_pool,
                                  int64_t kv_stride_page, int64_t kv_stride_tok,
                                  int64_t kv_stride_head, int64_t num_pages, int32_t page_size,
                                  int32_t kv_dtype, const int64_t* slot_mapping, float k_scale,
                                  float v_scale, void* hip_stream) {
    if (num_tokens < 0 || num_kv_heads < 1 || page_size < 1 || num_pages < 1)
        return PA_ERR_INVALID_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (kv_dtype != PA_KV_BF16 && kv_dtype != PA_KV_FP8_E4M3) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(page_size) || page_size > 4096) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_pool || !v_pool || !slot_mapping) return PA_ERR_NULL_POINTER;
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (kv_row_stride < row || kv_stride_page < 0 || kv_stride_tok < 0 || kv_stride_head < 0)
        return PA_ERR_INVALID_SHAPE;
    if (num_tokens * (row / 8) >= ((int64_t)1 << 40)) return PA_ERR_UNSUPPORTED;
    const int64_t eb = elem_bytes(kv_dtype);
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (kv_row_stride * 2) % 16 || (kv_stride_page * eb) % 16 || (kv_stride_tok * eb) % 16 ||
        (kv_stride_head * eb) % 16)
        return PA_ERR_MISALIGNED;
    if (kv_dtype == PA_KV_FP8_E4M3 &&
        !(isfinite(k_scale) && isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
        return PA_ERR_INVALID_SHAPE;
    AppendParams p;
    memset(&p, 0, sizeof p);
    p.key = key;
    p.value = value;
    p.row_stride = kv_row_stride;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.s_page = kv_stride_page;
    p.s_tok = kv_stride_tok;
    p.s_head = kv_stride_head;
    p.slot_mapping = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_kv_heads = num_kv_heads;
    p.head_dim = head_dim;
    p.page_shift = ilog2(page_size);
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    if (launch_cache_append(p, kv_dtype == PA_KV_FP8_E4M3, static_cast<hipStream_t>(hip_stream)) !=
        hipSuccess)
        return PA_ERR_HIP;
    return PA_OK;
}

pa_status paged_attn_check_inputs(const pa_plan* plan, const int32_t* lens,
                                  const int32_t* block_table, int64_t bt_stride,
                                  int64_t num_pages, const int32_t* cu_seqlens_q,
                                  int32_t* bad_array, int64_t* bad_index) {
    if (bad_array) *bad_array = 0;
    if (bad_index) *bad_index = -1;
    if (!plan) return PA_ERR_NULL_POINTER;
    const pa_problem& pr = plan->prob;
    const pa_status st = check_problem(pr);
    if (st != PA_OK) return st;
    if (bt_stride < pr.max_pages_per_seq || num_pages < 1) return PA_ERR_INVALID_SHAPE;
    if (pr.num_seqs == 0) return PA_OK;
    const bool extend = pr.mode == PA_MODE_EXTEND;
    if (!lens || !block_table || (extend && !cu_seqlens_q)) return PA_ERR_NULL_POINTER;
    const auto fail = [&](int32_t array, int64_t index) {
        if (bad_array) *bad_array = array;
        if (bad_index) *bad_index = index;
        return PA_ERR_INVALID_SHAPE;
    };
    for (int64_t b = 0; b < pr.num_seqs; ++b) {
        const int32_t L = lens[b];
        if (L < 0 || L > pr.max_kv_len) return fail(1, b);
        const int64_t pages = cdiv(L, pr.page_size);
        for (int64_t j = 0; j < pages; ++j) {
            const int32_t page = block_table[b * bt_stride + j];
            if (page < 0 || page >= num_pages) return fail(2, b * bt_stride + j);
        }
    }
    if (extend) {
        if (cu_seqlens_q[0] != 0) return fail(3, 0);
        for (int64_t b = 0; b < pr.num_seqs; ++b) {
            const int64_t n = (int64_t)cu_seqlens_q[b + 1] - cu_seqlens_q[b];
            if (n < 0 || n > pr.max_q_len) return fail(3, b + 1);
        }
        if (cu_seqlens_q[pr.num_seqs] != pr.total_q) return fail(3, pr.num_seqs);
    }
    return PA_OK;
}

pa_status paged_attn_extend(const pa_plan* plan, const void* q, const void* k_new,
                            const void* v_new, const int32_t* cu_seqlens_q,
                            const int32_t* ctx_lens, const void* k_pool, const void* v_pool,
                            int64_t kv_stride_page, int64_t kv_stride_tok,
                            int64_t kv_stride_head, int64_t num_pages,
                            const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                            float scale, float softcap, int32_t window, float k_scale,
                            float v_scale, void* out, void* workspace, uint64_t workspace_bytes,
                            const pa_extras* extras, void* hip_stream) {
    if (!plan) return PA_ERR_NULL_POINTER;
    const pa_plan& pl = *plan;
    const pa_problem& pr = pl.prob;
    pa_status st = check_problem(pr);
    if (st != PA_OK) return st;
    if (pr.mode != PA_MODE_EXTEND) return PA_ERR_PLAN_MISMATCH;
    if (page_size != pr.page_size || window != pr.window) return PA_ERR_PLAN_MISMATCH;
    if (pl.num_splits < 1 || pl.num_splits > kMaxWorkers ||
        pl.workspace_bytes != (uint64_t)extend_layout(pr, pl.num_splits).total)
        return PA_ERR_PLAN_MISMATCH;
    if (pr.num_seqs == 0 || pr.total_q == 0) return PA_OK;
    if (!q || !k_new || !v_new || !cu_seqlens_q || !ctx_lens || !out) return PA_ERR_NULL_POINTER;
    st = check_pools(pl, k_pool, v_pool, kv_stride_page, kv_stride_tok, kv_stride_head,
                     num_pages, block_table, bt_stride);
    if (st != PA_OK) return st;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
        return PA_ERR_MISALIGNED;
    if (!isfinite(scale) || !isfinite(softcap) || !isfinite(k_scale) || !isfinite(v_scale))
        return PA_ERR_INVALID_SHAPE;
    Extras ex;
    st = read_extras(extras, pr.num_seqs, &ex);
    if (st != PA_OK) return st;
    if (workspace_bytes < pl.workspace_bytes) return PA_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace) return PA_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return PA_ERR_MISALIGNED;

    ExtendParams p;
    memset(&p, 0, sizeof p);
    // (a piece costs its block a prologue and an output beyond its tiles:
    // the item stream charges each item that many tiles' worth)
    p.piece_cost = kExtendPieceCost;
    {
        const ExtLayout L = extend_layout(pr, pl.num_splits);
        char* ws = static_cast<char*>(workspace);
        p.pfx = reinterpret_cast<int64_t*>(ws);
        p.rec = reinterpret_cast<int32_t*>(ws + L.rec);
        p.part_lse = reinterpret_cast<float*>(ws + L.lse);
        p.part_o = reinterpret_cast<float*>(ws + L.o);
    }
    p.sinks = ex.sinks;
    p.alibi = ex.alibi;
    p.k_desc = ex.k_desc;
    p.v_desc = ex.v_desc;
    p.desc_per_seq = ex.per_seq;
    p.q = q;
    p.k_new = k_new;
    p.v_new = v_new;
    p.cu_seqlens_q = cu_seqlens_q;
    p.ctx_lens = ctx_lens;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.s_page = kv_stride_page;
    p.s_tok = kv_stride_tok;
    p.s_head = kv_stride_head;
    p.block_table = block_table;
    p.bt_stride = bt_stride;
    p.num_seqs = pr.num_seqs;
    p.num_q_heads = pr.num_q_heads;
    p.num_kv_heads = pr.num_kv_heads;
    p.group = pr.num_q_heads / pr.num_kv_heads;
    p.page_shift = ilog2(pr.page_size);
    p.window = pr.window;
    p.q_tiles = (int32_t)cdiv((int64_t)pr.max_q_len * p.group, extend_rows_per_block());
    const float kl2e = 1.4426950408889634f;
    p.has_cap = softcap > 0.f;
    p.qk_scale2 = scale * kl2e;
    p.qk_scale2_ctx = scale * k_scale * kl2e;
    if (p.has_cap) {
        p.cap_c1 = 2.f * scale * kl2e / softcap;
        p.cap_c1_ctx = 2.f * scale * k_scale * kl2e / softcap;
        p.cap_c2 = softcap * kl2e;
    }
    p.v_scale = v_scale;
    p.out = out;
    if (launch_extend(p, pr.head_dim, pr.kv_dtype == PA_KV_FP8_E4M3, pl.num_splits,
                      static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return PA_ERR_HIP;
    return PA_OK;
}

}  // extern "C"
