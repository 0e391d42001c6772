/*
 * pa_oracle.c -- plain, slow fp64 CPU oracle for paged GQA attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this file's library.  It shares no code,
 * header, table or helper with the HIP library; it decodes bf16 and fp8 itself
 * and walks the block table itself.
 *
 * What it computes (all arithmetic in double):
 *
 *  decode   For sequence b with L cached tokens and query head h, the key/value
 *           head is g = h / (Hq/Hkv) (contiguous grouping, as in the
 *           `_fwd_grouped_kernel_stage1` of "vllm/attention/ops/
 *           triton_decode_attention.py" and `cur_kv_head` in `_fwd_kernel` of
 *           "vllm/attention/ops/prefix_prefill.py").  Token t lives in
 *           physical page bt[b][t / P] at row t % P (the `Req_to_tokens`
 *           lookup of `_fwd_kernel_stage1`; the `[num_blocks, P, Hkv, D]`
 *           view of `_kv_cache_views` in the vLLM "b12x" backend page).
 *           The query is the token at position L-1; its own key/value is
 *           already in the cache (the b12x page writes the new token with
 *           `do_kv_cache_update` before attention runs).
 *           Keys t in [lo, L) are attended, lo = max(0, L-W) when a sliding
 *           window W > 0 is given: a key is kept iff pos_q - pos_k < W
 *           (the b12x page stores `window_left = sliding_window - 1`; the
 *           prefix_prefill `_fwd_kernel` keeps `pos_q - pos_k < SLIDING_WINDOW`).
 *             s_t   = scale * <q, k_t>,   k_t = dec(K) * k_scale
 *             s_t   = c * tanh(s_t / c)   if the soft-cap c > 0 (applied after
 *                                         the scale, as `logit_cap` in
 *                                         `_fwd_kernel_stage1`)
 *             out   = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m),  m = max s_t
 *             lse   = m + ln sum_t exp(s_t - m)
 *           An empty key range (L == 0) gives a zero row and lse = -inf
 *           (the b12x `forward` zero-fills its output when there is nothing
 *           to attend).
 *
 *  split    The key range [lo, L) is cut into S contiguous parts of
 *           ceil(n/S) tokens (the split partition of `_fwd_kernel_stage1`);
 *           each non-empty part yields (o_s, lse_s) by the definition above
 *           and the parts are merged as in `_fwd_kernel_stage2`:
 *             out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M),
 *             M = max_s lse_s, empty parts skipped.
 *
 *  extend   For sequence b with C cached tokens and n = cu[b+1]-cu[b] new
 *           tokens, new row i sits at position C + i and attends to every
 *           cached token j < C (through the pages, no causal mask) and to new
 *           tokens C+i' with i' <= i (contiguous k_new/v_new rows cu[b]+i'),
 *           with the same window rule, scale, soft-cap and softmax; the output
 *           is the normalised softmax-weighted sum (the two loops of
 *           `_fwd_kernel` in "vllm/attention/ops/prefix_prefill.py", and
 *           the final `acc / l_i` of `_fwd_kernel_flash_attn_v2`).  The cache
 *           scales apply to cached keys/values only; new rows are bf16.
 *
 *  verify   q_len query rows per sequence (the speculative verify step of
 *           the vLLM "b12x" backend page: `1 + num_speculative_tokens` rows
 *           for every request, their keys/values already in the cache and
 *           counted by seq_lens).  Row i of sequence b sits at position
 *           L - q_len + i and attends causally to the cached tokens up to
 *           it: the decode definition with L replaced by L - q_len + i + 1.
 *
 *  sinks    Optional per-query-head fp32 logits sink[h] (`attention_sink_bias`
 *           handed to `bind` by the vLLM "b12x" backend page, shape
 *           [num_heads], kept in fp32 after weight loading; the kernel that
 *           uses it is not printed).  Read as an attention sink: one more
 *           logit in the softmax normaliser that carries no value,
 *             out = sum_t exp(s_t - m) v_t / (exp(sink - m) + sum_t exp(s_t - m)),
 *             m = max(sink, max_t s_t),  lse = m + ln(that denominator);
 *           the sink is taken as it is (not scaled, not soft-capped).  With
 *           splits it enters the merge once:
 *             out = sum_s exp(lse_s - M) o_s / (exp(sink - M) + sum_s exp(lse_s - M)).
 *           A row with no key is still a zero row.
 *
 *  alibi    Optional per-query-head fp32 slopes a[h] (`_fwd_kernel_alibi` on
 *           the prefix_prefill page, whose `Alibi_slopes` is indexed by the
 *           query head): a key at position j seen from a query at position p
 *           gets the bias a[h] * (j - p) added to its scaled (and capped)
 *           score.  Keys after the query are masked as without ALiBi (that
 *           page's `alibi <= 0` test is this causal limit for the positive
 *           slopes ALiBi uses); the window rule is unchanged.
 *
 *  latent   Decode with a value head dim Dv smaller than the key head dim D
 *           (the grouped kernel `_fwd_grouped_kernel_stage1` of the decode
 *           page takes Lk != Lv, e.g. Lk = 576 split as 512 + 64 and
 *           Lv = 512): the scores use all D entries of q and of the key row,
 *           and the value of token t is the first Dv entries of the value
 *           pool's row at t's place; the value pool has the key pool's
 *           layout (rows of D entries).  A latent cache passes one pool as
 *           both, so the value is the first Dv entries of the key row.  The
 *           output rows have Dv entries.  Dv = D is ordinary decode.
 *
 *  descales Optional per-request fp32 descales kd[b], vd[b] (the b12x
 *           `_prepare_fp8_descales` gives one value per request): a cached
 *           key of sequence b is dec(K) * k_scale * kd[b], a cached value
 *           dec(V) * v_scale * vd[b].  New extend rows are not cache
 *           elements and take no descale.
 *
 *  append   The cache write that precedes attention (`do_kv_cache_update` on
 *           the vLLM "b12x" backend page, which hands key, value, the
 *           caches, `slot_mapping` and the k/v scales to
 *           `reshape_and_cache_flash`): new token i goes to flat slot
 *           s = slot_mapping[i] -- page s / P, row s % P -- for every kv head;
 *           s < 0 marks a padding token that is not written.  A bf16 cache
 *           receives the bf16 element unchanged; an e4m3fn cache receives
 *           enc(x / scale), the quotient a correctly rounded fp32 division
 *           and enc the nearest e4m3fn value (ties to the even code,
 *           magnitudes past 448 saturating to 448, NaN to NaN).
 *
 * Element decoding:
 *   bf16    the 16 bits are the high half of an IEEE binary32.
 *   e4m3fn  OCP 8-bit float: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 *           bits, subnormals when the exponent field is 0, S.1111.111 is NaN,
 *           no infinities (largest finite 448).
 *
 * Threads: the outer (row) loop is shared between `threads` POSIX threads;
 * each output row is computed by exactly one thread in a fixed order, so the
 * result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_KV_BF16 = 0, ORC_KV_E4M3FN = 1 };

double orc_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double orc_e4m3fn(uint8_t bits)
{
    int sign = bits >> 7;
    int expo = (bits >> 3) & 0xF;
    int mant = bits & 0x7;
    double mag;
    if (expo == 0xF && mant == 0x7)
        return NAN;
    if (expo == 0)
        mag = ldexp((double)mant, -9);              /* (mant/8) * 2^(1-7) */
    else
        mag = ldexp((double)(8 + mant), expo - 10); /* (1+mant/8) * 2^(expo-7) */
    return sign ? -mag : mag;
}

/* One cached element: page `page`, row `row`, head `g`, lane `d`. */
static double cache_elem(const void *pool, int kv_dtype, int64_t page, int row,
                         int g, int d, int P, int Hkv, int D)
{
    int64_t idx = ((page * P + row) * (int64_t)Hkv + g) * D + d;
    if (kv_dtype == ORC_KV_E4M3FN)
        return orc_e4m3fn(((const uint8_t *)pool)[idx]);
    return orc_bf16(((const uint16_t *)pool)[idx]);
}

/* ------------------------------------------------------------------ */
/* Shared problem description                                          */
/* ------------------------------------------------------------------ */
typedef struct {
    int B, Hq, Hkv, D, P, kv_dtype;
    int Dv;                     /* value entries per row (<= D; decode only < D) */
    const uint16_t *q;          /* decode [B][Hq][D]; extend [total_q][Hq][D] */
    const void *k_pool, *v_pool;/* [num_pages][P][Hkv][D] */
    int64_t num_pages;
    const int32_t *bt;          /* [B][bt_stride] */
    int64_t bt_stride;
    const int32_t *seq_lens;    /* decode: cached tokens incl. the query token */
    double scale, softcap, k_scale, v_scale;
    const float *sinks;         /* [Hq] or NULL */
    const float *alibi;         /* [Hq] ALiBi slopes or NULL */
    const float *k_desc, *v_desc; /* [B] per-request descales or NULL */
    int window;
    int num_splits;             /* decode: 0 = one pass over the key range */
    int q_len;                  /* verify: query rows per sequence */
    /* extend */
    const uint16_t *k_new, *v_new; /* [total_q][Hkv][D] */
    const int32_t *cu_q, *ctx_lens;
    const int64_t *rows;        /* token rows to compute (extend); NULL = all */
    int64_t n_rows;
    /* outputs */
    double *out, *lse;
    int status;
} orc_problem;

/*
 * Softmax-weighted sum over a list of keys given as (score, value row), with
 * an optional sink logit (-inf: none) that joins the normaliser only.
 * The definition: out = sum exp(s - m) v / (exp(sink - m) + sum exp(s - m)),
 * lse = m + ln(that denominator), m = max(sink, max s).
 */
static void softmax_sum(const double *s, const double *v, int64_t n, int D,
                        double sink, double *out, double *lse)
{
    double m = sink, z = 0.0;
    int64_t t;
    int d;
    for (d = 0; d < D; ++d)
        out[d] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    for (t = 0; t < n; ++t)
        if (s[t] > m)
            m = s[t];
    if (sink > -INFINITY)
        z = exp(sink - m);
    for (t = 0; t < n; ++t) {
        double w = exp(s[t] - m);
        z += w;
        for (d = 0; d < D; ++d)
            out[d] += w * v[t * D + d];
    }
    for (d = 0; d < D; ++d)
        out[d] /= z;
    *lse = m + log(z);
}

static double cap_score(double s, double c)
{
    return c > 0.0 ? c * tanh(s / c) : s;
}

/* The sink logit of query head h (-inf when there are none). */
static double sink_of(const orc_problem *pr, int h)
{
    return pr->sinks ? (double)pr->sinks[h] : -INFINITY;
}

/* The ALiBi bias of a key at position j for query head h at position pos. */
static double alibi_bias(const orc_problem *pr, int h, int64_t j, int64_t pos)
{
    return pr->alibi ? (double)pr->alibi[h] * (double)(j - pos) : 0.0;
}

/* Gather keys [t0, t1) of (b, g) from the cache: scores against q, and values. */
static void gather_cached(const orc_problem *pr, int b, int g, const double *q,
                          int64_t t0, int64_t t1, double *s, double *v)
{
    double ks = pr->k_scale * (pr->k_desc ? (double)pr->k_desc[b] : 1.0);
    double vs = pr->v_scale * (pr->v_desc ? (double)pr->v_desc[b] : 1.0);
    int64_t t;
    int d;
    for (t = t0; t < t1; ++t) {
        int64_t page = pr->bt[b * pr->bt_stride + t / pr->P];
        int row = (int)(t % pr->P);
        double dot = 0.0;
        for (d = 0; d < pr->D; ++d) {
            double k = cache_elem(pr->k_pool, pr->kv_dtype, page, row, g, d,
                                  pr->P, pr->Hkv, pr->D) * ks;
            dot += q[d] * k;
        }
        /* the value: the first Dv entries of the value pool's row */
        for (d = 0; d < pr->Dv; ++d)
            v[(t - t0) * pr->Dv + d] =
                cache_elem(pr->v_pool, pr->kv_dtype, page, row, g, d, pr->P,
                           pr->Hkv, pr->D) * vs;
        s[t - t0] = cap_score(pr->scale * dot, pr->softcap);
    }
}

/* ------------------------------------------------------------------ */
/* Decode                                                              */
/* ------------------------------------------------------------------ */
static void decode_row(const orc_problem *pr, int b, int h, double *q,
                       double *s, double *v, double *os, double *lses)
{
    int G = pr->Hq / pr->Hkv;
    int g = h / G;
    int D = pr->D, Dv = pr->Dv;
    int64_t L = pr->seq_lens[b];
    int64_t lo = (pr->window > 0 && L - pr->window > 0) ? L - pr->window : 0;
    double *out = pr->out + ((int64_t)b * pr->Hq + h) * Dv;
    double *lse = pr->lse + (int64_t)b * pr->Hq + h;
    int d;

    for (d = 0; d < D; ++d)
        q[d] = orc_bf16(pr->q[((int64_t)b * pr->Hq + h) * D + d]);

    if (pr->num_splits <= 0) {
        int64_t t;
        gather_cached(pr, b, g, q, lo, L, s, v);
        for (t = lo; t < L; ++t)
            s[t - lo] += alibi_bias(pr, h, t, L - 1);
        softmax_sum(s, v, L - lo, Dv, sink_of(pr, h), out, lse);
        return;
    }

    /* Split partition, then the log-sum-exp merge of the parts. */
    {
        int S = pr->num_splits, sp;
        int64_t n = L - lo;
        int64_t len = (n + S - 1) / S;
        double M = -INFINITY, z = 0.0;
        for (sp = 0; sp < S; ++sp) {
            int64_t a = lo + len * sp;
            int64_t e = a + len < L ? a + len : L;
            if (e <= a) {
                lses[sp] = -INFINITY;
                continue;
            }
            gather_cached(pr, b, g, q, a, e, s, v);
            {
                int64_t t;
                for (t = a; t < e; ++t)
                    s[t - a] += alibi_bias(pr, h, t, L - 1);
            }
            softmax_sum(s, v, e - a, Dv, -INFINITY, os + (int64_t)sp * Dv, &lses[sp]);
            if (lses[sp] > M)
                M = lses[sp];
        }
        for (d = 0; d < Dv; ++d)
            out[d] = 0.0;
        if (M == -INFINITY) {
            *lse = -INFINITY;
            return;
        }
        if (sink_of(pr, h) > M)
            M = sink_of(pr, h);
        if (sink_of(pr, h) > -INFINITY)
            z = exp(sink_of(pr, h) - M);
        for (sp = 0; sp < S; ++sp) {
            double w;
            if (lses[sp] == -INFINITY)
                continue;
            w = exp(lses[sp] - M);
            z += w;
            for (d = 0; d < Dv; ++d)
                out[d] += w * os[(int64_t)sp * Dv + d];
        }
        for (d = 0; d < Dv; ++d)
            out[d] /= z;
        *lse = M + log(z);
    }
}

/* ------------------------------------------------------------------ */
/* Verify: q_len query rows per sequence, the last q_len cached tokens. */
/* Row i sits at position L - q_len + i, so its keys are the first      */
/* L - q_len + i + 1 tokens (causal), with the decode window rule.      */
/* ------------------------------------------------------------------ */
static void verify_row(const orc_problem *pr, int64_t it, double *q, double *s, double *v)
{
    int Hq = pr->Hq, D = pr->D, ql = pr->q_len;
    int h = (int)(it % Hq);
    int64_t bi = it / Hq;                       /* (sequence, row) */
    int b = (int)(bi / ql), i = (int)(bi % ql);
    int64_t L = (int64_t)pr->seq_lens[b] - ql + i + 1;
    int64_t lo = (pr->window > 0 && L - pr->window > 0) ? L - pr->window : 0;
    double *out = pr->out + (bi * Hq + h) * D;
    double lse;
    int d;
    if (L <= 0) {                               /* nothing to attend: zero row */
        for (d = 0; d < D; ++d)
            out[d] = 0.0;
        return;
    }
    for (d = 0; d < D; ++d)
        q[d] = orc_bf16(pr->q[(bi * Hq + h) * D + d]);
    gather_cached(pr, b, h / (Hq / pr->Hkv), q, lo, L, s, v);
    {
        int64_t t;
        for (t = lo; t < L; ++t)
            s[t - lo] += alibi_bias(pr, h, t, L - 1);     /* query at L - 1 */
    }
    softmax_sum(s, v, L - lo, D, sink_of(pr, h), out, &lse);
}

/* ------------------------------------------------------------------ */
/* Extend                                                              */
/* ------------------------------------------------------------------ */
static void extend_row(const orc_problem *pr, int64_t r, int h, double *q,
                       double *s, double *v)
{
    int G = pr->Hq / pr->Hkv;
    int g = h / G;
    int D = pr->D;
    int b = 0, d;
    int64_t C, i, pos, j, n = 0;
    double lse;

    while (b + 1 < pr->B && pr->cu_q[b + 1] <= r)
        ++b;
    C = pr->ctx_lens[b];
    i = r - pr->cu_q[b];
    pos = C + i;
    for (d = 0; d < D; ++d)
        q[d] = orc_bf16(pr->q[(r * pr->Hq + h) * D + d]);

    /* cached keys j < C, through the block table */
    for (j = 0; j < C; ++j) {
        if (pr->window > 0 && pos - j >= pr->window)
            continue;
        gather_cached(pr, b, g, q, j, j + 1, s + n, v + n * D);
        s[n] += alibi_bias(pr, h, j, pos);
        ++n;
    }
    /* new keys C + i' for i' <= i, contiguous rows */
    for (j = 0; j <= i; ++j) {
        int64_t row = pr->cu_q[b] + j;
        double dot = 0.0;
        if (pr->window > 0 && pos - (C + j) >= pr->window)
            continue;
        for (d = 0; d < D; ++d) {
            dot += q[d] * orc_bf16(pr->k_new[(row * pr->Hkv + g) * D + d]);
            v[n * D + d] = orc_bf16(pr->v_new[(row * pr->Hkv + g) * D + d]);
        }
        s[n] = cap_score(pr->scale * dot, pr->softcap) + alibi_bias(pr, h, C + j, pos);
        ++n;
    }
    softmax_sum(s, v, n, D, sink_of(pr, h), pr->out + (r * pr->Hq + h) * D, &lse);
}

/* ------------------------------------------------------------------ */
/* Threading: rows are dealt by an atomic counter.                     */
/* ------------------------------------------------------------------ */
typedef struct {
    orc_problem *pr;
    int is_extend;
    int64_t n_items;
    int64_t max_keys;
    int64_t *next;
    pthread_mutex_t *mu;
} orc_job;

static void *worker(void *arg)
{
    orc_job *job = (orc_job *)arg;
    orc_problem *pr = job->pr;
    int D = pr->D;
    int S = pr->num_splits > 0 ? pr->num_splits : 1;
    double *q = malloc(sizeof(double) * D);
    double *s = malloc(sizeof(double) * (job->max_keys + 1));
    double *v = malloc(sizeof(double) * (job->max_keys + 1) * D);
    double *os = malloc(sizeof(double) * S * D);
    double *lses = malloc(sizeof(double) * S);
    if (!q || !s || !v || !os || !lses) {
        pthread_mutex_lock(job->mu);
        pr->status = -2;
        pthread_mutex_unlock(job->mu);
        goto done;
    }
    for (;;) {
        int64_t it;
        pthread_mutex_lock(job->mu);
        it = (*job->next)++;
        pthread_mutex_unlock(job->mu);
        if (it >= job->n_items)
            break;
        if (job->is_extend == 2) {
            verify_row(pr, it, q, s, v);
        } else if (job->is_extend) {
            int64_t r = pr->rows ? pr->rows[it / pr->Hq] : it / pr->Hq;
            extend_row(pr, r, (int)(it % pr->Hq), q, s, v);
        } else {
            decode_row(pr, (int)(it / pr->Hq), (int)(it % pr->Hq), q, s, v, os,
                       lses);
        }
    }
done:
    free(q);
    free(s);
    free(v);
    free(os);
    free(lses);
    return NULL;
}

static int run_jobs(orc_problem *pr, int is_extend, int64_t n_items,
                    int64_t max_keys, int threads)
{
    pthread_t *tid;
    orc_job job;
    pthread_mutex_t mu = PTHREAD_MUTEX_INITIALIZER;
    int64_t next = 0;
    int t;
    if (threads < 1)
        threads = 1;
    tid = malloc(sizeof(pthread_t) * threads);
    if (!tid)
        return -2;
    job.pr = pr;
    job.is_extend = is_extend;
    job.n_items = n_items;
    job.max_keys = max_keys;
    job.next = &next;
    job.mu = &mu;
    pr->status = 0;
    for (t = 0; t < threads; ++t)
        pthread_create(&tid[t], NULL, worker, &job);
    for (t = 0; t < threads; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    return pr->status;
}

static int check_common(int B, int Hq, int Hkv, int D, int P, int kv_dtype)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0)
        return -1;
    if (Hq % Hkv != 0)
        return -1;
    if (kv_dtype != ORC_KV_BF16 && kv_dtype != ORC_KV_E4M3FN)
        return -1;
    return 0;
}

/*
 * Decode oracle.  out [B][Hq][Dv] and lse [B][Hq] (natural log) are written;
 * Dv is the value head dim (0: D; else 1 <= Dv <= D, see "latent" above).
 * num_splits == 0 evaluates the definition in one pass over the key range;
 * num_splits > 0 evaluates the split partition and the log-sum-exp merge.
 * sinks [Hq], the per-request descales k_desc/v_desc [B] and the ALiBi
 * slopes alibi [Hq] are optional (NULL: none / 1 / none).  Returns 0, -1 on a bad argument, -2 when memory runs out.
 */
int orc_decode(int B, int Hq, int Hkv, int D, int Dv, int P, int kv_dtype,
               const uint16_t *q, const void *k_pool, const void *v_pool,
               int64_t num_pages, const int32_t *block_table,
               int64_t bt_stride, const int32_t *seq_lens, double scale,
               double softcap, int window, double k_scale, double v_scale,
               int num_splits, double *out, double *lse, int threads,
               const float *sinks, const float *k_desc, const float *v_desc,
               const float *alibi)
{
    orc_problem pr;
    int64_t max_keys = 0;
    int b;
    if (check_common(B, Hq, Hkv, D, P, kv_dtype) || num_splits < 0)
        return -1;
    if (Dv == 0)
        Dv = D;
    if (Dv < 1 || Dv > D)
        return -1;
    memset(&pr, 0, sizeof pr);
    pr.B = B; pr.Hq = Hq; pr.Hkv = Hkv; pr.D = D; pr.Dv = Dv; pr.P = P;
    pr.kv_dtype = kv_dtype;
    pr.q = q; pr.k_pool = k_pool; pr.v_pool = v_pool;
    pr.num_pages = num_pages;
    pr.bt = block_table; pr.bt_stride = bt_stride; pr.seq_lens = seq_lens;
    pr.scale = scale; pr.softcap = softcap; pr.window = window;
    pr.k_scale = k_scale; pr.v_scale = v_scale;
    pr.sinks = sinks; pr.k_desc = k_desc; pr.v_desc = v_desc; pr.alibi = alibi;
    pr.num_splits = num_splits;
    pr.out = out; pr.lse = lse;
    for (b = 0; b < B; ++b) {
        if (seq_lens[b] < 0)
            return -1;
        if (seq_lens[b] > max_keys)
            max_keys = seq_lens[b];
    }
    return run_jobs(&pr, 0, (int64_t)B * Hq, max_keys, threads);
}

/*
 * Extend oracle.  Computes output rows for the token indices listed in
 * `rows` (n_rows of them), or for every token when rows == NULL
 * (n_rows = total_q).  out is [total_q][Hq][D]; only listed rows are written.
 * sinks, k_desc, v_desc, alibi as for orc_decode.
 */
int orc_extend(int B, int Hq, int Hkv, int D, int P, int kv_dtype,
               const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
               const int32_t *cu_seqlens_q, const int32_t *ctx_lens,
               const void *k_pool, const void *v_pool, int64_t num_pages,
               const int32_t *block_table, int64_t bt_stride, double scale,
               double softcap, int window, double k_scale, double v_scale,
               const int64_t *rows, int64_t n_rows, double *out, int threads,
               const float *sinks, const float *k_desc, const float *v_desc,
               const float *alibi)
{
    orc_problem pr;
    int64_t max_keys = 0;
    int b;
    if (check_common(B, Hq, Hkv, D, P, kv_dtype) || B < 1)
        return -1;
    memset(&pr, 0, sizeof pr);
    pr.B = B; pr.Hq = Hq; pr.Hkv = Hkv; pr.D = D; pr.Dv = D; pr.P = P;
    pr.kv_dtype = kv_dtype;
    pr.q = q; pr.k_new = k_new; pr.v_new = v_new;
    pr.cu_q = cu_seqlens_q; pr.ctx_lens = ctx_lens;
    pr.k_pool = k_pool; pr.v_pool = v_pool; pr.num_pages = num_pages;
    pr.bt = block_table; pr.bt_stride = bt_stride;
    pr.scale = scale; pr.softcap = softcap; pr.window = window;
    pr.k_scale = k_scale; pr.v_scale = v_scale;
    pr.sinks = sinks; pr.k_desc = k_desc; pr.v_desc = v_desc; pr.alibi = alibi;
    pr.rows = rows; pr.n_rows = n_rows;
    pr.out = out;
    for (b = 0; b < B; ++b) {
        int64_t n = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        if (n < 0 || ctx_lens[b] < 0)
            return -1;
        if (ctx_lens[b] + n > max_keys)
            max_keys = ctx_lens[b] + n;
    }
    if (!rows)
        n_rows = cu_seqlens_q[B];
    return run_jobs(&pr, 1, n_rows * Hq, max_keys, threads);
}

/* e4m3fn code nearest to the float x: the table of the 127 finite
 * non-negative codes is searched for the closest magnitude (ties go to the
 * even code); NaN keeps its sign with the NaN code, everything past the
 * largest finite value lands on it. */
uint8_t orc_e4m3fn_encode(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    int best = 0, c;
    double best_d = INFINITY;
    if (isnan(x))
        return (uint8_t)(sign | 0x7F);
    if (a > 448.0)          /* saturation (the distances would lose precision) */
        a = 448.0;
    for (c = 0; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3fn((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)(sign | best);
}

/* Cache append: key/value bf16 rows [num_tokens, Hkv, D] with token stride
 * `row_stride` elements; the pools as in decode (strides in elements). */
int orc_cache_append(int64_t num_tokens, int Hkv, int D, int P, int kv_dtype,
                     const uint16_t *key, const uint16_t *value, int64_t row_stride,
                     void *k_pool, void *v_pool, int64_t s_page, int64_t s_tok,
                     int64_t s_head, int64_t num_pages, const int64_t *slot_mapping,
                     float k_scale, float v_scale)
{
    int64_t i;
    if (num_tokens < 0 || Hkv < 1 || D < 1 || P < 1 ||
        (kv_dtype != ORC_KV_BF16 && kv_dtype != ORC_KV_E4M3FN))
        return -1;
    for (i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i], page, off;
        int h, d;
        if (slot < 0)
            continue;
        page = slot / P;
        if (page >= num_pages)
            return -2;
        for (h = 0; h < Hkv; ++h) {
            off = page * s_page + (slot % P) * s_tok + (int64_t)h * s_head;
            for (d = 0; d < D; ++d) {
                uint16_t kb = key[i * row_stride + (int64_t)h * D + d];
                uint16_t vb = value[i * row_stride + (int64_t)h * D + d];
                if (kv_dtype == ORC_KV_BF16) {
                    ((uint16_t *)k_pool)[off + d] = kb;
                    ((uint16_t *)v_pool)[off + d] = vb;
                } else {
                    float kf = (float)orc_bf16(kb), vf = (float)orc_bf16(vb);
                    ((uint8_t *)k_pool)[off + d] = orc_e4m3fn_encode(kf / k_scale);
                    ((uint8_t *)v_pool)[off + d] = orc_e4m3fn_encode(vf / v_scale);
                }
            }
        }
    }
    return 0;
}

/*
 * Verify oracle: q [B][q_len][Hq][D] (bf16), seq_lens counting the q_len
 * query tokens themselves; out [B][q_len][Hq][D].  sinks, k_desc, v_desc,
 * alibi as for orc_decode.
 */
int orc_verify(int B, int Hq, int Hkv, int D, int P, int kv_dtype, int q_len,
               const uint16_t *q, const void *k_pool, const void *v_pool,
               int64_t num_pages, const int32_t *block_table, int64_t bt_stride,
               const int32_t *seq_lens, double scale, double softcap, int window,
               double k_scale, double v_scale, double *out, int threads,
               const float *sinks, const float *k_desc, const float *v_desc,
               const float *alibi)
{
    orc_problem pr;
    int64_t max_keys = 0;
    int b;
    if (check_common(B, Hq, Hkv, D, P, kv_dtype) || q_len < 1)
        return -1;
    memset(&pr, 0, sizeof pr);
    pr.B = B; pr.Hq = Hq; pr.Hkv = Hkv; pr.D = D; pr.Dv = D; pr.P = P;
    pr.kv_dtype = kv_dtype;
    pr.q = q; pr.k_pool = k_pool; pr.v_pool = v_pool;
    pr.num_pages = num_pages;
    pr.bt = block_table; pr.bt_stride = bt_stride; pr.seq_lens = seq_lens;
    pr.scale = scale; pr.softcap = softcap; pr.window = window;
    pr.k_scale = k_scale; pr.v_scale = v_scale;
    pr.sinks = sinks; pr.k_desc = k_desc; pr.v_desc = v_desc; pr.alibi = alibi;
    pr.q_len = q_len;
    pr.out = out;
    for (b = 0; b < B; ++b) {
        if (seq_lens[b] < 0)
            return -1;
        if (seq_lens[b] > max_keys)
            max_keys = seq_lens[b];
    }
    return run_jobs(&pr, 2, (int64_t)B * q_len * Hq, max_keys, threads);
}
