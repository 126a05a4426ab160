/*
 * fp64 CPU oracle for multi-head latent attention (MLA) decode, with one or
 * several query tokens per sequence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the HIP library and is deliberately plain and slow:
 * scalar loops in double precision, no blocking, no fusion, no fast-math.
 *
 * What it computes (the plain definition of attention decode over the
 * dequantised latent cache).  For sequence b and query head h:
 *
 *   c_t   = dequant(stored row of token t)            (576 values, fp64)
 *   z_t   = sm_scale * sum_{d<576} q[b,h,d] * c_t[d]
 *   m     = max_t z_t ;  w_t = exp(z_t - m) ;  Z = sum_t w_t
 *   out[b,h,d] = sum_t w_t * c_t[d] / Z               (d < 512)
 *   lse[b,h]   = m + log(Z)
 *
 * Sources (amd-mixed-mla leaderboard submissions for MI355X):
 *   - the score/softmax/value formula and V = first 512 cache columns:
 *     submission 599694 ("overhead elimination"), function `_bmm` (the torch
 *     bmm path) and the fp8 flash-decode kernel `_flash_fp8_single`;
 *   - scale 1/sqrt(576): submission 727205 ("v25: LEAN"), module constants;
 *   - fp8 dequantisation = code value x per-tensor scale: 599694,
 *     `_flash_fp8_single` (fp8 load times kv_scale);
 *   - MXFP4 rows, low nibble = even element, one e8m0 scale per 32 elements:
 *     submission 700955 ("locked baseline dispatch"), kernels `mla_attn_v71`
 *     and `mla_attn_v74` (their fp4 unpacking loops).
 *   - an empty sequence gives a zero output: 700955 `mla_attn_v71` (empty split
 *     writes zeros) and 599694 `_flash_fp8_split_s2` (it skips empty splits).
 * Where the pages leave a step open the oracle takes the plainest reading:
 *   - e4m3 is the OCP "fn" variant (bias 7, subnormals, max 448, S.1111.111 is
 *     NaN, no infinities);
 *   - e8m0 decodes to 2^(e-127), with 255 = NaN;
 *   - e2m1 is the OCP MX element type: 1 sign, 2 exponent (bias 1), 1 mantissa
 *     bit, exponent 0 subnormal;
 *   - page tables: kv_indptr counts pages, the last page holds
 *     kv_last_page_len tokens (page_size 1: kv_indptr counts tokens).
 *
 * Multi-token decode (oracle_mla_decode_multi): sequence b has q_b query
 * tokens, rows qo_indptr[b] .. qo_indptr[b+1]-1 of q and out.  Query token j is
 * the token at position n_b - q_b + j of its sequence (the cache holds the
 * rows of all its query tokens) and attends causally: every cache token gets
 * a score, and the tokens after position n_b - q_b + j are masked out of the
 * maximum and the sum.  The submissions pass qo_indptr = 0, 1, .., bs with a
 * maximum query length of 1 to aiter (599694 "overhead elimination", its
 * aiter path; 727205 "v25: LEAN", its metadata call); the causal placement of
 * longer query runs is the plainest reading of that argument.
 *
 * The low-precision query (oracle_round_query_e4m3) is a pre-processing of q
 * for the exact decode: submission 599694 ("overhead elimination") quantises
 * the query to fp8 e4m3 under a scale (the static query scale of its fast
 * path) before its aiter call.  Here the scale is the power of two 2^s per
 * (row, head) that puts the head's largest |q| in [128, 256) -- the reading
 * of "a scale" that needs no assumption about the query's range -- and
 * q * 2^s is rounded to the nearest e4m3 value, ties to even, then scaled
 * back.  The decode of the rounded query is the definition of that mode.
 *
 * The optional split mode computes, for a caller-given partition of each
 * sequence into token ranges, every range's exact (normalised output, lse) and
 * then merges them by lse weights: M = max_s lse_s, w_s = exp(lse_s - M),
 * out = sum_s w_s O_s / sum_s w_s (submission 599694, `_flash_fp8_split_s2`;
 * 700955, `reduce_lse_v71`).  Mathematically it equals the unsplit result.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_BF16 = 0, OR_FP8 = 1, OR_MXFP4 = 2 };

/* ---- element decoders, from the bit fields ------------------------------ */

double oracle_bf16_to_f64(uint16_t bits) {
    /* bf16 is the top half of an IEEE binary32 */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_e4m3_to_f64(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, 1 - 7);           /* subnormal: 0.m * 2^(1-bias) */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);     /* normal: 1.m * 2^(e-bias) */
    return s ? -v : v;
}

double oracle_e8m0_to_f64(uint8_t code) {
    if (code == 0xFF) return NAN;
    return ldexp(1.0, (int)code - 127);
}

double oracle_e2m1_to_f64(uint8_t nibble) {
    int s = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 0x3;
    int m = nibble & 0x1;
    double v;
    if (e == 0)
        v = ldexp((double)m / 2.0, 1 - 1);           /* subnormal: 0.m * 2^(1-bias) */
    else
        v = ldexp(1.0 + (double)m / 2.0, e - 1);
    return s ? -v : v;
}

/* ---- cache access -------------------------------------------------------- */

typedef struct {
    int fmt;
    int qk_dim;
    const uint8_t* kv;         /* row-major stored rows */
    const uint8_t* scales;     /* MXFP4: [rows, scale_stride] e8m0 */
    int64_t scale_stride;
    double kv_scale;           /* fp8 per-tensor scale */
} cache_t;

static int64_t row_bytes(const cache_t* c) {
    if (c->fmt == OR_BF16) return 2 * (int64_t)c->qk_dim;
    if (c->fmt == OR_FP8) return c->qk_dim;
    return c->qk_dim / 2;
}

/* Dequantise one stored row into out[qk_dim]. */
static void dequant_row(const cache_t* c, int64_t row, double* out) {
    const uint8_t* r = c->kv + row * row_bytes(c);
    int d;
    if (c->fmt == OR_BF16) {
        for (d = 0; d < c->qk_dim; ++d) {
            uint16_t bits = (uint16_t)(r[2 * d] | ((uint16_t)r[2 * d + 1] << 8));
            out[d] = oracle_bf16_to_f64(bits);
        }
    } else if (c->fmt == OR_FP8) {
        for (d = 0; d < c->qk_dim; ++d) out[d] = oracle_e4m3_to_f64(r[d]) * c->kv_scale;
    } else {
        const uint8_t* sc = c->scales + row * c->scale_stride;
        for (d = 0; d < c->qk_dim; ++d) {
            uint8_t byte = r[d / 2];
            uint8_t nib = (d % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            out[d] = oracle_e2m1_to_f64(nib) * oracle_e8m0_to_f64(sc[d / 32]);
        }
    }
}

/* ---- the low-precision query --------------------------------------------- */

/* Nearest e4m3 value to x, ties to the even code: 4 significant bits with the
 * leading bit at 2^e, e >= -6 (steps of 2^-9 below 2^-6).  |x| < 448 here. */
static double round_e4m3(double x) {
    double a = fabs(x), r;
    int e;
    if (a == 0.0) return x;
    frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1): leading bit 2^(e-1) */
    e = e - 1;
    if (e < -6) e = -6;
    r = nearbyint(ldexp(a, 3 - e));   /* in units of 2^(e-3); the default mode rounds ties to even */
    r = ldexp(r, e - 3);
    return copysign(r, x);
}

/* q [rows, nh, qk_dim] bf16 bit patterns -> out, the same shape: each element
 * rounded to one e4m3 code under the per-(row, head) scale 2^s, s = 8 - e for
 * the head's largest |q| = f * 2^e, f in [0.5, 1) (s = 0 for a zero head).
 * The result is exact in bf16.  Returns 0, or -1 for a non-finite query
 * element, -2 if a result would not be a bf16 value. */
int oracle_round_query_e4m3(const uint16_t* q, int64_t rows, int nh, int qk_dim, uint16_t* out) {
    int64_t r;
    int h, d;
    for (r = 0; r < rows; ++r)
        for (h = 0; h < nh; ++h) {
            const uint16_t* qh = q + (r * nh + h) * qk_dim;
            uint16_t* oh = out + (r * nh + h) * qk_dim;
            double amax = 0.0;
            int s = 0, e;
            for (d = 0; d < qk_dim; ++d) {
                double v = fabs(oracle_bf16_to_f64(qh[d]));
                if (!isfinite(v)) return -1;
                if (v > amax) amax = v;
            }
            if (amax > 0.0) {
                frexp(amax, &e);
                s = 8 - e;
            }
            for (d = 0; d < qk_dim; ++d) {
                double y = ldexp(round_e4m3(ldexp(oracle_bf16_to_f64(qh[d]), s)), -s);
                float f = (float)y;
                uint32_t u;
                if ((double)f != y) return -2;
                memcpy(&u, &f, sizeof u);
                if (u & 0xFFFFu) return -2;
                oh[d] = (uint16_t)(u >> 16);
            }
        }
    return 0;
}

int oracle_dequant_rows(int fmt, int qk_dim, const uint8_t* kv, const uint8_t* scales,
                        int64_t scale_stride, double kv_scale, const int64_t* rows,
                        int64_t n, double* out) {
    cache_t c = {fmt, qk_dim, kv, scales, scale_stride, kv_scale};
    int64_t i;
    if (fmt < 0 || fmt > 2) return 1;
    for (i = 0; i < n; ++i) dequant_row(&c, rows[i], out + i * qk_dim);
    return 0;
}

/* ---- problem description ------------------------------------------------- */

typedef struct {
    const uint16_t* q;          /* bf16 bits [bs, nh, qk_dim] */
    int bs, nh, qk_dim, v_dim;
    double sm_scale;
    cache_t cache;
    const int32_t* kv_indptr;   /* [bs+1] tokens (page_size 1) or pages */
    const int32_t* page_indices;
    const int32_t* last_page_len;
    int page_size;
    const int32_t* qo_indptr;     /* optional [bs+1]: multi-token rows (see above) */
    const int32_t* split_indptr;  /* optional [bs+1] into split_bounds */
    const int32_t* split_bounds;  /* per split: end token (exclusive) within the sequence */
    double* out;                /* [bs, nh, v_dim] */
    double* lse;                /* [bs, nh] or NULL */
} problem_t;

static int64_t seq_len(const problem_t* p, int b) {
    int64_t n = (int64_t)p->kv_indptr[b + 1] - p->kv_indptr[b];
    if (p->page_size == 1) return n;
    if (n <= 0) return 0;
    return (n - 1) * p->page_size + p->last_page_len[b];
}

static int64_t token_row(const problem_t* p, int b, int64_t j) {
    if (p->page_size == 1) return (int64_t)p->kv_indptr[b] + j;
    {
        int64_t page = p->page_indices[(int64_t)p->kv_indptr[b] + j / p->page_size];
        return page * p->page_size + j % p->page_size;
    }
}

/* Exact attention of head h over tokens [t0, t1) of an already-dequantised
 * sequence c[len][qk_dim]: writes o[v_dim] (normalised) and returns the lse.
 * An empty range returns -inf and a zero output. */
static double attend_range(const problem_t* p, int b, int h, const double* c,
                           int64_t t0, int64_t t1, double* z, double* o) {
    const uint16_t* qh = p->q + ((int64_t)b * p->nh + h) * p->qk_dim;
    int64_t t;
    int d;
    double m = -INFINITY, Z = 0.0;
    for (d = 0; d < p->v_dim; ++d) o[d] = 0.0;
    if (t1 <= t0) return -INFINITY;
    for (t = t0; t < t1; ++t) {
        const double* ct = c + t * p->qk_dim;
        double s = 0.0;
        for (d = 0; d < p->qk_dim; ++d) s += oracle_bf16_to_f64(qh[d]) * ct[d];
        z[t] = p->sm_scale * s;
        if (z[t] > m) m = z[t];
    }
    for (t = t0; t < t1; ++t) {
        const double* ct = c + t * p->qk_dim;
        double w = exp(z[t] - m);
        Z += w;
        for (d = 0; d < p->v_dim; ++d) o[d] += w * ct[d];
    }
    for (d = 0; d < p->v_dim; ++d) o[d] /= Z;
    return m + log(Z);
}

/* Multi-token decode of sequence b: the causal definition written out. */
static void solve_sequence_multi(const problem_t* p, int b, const double* c, double* z) {
    int64_t n = seq_len(p, b), t;
    int q = p->qo_indptr[b + 1] - p->qo_indptr[b], j, h, d;
    for (j = 0; j < q; ++j) {
        int64_t row = (int64_t)p->qo_indptr[b] + j;
        int64_t pos = n - q + j; /* this query token's position */
        for (h = 0; h < p->nh; ++h) {
            const uint16_t* qh = p->q + (row * p->nh + h) * p->qk_dim;
            double* o = p->out + (row * p->nh + h) * p->v_dim;
            double m = -INFINITY, Z = 0.0;
            for (t = 0; t < n; ++t) {
                const double* ct = c + t * p->qk_dim;
                double s = 0.0;
                for (d = 0; d < p->qk_dim; ++d) s += oracle_bf16_to_f64(qh[d]) * ct[d];
                z[t] = p->sm_scale * s;
            }
            for (t = 0; t < n; ++t)
                if (t <= pos && z[t] > m) m = z[t]; /* causal mask */
            for (d = 0; d < p->v_dim; ++d) o[d] = 0.0;
            for (t = 0; t < n; ++t) {
                const double* ct = c + t * p->qk_dim;
                double w = t <= pos ? exp(z[t] - m) : 0.0; /* causal mask */
                Z += w;
                for (d = 0; d < p->v_dim; ++d) o[d] += w * ct[d];
            }
            for (d = 0; d < p->v_dim; ++d) o[d] /= Z;
            if (p->lse) p->lse[row * p->nh + h] = m + log(Z);
        }
    }
}

static void solve_sequence(const problem_t* p, int b, double* cbuf, double* z, double* tmp) {
    int64_t n = seq_len(p, b), j;
    int h, d;
    for (j = 0; j < n; ++j) dequant_row(&p->cache, token_row(p, b, j), cbuf + j * p->qk_dim);
    if (p->qo_indptr) {
        solve_sequence_multi(p, b, cbuf, z);
        return;
    }
    for (h = 0; h < p->nh; ++h) {
        double* o = p->out + ((int64_t)b * p->nh + h) * p->v_dim;
        double lse;
        if (n == 0) {
            for (d = 0; d < p->v_dim; ++d) o[d] = 0.0;
            lse = -INFINITY;
        } else if (!p->split_indptr) {
            lse = attend_range(p, b, h, cbuf, 0, n, z, o);
        } else {
            /* split mode: exact per-range results, merged by their lse */
            int s, s0 = p->split_indptr[b], s1 = p->split_indptr[b + 1];
            double M = -INFINITY, W = 0.0;
            int64_t start;
            start = 0;
            for (s = s0; s < s1; ++s) {
                double l = attend_range(p, b, h, cbuf, start, p->split_bounds[s], z, tmp);
                if (l > M) M = l;
                start = p->split_bounds[s];
            }
            for (d = 0; d < p->v_dim; ++d) o[d] = 0.0;
            start = 0;
            for (s = s0; s < s1; ++s) {
                double l = attend_range(p, b, h, cbuf, start, p->split_bounds[s], z, tmp);
                double w = (l == -INFINITY) ? 0.0 : exp(l - M);
                W += w;
                for (d = 0; d < p->v_dim; ++d) o[d] += w * tmp[d];
                start = p->split_bounds[s];
            }
            for (d = 0; d < p->v_dim; ++d) o[d] /= W;
            lse = M + log(W);
        }
        if (p->lse) p->lse[(int64_t)b * p->nh + h] = lse;
    }
}

typedef struct {
    const problem_t* p;
    const int32_t* batches;
    int n_batches;
    int next;
    pthread_mutex_t mu;
    int64_t max_len;
    int failed;
} pool_t;

static void* worker(void* arg) {
    pool_t* pool = (pool_t*)arg;
    const problem_t* p = pool->p;
    int64_t cap = pool->max_len > 0 ? pool->max_len : 1;
    double* cbuf = (double*)malloc((size_t)cap * p->qk_dim * sizeof(double));
    double* z = (double*)malloc((size_t)cap * sizeof(double));
    double* tmp = (double*)malloc((size_t)p->v_dim * sizeof(double));
    if (!cbuf || !z || !tmp) {
        pthread_mutex_lock(&pool->mu);
        pool->failed = 1;
        pthread_mutex_unlock(&pool->mu);
    } else {
        for (;;) {
            int i;
            pthread_mutex_lock(&pool->mu);
            i = pool->next++;
            pthread_mutex_unlock(&pool->mu);
            if (i >= pool->n_batches) break;
            solve_sequence(p, pool->batches[i], cbuf, z, tmp);
        }
    }
    free(cbuf);
    free(z);
    free(tmp);
    return NULL;
}

/* Full decode, single-token (qo_indptr NULL) or multi-token; see the two
 * exported entry points below. */
static int decode(const uint16_t* q, int bs, int nh, int qk_dim, int v_dim, double sm_scale, int fmt,
                  const uint8_t* kv, double kv_scale, const uint8_t* scales, int64_t scale_stride,
                  const int32_t* kv_indptr, const int32_t* page_indices, const int32_t* last_page_len,
                  int page_size, const int32_t* qo_indptr, const int32_t* split_indptr,
                  const int32_t* split_bounds, const int32_t* batches, int n_batches, int nthreads,
                  double* out, double* lse) {
    problem_t p;
    pool_t pool;
    pthread_t* th;
    int32_t* all = NULL;
    int i, b;
    if (!q || !kv || !kv_indptr || !out || bs < 0 || nh <= 0 || qk_dim <= 0 || v_dim <= 0 ||
        v_dim > qk_dim || fmt < 0 || fmt > 2 || page_size < 1)
        return 1;
    if (fmt == OR_MXFP4 && (!scales || qk_dim % 32 || scale_stride < qk_dim / 32)) return 1;
    if (page_size > 1 && (!page_indices || !last_page_len)) return 1;
    p.q = q; p.bs = bs; p.nh = nh; p.qk_dim = qk_dim; p.v_dim = v_dim; p.sm_scale = sm_scale;
    p.cache.fmt = fmt; p.cache.qk_dim = qk_dim; p.cache.kv = kv; p.cache.scales = scales;
    p.cache.scale_stride = scale_stride; p.cache.kv_scale = kv_scale;
    p.kv_indptr = kv_indptr; p.page_indices = page_indices; p.last_page_len = last_page_len;
    p.page_size = page_size; p.split_indptr = split_indptr; p.split_bounds = split_bounds;
    p.qo_indptr = qo_indptr;
    if (qo_indptr && split_indptr) return 1;
    p.out = out; p.lse = lse;

    if (!batches) {
        all = (int32_t*)malloc((size_t)(bs > 0 ? bs : 1) * sizeof(int32_t));
        if (!all) return 2;
        for (b = 0; b < bs; ++b) all[b] = b;
        batches = all;
        n_batches = bs;
    }
    pool.p = &p; pool.batches = batches; pool.n_batches = n_batches; pool.next = 0;
    pool.max_len = 0; pool.failed = 0;
    for (i = 0; i < n_batches; ++i) {
        int64_t n;
        if (batches[i] < 0 || batches[i] >= bs) { free(all); return 1; }
        n = seq_len(&p, batches[i]);
        if (n < 0) { free(all); return 1; }
        if (qo_indptr) {
            int qn = qo_indptr[batches[i] + 1] - qo_indptr[batches[i]];
            if (qn < 0 || qn > n) { free(all); return 1; }
        }
        if (n > pool.max_len) pool.max_len = n;
    }
    pthread_mutex_init(&pool.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n_batches) nthreads = n_batches > 0 ? n_batches : 1;
    th = (pthread_t*)malloc((size_t)nthreads * sizeof(pthread_t));
    if (!th) { free(all); return 2; }
    for (i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &pool);
    for (i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&pool.mu);
    free(th);
    free(all);
    return pool.failed ? 2 : 0;
}

/*
 * Single-token decode: row b of q and out is sequence b.  Returns 0 on
 * success, nonzero on bad arguments or allocation failure.  `batches`
 * (optional, n_batches entries) restricts the work to the listed sequences;
 * the other rows of `out`/`lse` are left untouched.  `split_indptr` /
 * `split_bounds` (optional) switch on split mode.
 */
int oracle_mla_decode(const uint16_t* q, int bs, int nh, int qk_dim, int v_dim, double sm_scale,
                      int fmt, const uint8_t* kv, double kv_scale, const uint8_t* scales,
                      int64_t scale_stride, const int32_t* kv_indptr, const int32_t* page_indices,
                      const int32_t* last_page_len, int page_size, const int32_t* split_indptr,
                      const int32_t* split_bounds, const int32_t* batches, int n_batches,
                      int nthreads, double* out, double* lse) {
    return decode(q, bs, nh, qk_dim, v_dim, sm_scale, fmt, kv, kv_scale, scales, scale_stride, kv_indptr,
                  page_indices, last_page_len, page_size, NULL, split_indptr, split_bounds, batches, n_batches,
                  nthreads, out, lse);
}

/*
 * Multi-token decode (see the header): q and out have qo_indptr[bs] rows;
 * `batches` lists sequences, all of whose rows are computed.  No split mode.
 */
int oracle_mla_decode_multi(const uint16_t* q, int bs, int nh, int qk_dim, int v_dim, double sm_scale,
                            int fmt, const uint8_t* kv, double kv_scale, const uint8_t* scales,
                            int64_t scale_stride, const int32_t* kv_indptr, const int32_t* page_indices,
                            const int32_t* last_page_len, int page_size, const int32_t* qo_indptr,
                            const int32_t* batches, int n_batches, int nthreads, double* out, double* lse) {
    if (!qo_indptr || qo_indptr[0] != 0) return 1;
    return decode(q, bs, nh, qk_dim, v_dim, sm_scale, fmt, kv, kv_scale, scales, scale_stride, kv_indptr,
                  page_indices, last_page_len, page_size, qo_indptr, NULL, NULL, batches, n_batches, nthreads,
                  out, lse);
}
