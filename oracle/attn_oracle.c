/*
 * attn_oracle.c -- plain, slow, fp64 CPU evaluation of scaled-dot-product
 * attention with its per-row log-sum-exp.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no code,
 * header, table or constant with the HIP path and is never on the product
 * path.
 *
 * What it computes (the definition the FlashAttention-2 forward reaches
 * exactly, up to rounding order):
 *   for every batch b, head h and query row i
 *     J_i  = { 0 .. N-1 }                     (non-causal)
 *          = { j : j <= i, j < N }            (causal, top-left aligned)
 *     s_j  = scale * sum_d q[i,d] * k[j,d]    for j in J_i
 *     m    = max_j s_j
 *     e_j  = exp(s_j - m)
 *     l    = sum_j e_j
 *     O[i] = (sum_j e_j * v[j,:]) / l
 *     L[i] = m + ln(l)                        (natural log)
 *
 * Sources on the pages:
 *   - "Extend Thunder with CUDA-Python", Python reference section
 *     (flash_attention_reference): the tiled form whose result this is when
 *     one tile spans all keys -- S = scale * Q K^T, the running max/sum, the
 *     final O / l and L = m + log(l); its causal mask keeps key index <= query
 *     index in absolute positions (top-left), masked scores are -inf.
 *   - the same page, "Running our kernel in Thunder" trace: SDPA decomposed as
 *     matmul -> amax / sub / exp / sum / div -> matmul with V.
 *   - "Blackwell Attention Example", attention kernel: lse is one fp32 value
 *     per query row of shape [B, H, M] (the oracle reports it in fp64).
 *
 * No blocking, fusion or reordering beyond the definition: each row is a
 * straight loop over its visible keys. Arithmetic is IEEE fp64 with libm exp
 * and log; build without -ffast-math.
 *
 * Layout: q, o are [B, H, M, D]; k, v are [B, H, N, D]; lse is [B, H, M];
 * all contiguous row-major fp64 host arrays owned by the caller.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

/* Number of keys row i may see: all N, or the top-left causal prefix. */
static int64_t visible_keys(int64_t i, int64_t N, int is_causal)
{
    if (!is_causal) return N;
    return (i + 1 < N) ? (i + 1) : N;
}

/*
 * One query row against the first n_vis rows of k / v.
 * s is caller scratch of at least n_vis doubles. Returns 0, or -1 if
 * n_vis < 1 (the definition needs at least one visible key).
 */
static int row_attention(const double *q, const double *k, const double *v,
                         int64_t n_vis, int64_t D, double scale, double *s,
                         double *o, double *lse)
{
    if (n_vis < 1) return -1;
    /* scores */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j) {
        const double *kj = k + j * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += q[d] * kj[d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    /* exponentials, their sum, and the weighted sum of values */
    double l = 0.0;
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        const double e = exp(s[j] - m);
        l += e;
        const double *vj = v + j * D;
        for (int64_t d = 0; d < D; ++d) o[d] += e * vj[d];
    }
    for (int64_t d = 0; d < D; ++d) o[d] = o[d] / l;
    *lse = m + log(l);
    return 0;
}

typedef struct {
    const double *q, *k, *v;
    double *o, *lse;
    int64_t H, M, N, D;
    double scale;
    int is_causal;
    const int64_t *rows;   /* NULL: every row; else flat row ids b*H*M + h*M + i */
    int64_t nrows;         /* number of rows to do */
    int64_t begin, end;    /* this worker's share of [0, nrows) */
    int status;
} work_t;

static void *worker(void *arg)
{
    work_t *w = (work_t *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)(w->N > 0 ? w->N : 1));
    if (!s) { w->status = -2; return NULL; }
    for (int64_t t = w->begin; t < w->end; ++t) {
        const int64_t r = w->rows ? w->rows[t] : t;   /* flat query row */
        const int64_t bh = r / w->M;                    /* b*H + h */
        const int64_t i = r % w->M;                     /* query index */
        const double *kh = w->k + bh * w->N * w->D;
        const double *vh = w->v + bh * w->N * w->D;
        /* outputs: full layout for the all-rows call, packed for a row list */
        double *o = w->o + (w->rows ? t : r) * w->D;
        double *lse = w->lse + (w->rows ? t : r);
        if (row_attention(w->q + r * w->D, kh, vh,
                          visible_keys(i, w->N, w->is_causal), w->D,
                          w->scale, s, o, lse) != 0) {
            w->status = -1;
            break;
        }
    }
    free(s);
    return NULL;
}

static int run(const double *q, const double *k, const double *v, double *o,
               double *lse, int64_t B, int64_t H, int64_t M, int64_t N,
               int64_t D, double scale, int is_causal, const int64_t *rows,
               int64_t nrows, int nthreads)
{
    if (B < 0 || H < 0 || M < 0 || N < 1 || D < 1) return -1;
    if (is_causal != 0 && is_causal != 1) return -1;
    if (nrows == 0) return 0;
    if (rows) {
        for (int64_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= B * H * M) return -1;
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = (int)nrows;

    work_t w[256];
    pthread_t th[256];
    const int64_t chunk = (nrows + nthreads - 1) / nthreads;
    nthreads = (int)((nrows + chunk - 1) / chunk);   /* every worker non-empty */
    for (int t = 0; t < nthreads; ++t) {
        const int64_t end = (t + 1) * chunk < nrows ? (t + 1) * chunk : nrows;
        w[t] = (work_t){q, k, v, o, lse, H, M, N, D, scale, is_causal, rows,
                        nrows, t * chunk, end, 0};
    }
    int started = 0;   /* workers 1..started run on their own threads */
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &w[t]) != 0) break;
        started = t;
    }
    /* worker 0, and any worker whose thread could not start, run here */
    worker(&w[0]);
    for (int t = started + 1; t < nthreads; ++t) worker(&w[t]);
    int status = 0;
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (w[t].status) status = w[t].status;
    return status;
}

/*
 * Every row: o [B,H,M,D], lse [B,H,M]. Returns 0 on success, -1 on bad
 * arguments (negative sizes, N < 1, is_causal not 0/1), -2 if a worker could
 * not be started or allocate its scratch.
 */
int oracle_attn_fwd(const double *q, const double *k, const double *v,
                    double *o, double *lse, int64_t B, int64_t H, int64_t M,
                    int64_t N, int64_t D, double scale, int is_causal,
                    int nthreads)
{
    return run(q, k, v, o, lse, B, H, M, N, D, scale, is_causal, NULL,
               B * H * M, nthreads);
}

/*
 * Listed rows only: rows[t] is the flat query row b*H*M + h*M + i; row t's
 * output goes to o[t*D .. t*D+D) and lse[t]. Same return codes; a row id out
 * of range is -1.
 */
int oracle_attn_rows(const double *q, const double *k, const double *v,
                     double *o, double *lse, int64_t B, int64_t H, int64_t M,
                     int64_t N, int64_t D, double scale, int is_causal,
                     const int64_t *rows, int64_t nrows, int nthreads)
{
    if (nrows < 0 || (nrows > 0 && !rows)) return -1;
    return run(q, k, v, o, lse, B, H, M, N, D, scale, is_causal, rows, nrows,
               nthreads);
}
