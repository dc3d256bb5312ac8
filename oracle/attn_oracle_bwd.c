/*
 * attn_oracle_bwd.c -- plain, slow, fp64 CPU evaluation of the gradient of
 * scaled-dot-product attention with respect to its inputs.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no code,
 * header, table or constant with the HIP path and is never on the product
 * path.
 *
 * What it computes. For every batch b, head h, with J_i the keys query i may
 * see (all N, or j <= i under the top-left causal mask), the forward is
 *     s_ij = scale * <q_i, k_j>,  P_ij = exp(s_ij - L_i),  L_i = ln sum_j exp(s_ij)
 *     O_i  = sum_j P_ij v_j
 * and, for an upstream gradient dO, the chain rule through the product, the
 * softmax and the scaled dot product gives
 *     dV_j  = sum_i P_ij dO_i
 *     dP_ij = <dO_i, v_j>
 *     dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)     (softmax Jacobian:
 *                                                  dP_ij/ds_ik = P_ij (1[j=k] - P_ik))
 *     dQ_i  = scale * sum_j dS_ij k_j
 *     dK_j  = scale * sum_i dS_ij q_i
 * with P_ij = dS_ij = 0 for masked pairs. This is the quantity that the
 * backward kernel of "Blackwell Attention Example" (backward kernel
 * implementation and autograd function sections) evaluates tile by tile; that
 * kernel takes the row term sum_k P_ik dP_ik as rowsum(O * dO), which equals it
 * exactly. The oracle keeps the Jacobian form as written above.
 *
 * No blocking, fusion or reordering beyond the definition: per head, a pass
 * over query rows forms the rows of P, dP and dS and dQ; a pass over key rows
 * forms dK and dV. Arithmetic is IEEE fp64 with libm exp and log; build
 * without -ffast-math.
 *
 * Layout: q, dO, dQ are [B, H, M, D]; k, v, dK, dV are [B, H, N, D]; all
 * contiguous row-major fp64 host arrays owned by the caller.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

static int64_t n_visible(int64_t i, int64_t N, int is_causal)
{
    if (!is_causal) return N;
    return (i + 1 < N) ? (i + 1) : N;
}

typedef struct {
    const double *q, *k, *v, *dout;
    double *dq, *dk, *dv;
    double *P, *dS;          /* this head's M x N rows (zero where masked) */
    int64_t M, N, D;
    double scale;
    int is_causal;
    int64_t begin, end;      /* this worker's share of rows */
    int status;
} head_work_t;

/* Query rows [begin, end): P, dS rows and dQ. */
static void *query_rows(void *arg)
{
    head_work_t *w = (head_work_t *)arg;
    const int64_t N = w->N, D = w->D;
    double *dP = (double *)malloc(sizeof(double) * (size_t)N);
    if (!dP) { w->status = -2; return NULL; }
    for (int64_t i = w->begin; i < w->end; ++i) {
        const int64_t nv = n_visible(i, N, w->is_causal);
        const double *qi = w->q + i * D;
        const double *gi = w->dout + i * D;
        double *Pi = w->P + i * N;
        double *dSi = w->dS + i * N;
        /* scores and their log-sum-exp */
        double m = -INFINITY;
        for (int64_t j = 0; j < nv; ++j) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += qi[d] * w->k[j * D + d];
            Pi[j] = w->scale * dot;
            if (Pi[j] > m) m = Pi[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < nv; ++j) l += exp(Pi[j] - m);
        const double L = m + log(l);
        /* probabilities, dP = dO v^T, and the row term sum_k P_ik dP_ik */
        double row = 0.0;
        for (int64_t j = 0; j < nv; ++j) {
            Pi[j] = exp(Pi[j] - L);
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += gi[d] * w->v[j * D + d];
            dP[j] = dot;
            row += Pi[j] * dP[j];
        }
        for (int64_t j = nv; j < N; ++j) { Pi[j] = 0.0; dSi[j] = 0.0; }
        for (int64_t j = 0; j < nv; ++j) dSi[j] = Pi[j] * (dP[j] - row);
        /* dQ_i = scale * sum_j dS_ij k_j */
        double *dqi = w->dq + i * D;
        for (int64_t d = 0; d < D; ++d) dqi[d] = 0.0;
        for (int64_t j = 0; j < nv; ++j)
            for (int64_t d = 0; d < D; ++d) dqi[d] += dSi[j] * w->k[j * D + d];
        for (int64_t d = 0; d < D; ++d) dqi[d] *= w->scale;
    }
    free(dP);
    return NULL;
}

/* Key rows [begin, end): dK and dV from the columns of dS and P. */
static void *key_rows(void *arg)
{
    head_work_t *w = (head_work_t *)arg;
    const int64_t M = w->M, N = w->N, D = w->D;
    for (int64_t j = w->begin; j < w->end; ++j) {
        double *dkj = w->dk + j * D;
        double *dvj = w->dv + j * D;
        for (int64_t d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; }
        for (int64_t i = 0; i < M; ++i) {
            const double p = w->P[i * N + j];
            const double ds = w->dS[i * N + j];
            for (int64_t d = 0; d < D; ++d) {
                dvj[d] += p * w->dout[i * D + d];
                dkj[d] += ds * w->q[i * D + d];
            }
        }
        for (int64_t d = 0; d < D; ++d) dkj[d] *= w->scale;
    }
    return NULL;
}

/* Run fn over [0, n) split across up to nthreads workers (template in w0). */
static int parallel_rows(void *(*fn)(void *), const head_work_t *w0, int64_t n,
                         int nthreads)
{
    if (n == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)n;
    head_work_t w[256];
    pthread_t th[256];
    const int64_t chunk = (n + nthreads - 1) / nthreads;
    nthreads = (int)((n + chunk - 1) / chunk);
    for (int t = 0; t < nthreads; ++t) {
        w[t] = *w0;
        w[t].begin = t * chunk;
        w[t].end = (t + 1) * chunk < n ? (t + 1) * chunk : n;
        w[t].status = 0;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, fn, &w[t]) != 0) break;
        started = t;
    }
    fn(&w[0]);
    for (int t = started + 1; t < nthreads; ++t) fn(&w[t]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    int status = 0;
    for (int t = 0; t < nthreads; ++t)
        if (w[t].status) status = w[t].status;
    return status;
}

/*
 * dQ [B,H,M,D], dK, dV [B,H,N,D] for upstream gradient dout [B,H,M,D].
 * Returns 0, -1 on bad arguments (negative sizes, N < 1 while M > 0,
 * D < 1, is_causal not 0/1), -2 if scratch could not be allocated.
 * With M == 0 the key gradients are zero.
 */
int oracle_attn_bwd(const double *q, const double *k, const double *v,
                    const double *dout, double *dq, double *dk, double *dv,
                    int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                    double scale, int is_causal, int nthreads)
{
    if (B < 0 || H < 0 || M < 0 || N < 0 || D < 1) return -1;
    if (M > 0 && N < 1) return -1;
    if (is_causal != 0 && is_causal != 1) return -1;
    if (B * H == 0) return 0;
    double *P = (double *)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
    double *dS = (double *)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
    if (!P || !dS) { free(P); free(dS); return -2; }
    int status = 0;
    for (int64_t bh = 0; bh < B * H && status == 0; ++bh) {
        head_work_t w = {q + bh * M * D, k + bh * N * D, v + bh * N * D,
                         dout + bh * M * D, dq + bh * M * D, dk + bh * N * D,
                         dv + bh * N * D, P, dS, M, N, D, scale, is_causal,
                         0, 0, 0};
        status = parallel_rows(query_rows, &w, M, nthreads);
        if (status == 0) status = parallel_rows(key_rows, &w, N, nthreads);
    }
    free(P);
    free(dS);
    return status;
}
