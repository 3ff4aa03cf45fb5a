/*
 * ssd_oracle.c -- fp64 CPU reference for the Mamba-2 SSD forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU path is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it; the product library never links or calls it, and
 * it shares no code, header or table with the HIP kernels.
 *
 * What it computes (source: "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核",
 * dbyun.net, section "Mamba-2 架构", the core recurrence):
 *
 *     h_t = exp(A * dt_t) * h_{t-1} + dt_t * x_t (outer) B_t      state h is [P, N]
 *     y_t = h_t . C_t + D * x_t                                    y_t is [P]
 *
 * run token by token, in double precision, separately for every (batch, head)
 * pair.  Heads map to B/C groups in contiguous blocks, g = h / (H / G) (same
 * page, section "Kernel 2: fwd_pass_state", the head->group mapping).  The
 * output at token t uses the state *after* token t's update (the output
 * equation pairs y_t with h_t; the simplified restatement on the same page that
 * writes h_{t-1} is read as a typo, because the causal mask of the chunked form
 * keeps the diagonal i == j).
 *
 * Chunk-start snapshots: when `chunk` > 0 the state *before* tokens
 * 0, chunk, 2*chunk, ... is recorded (the per-chunk initial hidden state that
 * the "fwd_pass_state" kernel stores), the first one being h0.
 *
 * ssd_oracle_chunk_cumsum() is the plain definition of the first kernel's
 * output (section "Kernel 1：计算累积和"): within each chunk, the inclusive
 * running sum of A[h] * dt[b,t,h], multiplied by log2(e).
 *
 * Inputs are read in their stored type (fp64, fp32 or bf16 bit patterns) and
 * widened exactly to double; no arithmetic happens in lower precision.
 * Compile with -O2 and without -ffast-math; exp() is libm's.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

static double load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORC_F64) return ((const double *)base)[i];
    if (dtype == ORC_F32) return (double)((const float *)base)[i];
    /* bf16: the upper 16 bits of an IEEE binary32; widening is exact. */
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    int64_t batch, seqlen, nheads, ngroups, headdim, dstate;
    int dtype;
    const void *x, *dt, *B, *C;
    const double *A, *D, *h0;
    const int64_t *units;
    int64_t n_units;
    int64_t chunk;
    double *y, *hT, *snaps;
    int64_t next;               /* next unit index to claim */
    pthread_mutex_t lock;
} oracle_job;

/* One (batch, head) pair, sequential over tokens. */
static void run_unit(const oracle_job *jb, int64_t ui, double *S, double *xrow, double *brow,
                     double *crow)
{
    const int64_t L = jb->seqlen, H = jb->nheads, G = jb->ngroups;
    const int64_t P = jb->headdim, N = jb->dstate;
    const int64_t u = jb->units ? jb->units[ui] : ui;
    const int64_t b = u / H, h = u % H;
    const int64_t g = h / (H / G);
    const double A = jb->A[h], Dh = jb->D[h];
    const int64_t nc = jb->chunk > 0 ? (L + jb->chunk - 1) / jb->chunk : 0;

    if (jb->h0) memcpy(S, jb->h0 + (b * H + h) * P * N, (size_t)(P * N) * sizeof(double));
    else memset(S, 0, (size_t)(P * N) * sizeof(double));

    for (int64_t t = 0; t < L; ++t) {
        if (jb->chunk > 0 && t % jb->chunk == 0 && jb->snaps)
            memcpy(jb->snaps + (ui * nc + t / jb->chunk) * P * N, S, (size_t)(P * N) * sizeof(double));

        const double dt = load_elem(jb->dt, jb->dtype, (b * L + t) * H + h);
        const double decay = exp(A * dt);
        const int64_t xoff = ((b * L + t) * H + h) * P;
        const int64_t boff = ((b * L + t) * G + g) * N;
        for (int64_t p = 0; p < P; ++p) xrow[p] = load_elem(jb->x, jb->dtype, xoff + p);
        for (int64_t n = 0; n < N; ++n) brow[n] = load_elem(jb->B, jb->dtype, boff + n);
        for (int64_t n = 0; n < N; ++n) crow[n] = load_elem(jb->C, jb->dtype, boff + n);

        /* state update: h <- exp(A dt) h + dt * x (outer) B */
        for (int64_t p = 0; p < P; ++p) {
            const double coef = dt * xrow[p];
            double *Sp = S + p * N;
            for (int64_t n = 0; n < N; ++n)
                Sp[n] = decay * Sp[n] + coef * brow[n];
        }
        /* output: y = h . C + D x */
        if (jb->y) {
            double *yrow = jb->y + (ui * L + t) * P;
            for (int64_t p = 0; p < P; ++p) {
                const double *Sp = S + p * N;
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += Sp[n] * crow[n];
                yrow[p] = acc + Dh * xrow[p];
            }
        }
    }
    if (jb->hT) memcpy(jb->hT + ui * P * N, S, (size_t)(P * N) * sizeof(double));
}

static void *worker(void *arg)
{
    oracle_job *jb = (oracle_job *)arg;
    double *S = (double *)malloc((size_t)(jb->headdim * jb->dstate) * sizeof(double));
    double *xrow = (double *)malloc((size_t)jb->headdim * sizeof(double));
    double *brow = (double *)malloc((size_t)jb->dstate * sizeof(double));
    double *crow = (double *)malloc((size_t)jb->dstate * sizeof(double));
    if (!S || !xrow || !brow || !crow) {
        free(S); free(xrow); free(brow); free(crow);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        int64_t ui = jb->next++;
        pthread_mutex_unlock(&jb->lock);
        if (ui >= jb->n_units) break;
        run_unit(jb, ui, S, xrow, brow, crow);
    }
    free(S);
    free(xrow);
    free(brow);
    free(crow);
    return NULL;
}

/*
 * Runs the recurrence for the listed units.
 *   x [b,L,H,P], dt [b,L,H], B and C [b,L,G,N] in `dtype`; A, D [H] and
 *   h0 [b,H,P,N] (NULL = zero) as double.
 *   units: flat ids b*H + h (NULL = all b*H units in order); n_units entries.
 *   y [n_units, L, P], hT [n_units, P, N], snaps [n_units, ceil(L/chunk), P, N];
 *   any of them may be NULL.  Returns 0, or a negative code for bad arguments.
 */
int ssd_oracle_forward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups,
                       int64_t headdim, int64_t dstate, int dtype,
                       const void *x, const void *dt, const void *B, const void *C,
                       const double *A, const double *D, const double *h0,
                       const int64_t *units, int64_t n_units, int64_t chunk,
                       double *y, double *hT, double *snaps, int nthreads)
{
    if (batch <= 0 || seqlen <= 0 || nheads <= 0 || ngroups <= 0 || headdim <= 0 || dstate <= 0)
        return -1;
    if (nheads % ngroups != 0) return -2;
    if (dtype < ORC_F64 || dtype > ORC_BF16) return -3;
    if (!x || !dt || !B || !C || !A || !D) return -4;
    if (snaps && chunk <= 0) return -5;
    if (!units) n_units = batch * nheads;
    for (int64_t i = 0; units && i < n_units; ++i)
        if (units[i] < 0 || units[i] >= batch * nheads) return -6;

    oracle_job jb;
    jb.batch = batch; jb.seqlen = seqlen; jb.nheads = nheads; jb.ngroups = ngroups;
    jb.headdim = headdim; jb.dstate = dstate; jb.dtype = dtype;
    jb.x = x; jb.dt = dt; jb.B = B; jb.C = C; jb.A = A; jb.D = D; jb.h0 = h0;
    jb.units = units; jb.n_units = n_units; jb.chunk = chunk;
    jb.y = y; jb.hT = hT; jb.snaps = snaps; jb.next = 0;
    pthread_mutex_init(&jb.lock, NULL);

    if (nthreads < 1) nthreads = 1;
    if (nthreads > n_units) nthreads = (int)n_units;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int rc = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &jb) != 0) break;
        ++started;
    }
    if (started == 0) rc = (worker(&jb) != NULL) ? -7 : 0;
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r) rc = -7;
    }
    free(th);
    pthread_mutex_destroy(&jb.lock);
    return rc;
}

/*
 * G2[b,h,t] = log2(e) * sum_{k = chunk start of t .. t} A[h] * dt[b,k,h]
 * dtc[b,h,t] = dt[b,t,h] widened to double.  Both [b, H, L].
 */
int ssd_oracle_chunk_cumsum(int64_t batch, int64_t seqlen, int64_t nheads, int dtype,
                            const void *dt, const double *A, int64_t chunk,
                            double *G2, double *dtc)
{
    if (batch <= 0 || seqlen <= 0 || nheads <= 0 || chunk <= 0) return -1;
    if (dtype < ORC_F64 || dtype > ORC_BF16) return -3;
    if (!dt || !A || !G2) return -4;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < nheads; ++h) {
            double run = 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                if (t % chunk == 0) run = 0.0;
                const double d = load_elem(dt, dtype, (b * seqlen + t) * nheads + h);
                run += A[h] * d;
                G2[(b * nheads + h) * seqlen + t] = run * M_LOG2E;
                if (dtc) dtc[(b * nheads + h) * seqlen + t] = d;
            }
        }
    return 0;
}
