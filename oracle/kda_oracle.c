/*
 * KDA fp64 reference oracle — TEST INFRASTRUCTURE ONLY (see kda_oracle.h).
 *
 * Plain token-by-token recurrence, one (batch, head) pair per task, tasks
 * handed out to a small pthread pool. No blocking, fusion or reordering beyond
 * the definition: for every token the state is decayed row by row, the
 * retrieval Sbar^T k is formed, the delta write is added, and the output is
 * read from the updated state.
 */
#include "kda_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *la, *beta, *S0;
    double *o, *S_final;
    long B, T, H, dk, dv;
    long next;                 /* next (b,h) task */
    pthread_mutex_t lock;
} job_t;

/* One recurrence step on S (dk x dv) for token inputs qt, kt, vt, lat, bt.
 * w is dv doubles of scratch. ot may be NULL. */
static void kda_step(double* S, const double* qt, const double* kt, const double* vt,
                     const double* lat, double bt, double* w, double* ot,
                     long dk, long dv)
{
    /* Decay old memory: Sbar = Diag(alpha) S (each key channel row by its own alpha). */
    for (long i = 0; i < dk; ++i) {
        const double a = exp(lat[i]);
        double* row = S + i * dv;
        for (long j = 0; j < dv; ++j) row[j] *= a;
    }
    /* Prediction from the decayed memory: v_old = Sbar^T k. */
    for (long j = 0; j < dv; ++j) w[j] = 0.0;
    for (long i = 0; i < dk; ++i) {
        const double ki = kt[i];
        const double* row = S + i * dv;
        for (long j = 0; j < dv; ++j) w[j] += row[j] * ki;
    }
    /* Delta write: S = Sbar + beta k (v - v_old)^T. */
    for (long j = 0; j < dv; ++j) w[j] = bt * (vt[j] - w[j]);
    for (long i = 0; i < dk; ++i) {
        const double ki = kt[i];
        double* row = S + i * dv;
        for (long j = 0; j < dv; ++j) row[j] += ki * w[j];
    }
    /* Read-out from the updated state: o = S^T q. */
    if (ot) {
        for (long j = 0; j < dv; ++j) ot[j] = 0.0;
        for (long i = 0; i < dk; ++i) {
            const double qi = qt[i];
            const double* row = S + i * dv;
            for (long j = 0; j < dv; ++j) ot[j] += row[j] * qi;
        }
    }
}

static void run_head(job_t* J, long b, long h, double* S, double* w)
{
    const long dk = J->dk, dv = J->dv, T = J->T, H = J->H;
    const size_t sz = (size_t)dk * (size_t)dv;
    if (J->S0) memcpy(S, J->S0 + ((size_t)b * H + h) * sz, sz * sizeof(double));
    else memset(S, 0, sz * sizeof(double));
    for (long t = 0; t < T; ++t) {
        const size_t th = (size_t)(b * T + t) * H + h;     /* token-head index */
        kda_step(S, J->q + th * dk, J->k + th * dk, J->v + th * dv, J->la + th * dk,
                 J->beta[th], w, J->o ? J->o + th * dv : NULL, dk, dv);
    }
    if (J->S_final) memcpy(J->S_final + ((size_t)b * H + h) * sz, S, sz * sizeof(double));
}

static void* worker(void* arg)
{
    job_t* J = (job_t*)arg;
    double* S = (double*)malloc(sizeof(double) * (size_t)J->dk * (size_t)J->dv);
    double* w = (double*)malloc(sizeof(double) * (size_t)J->dv);
    if (!S || !w) { free(S); free(w); return NULL; }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const long task = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (task >= J->B * J->H) break;
        run_head(J, task / J->H, task % J->H, S, w);
    }
    free(S);
    free(w);
    return NULL;
}

static int run_pool(job_t* J, int nthreads)
{
    const long tasks = J->B * J->H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > tasks) nthreads = (int)(tasks > 0 ? tasks : 1);
    pthread_mutex_init(&J->lock, NULL);
    J->next = 0;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -1;
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, worker, J) == 0) ++started;
    if (started == 0) worker(J);   /* no threads available: run inline */
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J->lock);
    return 0;
}

int kda_oracle_prefill_f64(const double* q, const double* k, const double* v,
                           const double* log_alpha, const double* beta,
                           const double* S0, double* o, double* S_final,
                           long B, long T, long H, long dk, long dv, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (T > 0 && (!q || !k || !v || !log_alpha || !beta)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.la = log_alpha; J.beta = beta; J.S0 = S0;
    J.o = o; J.S_final = S_final;
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv;
    return run_pool(&J, nthreads);
}

int kda_oracle_decode_f64(const double* q, const double* k, const double* v,
                          const double* log_alpha, const double* beta,
                          double* S, double* o,
                          long B, long H, long dk, long dv, int nthreads)
{
    /* A decode step is one token of the recurrence on the caller's state;
     * it runs the same step function head by head. */
    if (B < 0 || H < 0 || dk <= 0 || dv <= 0 || !S) return -1;
    (void)nthreads;
    double* w = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!w) return -1;
    const size_t sz = (size_t)dk * (size_t)dv;
    for (long bh = 0; bh < B * H; ++bh)
        kda_step(S + (size_t)bh * sz, q + (size_t)bh * dk, k + (size_t)bh * dk,
                 v + (size_t)bh * dv, log_alpha + (size_t)bh * dk, beta[bh], w,
                 o ? o + (size_t)bh * dv : NULL, dk, dv);
    free(w);
    return 0;
}
