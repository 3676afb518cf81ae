/*
 * lla_oracle.c -- the CPU oracle for causal linear attention (TEST INFRASTRUCTURE).
 *
 * This file is test infrastructure (the oracle), not the product.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it.  It shares no source,
 * header or helper with the GPU library.
 *
 * What it computes (one (batch, head) stream at a time, all in double):
 *
 *   "Chunking, causality, and parallel prefill" (English slide deck),
 *   section "Naive recurrence": the memory state is advanced one token at a
 *   time, each S_t depending on S_{t-1}:
 *
 *       S_t = S_{t-1} + k_t v_t^T          (S is d_k x d_v, row index = key dim)
 *       o_t = S_t^T q_t                    (o_t[j] = sum_i q_t[i] * S_t[i][j])
 *
 *   The same deck, "Worked case - full trace", fixes S_0 = 0 for a fresh
 *   prompt and the orientation of S (S_4 = K_1^T V_1 = [[3,4],[5,5]]: row i
 *   collects the values of the tokens whose key has a 1 in position i).
 *   The deck's "Mechanism map" reduces decode to one token: the triangle is
 *   1x1 and what remains is the state read o = q^T S after the rank-1 update,
 *   i.e. exactly one iteration of the loop body below.
 *
 * Inputs are double arrays holding the exact values the GPU path is given
 * (bf16 or fp32 values upcast without rounding).  Layouts are dense row-major:
 *   q, k : [BH][T][dk]     v : [BH][T][dv]     O : [BH][T][dv]
 *   S    : [BH][dk][dv]    (in: S_0, out: S_T)
 * Every (batch, head) stream is independent; `nthreads` worker threads take
 * streams round-robin.  No blocking, fusion or reordering beyond the
 * recurrence itself: the update is applied, then the state is read.
 *
 * Gated (decayed) state -- a reading, not a formula of the pages: the deck's
 * "Boundary, evidence, and sources" cites the chunkwise form of gated linear
 * attention without stating a gate.  Read as one scalar gate g_t per stream
 * and token, applied to the previous state before the token's update:
 *
 *       S_t = g_t S_{t-1} + k_t v_t^T,     o_t = S_t^T q_t
 *
 * With g_t = 1 this is the recurrence above, operation for operation
 * (1.0 * x == x).  gate : [BH][T].
 *
 * Parity: pinned by the tests against the deck's printed trace values, the
 * closed forms O = tril(Q K^T) V + Q S_0 and S_T = S_0 + K^T V, and brute force;
 * the gated form against its own closed form (tril(Q K^T) weighted by the
 * products of the gates in between), g = 1 (the trace) and g = 0.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (no FMA contraction,
 * so each product and each sum is rounded as written).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v;
    const double *gate;   /* [BH][T] or NULL (no gate) */
    double *S, *O;
    int64_t BH, T, dk, dv;
    int64_t ckpt_every;   /* > 0: copy S after every ckpt_every tokens */
    double *ckpt;         /* [BH][T/ckpt_every][dk][dv] or NULL */
    int tid, nthreads;
} job_t;

/* One token of the recurrence on one stream: S += k v^T, then o = S^T q. */
static void recurrence_token(const double *qt, const double *kt, const double *vt,
                             double *S, double *ot, int64_t dk, int64_t dv)
{
    for (int64_t i = 0; i < dk; ++i) {
        const double ki = kt[i];
        double *row = S + i * dv;
        for (int64_t j = 0; j < dv; ++j)
            row[j] = row[j] + ki * vt[j];
    }
    for (int64_t j = 0; j < dv; ++j)
        ot[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i) {
        const double qi = qt[i];
        const double *row = S + i * dv;
        for (int64_t j = 0; j < dv; ++j)
            ot[j] = ot[j] + qi * row[j];
    }
}

/* One token of the gated recurrence: S = g S, then S += k v^T, then o = S^T q. */
static void gated_token(const double *qt, const double *kt, const double *vt, double g,
                        double *S, double *ot, int64_t dk, int64_t dv)
{
    for (int64_t i = 0; i < dk * dv; ++i)
        S[i] = g * S[i];
    recurrence_token(qt, kt, vt, S, ot, dk, dv);
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    const int64_t dk = jb->dk, dv = jb->dv, T = jb->T;
    const int64_t n_ckpt = jb->ckpt_every > 0 ? T / jb->ckpt_every : 0;
    for (int64_t bh = jb->tid; bh < jb->BH; bh += jb->nthreads) {
        double *S = jb->S + bh * dk * dv;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t row = bh * T + t;
            if (jb->gate)
                gated_token(jb->q + row * dk, jb->k + row * dk, jb->v + row * dv, jb->gate[row],
                            S, jb->O + row * dv, dk, dv);
            else
                recurrence_token(jb->q + row * dk, jb->k + row * dk, jb->v + row * dv,
                                 S, jb->O + row * dv, dk, dv);
            if (jb->ckpt && jb->ckpt_every > 0 && (t + 1) % jb->ckpt_every == 0) {
                const int64_t c = (t + 1) / jb->ckpt_every - 1;
                memcpy(jb->ckpt + (bh * n_ckpt + c) * dk * dv, S,
                       (size_t)(dk * dv) * sizeof(double));
            }
        }
    }
    return NULL;
}

/*
 * Token-by-token recurrence over T tokens for BH independent streams.
 * S holds S_0 on entry and S_T on return.  If ckpt is non-NULL and
 * ckpt_every > 0, the state after tokens ckpt_every, 2*ckpt_every, ... is
 * copied to ckpt[bh][c] (floor(T / ckpt_every) checkpoints per stream).
 * Returns 0, or -1 on a bad argument.
 */
static int run_jobs(const double *q, const double *k, const double *v, const double *gate,
                    double *S, double *O, int64_t BH, int64_t T, int64_t dk, int64_t dv,
                    int64_t ckpt_every, double *ckpt, int nthreads)
{
    if (BH < 0 || T < 0 || dk < 1 || dv < 1 || !S || (T > 0 && (!q || !k || !v || !O)))
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > BH)
        nthreads = BH > 0 ? (int)BH : 1;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        job_t j = {q, k, v, gate, S, O, BH, T, dk, dv, ckpt_every, ckpt, i, nthreads};
        jobs[i] = j;
    }
    /* Each job owns a disjoint set of streams; a job whose thread cannot be
       started runs on the caller instead, so the result never depends on how
       many threads actually started. */
    char *joined = (char *)calloc((size_t)nthreads, 1);
    for (int i = 1; i < nthreads; ++i)
        joined[i] = joined ? (pthread_create(&th[i], NULL, worker, &jobs[i]) == 0) : 0;
    worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) {
        if (joined && joined[i])
            pthread_join(th[i], NULL);
        else
            worker(&jobs[i]);
    }
    free(joined);
    free(jobs);
    free(th);
    return 0;
}

int lla_oracle_recurrence(const double *q, const double *k, const double *v,
                          double *S, double *O,
                          int64_t BH, int64_t T, int64_t dk, int64_t dv,
                          int64_t ckpt_every, double *ckpt, int nthreads)
{
    return run_jobs(q, k, v, NULL, S, O, BH, T, dk, dv, ckpt_every, ckpt, nthreads);
}

/*
 * The gated recurrence (see the header): gate [BH][T], one g_t per stream and
 * token.  S holds S_0 on entry and S_T on return.  Returns 0, or -1 on a bad
 * argument.
 */
int lla_oracle_gated_recurrence(const double *q, const double *k, const double *v,
                                const double *gate, double *S, double *O,
                                int64_t BH, int64_t T, int64_t dk, int64_t dv, int nthreads)
{
    if (T > 0 && !gate)
        return -1;
    return run_jobs(q, k, v, gate, S, O, BH, T, dk, dv, 0, NULL, nthreads);
}

/*
 * One decode step for BH independent streams: the 1x1-triangle case of the
 * deck's "Mechanism map" -- S += k v^T, then o = S^T q.
 * q, k : [BH][dk]   v, o : [BH][dv]   S : [BH][dk][dv] (in/out).
 */
int lla_oracle_decode_step(const double *q, const double *k, const double *v,
                           double *S, double *o, int64_t BH, int64_t dk, int64_t dv)
{
    if (BH < 0 || dk < 1 || dv < 1 || (BH > 0 && (!q || !k || !v || !S || !o)))
        return -1;
    for (int64_t bh = 0; bh < BH; ++bh)
        recurrence_token(q + bh * dk, k + bh * dk, v + bh * dv, S + bh * dk * dv,
                         o + bh * dv, dk, dv);
    return 0;
}

/* One gated decode step per stream: S = g S, S += k v^T, o = S^T q; gate [BH]. */
int lla_oracle_gated_decode_step(const double *q, const double *k, const double *v,
                                 const double *gate, double *S, double *o,
                                 int64_t BH, int64_t dk, int64_t dv)
{
    if (BH < 0 || dk < 1 || dv < 1 || (BH > 0 && (!q || !k || !v || !gate || !S || !o)))
        return -1;
    for (int64_t bh = 0; bh < BH; ++bh)
        gated_token(q + bh * dk, k + bh * dk, v + bh * dv, gate[bh], S + bh * dk * dv,
                    o + bh * dv, dk, dv);
    return 0;
}
