/*
 * swa_oracle.c -- plain, slow fp64 CPU reference for SWA(w,s) attention with
 * attention sinks.  TEST INFRASTRUCTURE ONLY: nothing in the product path may
 * link, load or call this file.  It shares no code, header or table with the
 * HIP library; it is compiled with gcc on its own.
 *
 * What it computes (paper.rainbus.top summary of arXiv 2608.28444, section
 * "滑窗注意力 SWA(w, s)" and the core-method section, the windowed-softmax
 * equation; method steps, step 2; the ai-blog.deepmagic.app post, section
 * "他們測了什麼"):
 *
 *   For a query at 1-based position t, SWA(w,s) attends the first s tokens
 *   and the most recent w-s tokens, t itself included:
 *
 *     S_t = { i : 1 <= i <= min(s,t) }  U  { i : max(s+1, t-w+s+1) <= i <= t }
 *
 *   and normalises the softmax over S_t only, with scale 1/sqrt(d), d the
 *   head dimension:
 *
 *     x_t = sum_{i in S_t} exp(q_t.k_i/sqrt(d)) v_i / sum_{i in S_t} exp(q_t.k_i/sqrt(d))
 *
 *   With s = 0 this is exactly the windowed-softmax equation printed on the
 *   page (the sum from max(1, t-w+1) to t).  The window w counts the s sink
 *   slots (the same section's note on the notation says the w places include
 *   the s sinks).
 *
 * Learned sink (the Hugging Face follow-up story's Qwen3-4B study lists a
 * "576-token SWA (learned sink)" student beside "572-token SWA + 4 sink
 * tokens"; the pages do not define it further): the reading used here is a
 * per-query-head logit b_h that adds exp(b_h) to the denominator of every
 * row of that head and contributes no value:
 *
 *     x_t = sum_{i in S_t} e^{q_t.k_i/sqrt(d)} v_i / (e^{b_h} + sum_{i in S_t} e^{q_t.k_i/sqrt(d)})
 *
 * and the row's log-sum-exp includes the e^{b_h} term.
 *
 * Grouped-query attention: query head h reads key/value head h / G, where
 * G = Hq / Hkv (the pages are silent; contiguous groups are the reading used).
 *
 * All arithmetic is fp64.  Inputs are fp32 arrays holding the exact values the
 * device sees (bf16 inputs are widened exactly on the host before the call).
 * The softmax is shifted by the maximum score over S_t for range safety; in
 * exact arithmetic the shift cancels.
 *
 * Layouts (row-major, contiguous):
 *   prefill: Q, O [B, L, Hq, d]; K, V [B, L, Hkv, d]; lse [B, Hq, L]
 *   decode:  Q, O [B, Hq, d]; history rows Kh, Vh [B, npos, Hkv, d] holding
 *            the key/value rows of the 1-based positions pos[0..npos-1]
 *            (strictly increasing).  pos must contain every member of S_n;
 *            other positions are allowed and ignored.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

/* --- the attended set, straight from its definition --------------------- */

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

/* Writes the members of S_t in increasing order into out (capacity >= t) and
 * returns how many there are.  First the sinks 1..min(s,t), then the recent
 * part max(s+1, t-w+s+1)..t. */
int64_t swa_oracle_attended(int64_t w, int64_t s, int64_t t, int64_t *out)
{
    int64_t n = 0;
    if (t < 1 || w < 1 || s < 0 || s >= w) return -1;
    for (int64_t i = 1; i <= min64(s, t); ++i) out[n++] = i;
    for (int64_t i = max64(s + 1, t - w + s + 1); i <= t; ++i) out[n++] = i;
    return n;
}

/* --- one output row ------------------------------------------------------- */

/* Masked softmax of one query row over the rows listed in idx (0-based row
 * numbers into krow/vrow with stride `stride` floats).  Writes d outputs and
 * returns the log-sum-exp of the scaled scores.  `sink` is the learned-sink
 * logit of the row's head: one more term exp(sink) in the denominator, with
 * no value vector (-INFINITY: none). */
static double attend_row(const float *q, const float *kbase, const float *vbase,
                         int64_t stride, const int64_t *idx, int64_t cnt, int d,
                         double sink, double *sc, double *o)
{
    const double scale = 1.0 / sqrt((double)d);
    double m = sink;
    for (int64_t j = 0; j < cnt; ++j) {
        const float *k = kbase + idx[j] * stride;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)q[c] * (double)k[c];
        sc[j] = acc * scale;
        if (sc[j] > m) m = sc[j];
    }
    double den = sink == -INFINITY ? 0.0 : exp(sink - m);
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < cnt; ++j) {
        const double p = exp(sc[j] - m);
        const float *v = vbase + idx[j] * stride;
        den += p;
        for (int c = 0; c < d; ++c) o[c] += p * (double)v[c];
    }
    for (int c = 0; c < d; ++c) o[c] /= den;
    return m + log(den);
}

/* --- threading: a static split of the (b, h_q) pairs ----------------------- */

typedef struct {
    int kind; /* 0 prefill, 1 decode */
    const float *Q, *K, *V;
    double *O, *lse;
    const double *sink; /* per query head, or NULL */
    const int64_t *pos;
    int64_t npos, n;
    int B, L, Hq, Hkv, d;
    int64_t w, s;
    int first, last; /* range of b*Hq + h */
    int status;
} job_t;

static void *run_prefill(job_t *jb)
{
    const int d = jb->d, Hq = jb->Hq, Hkv = jb->Hkv, L = jb->L;
    const int G = Hq / Hkv;
    int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
    double *sc = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    if (!idx || !sc || !o) { jb->status = -2; goto done; }
    for (int bh = jb->first; bh < jb->last; ++bh) {
        const int b = bh / Hq, h = bh % Hq, hk = h / G;
        const int64_t kstride = (int64_t)Hkv * d;
        const float *kbase = jb->K + ((int64_t)b * L * Hkv + hk) * d;
        const float *vbase = jb->V + ((int64_t)b * L * Hkv + hk) * d;
        for (int64_t t = 1; t <= L; ++t) {
            const int64_t cnt = swa_oracle_attended(jb->w, jb->s, t, idx);
            if (cnt < 0) { jb->status = -1; goto done; }
            for (int64_t j = 0; j < cnt; ++j) idx[j] -= 1; /* position -> row */
            const float *q = jb->Q + (((int64_t)b * L + (t - 1)) * Hq + h) * d;
            const double l = attend_row(q, kbase, vbase, kstride, idx, cnt, d,
                                        jb->sink ? jb->sink[h] : -INFINITY, sc, o);
            double *dst = jb->O + (((int64_t)b * L + (t - 1)) * Hq + h) * d;
            for (int c = 0; c < d; ++c) dst[c] = o[c];
            if (jb->lse) jb->lse[((int64_t)b * Hq + h) * L + (t - 1)] = l;
        }
    }
done:
    free(idx); free(sc); free(o);
    return NULL;
}

/* position -> row number in the supplied history, or -1 if absent */
static int64_t find_pos(const int64_t *pos, int64_t npos, int64_t p)
{
    int64_t lo = 0, hi = npos - 1;
    while (lo <= hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (pos[mid] == p) return mid;
        if (pos[mid] < p) lo = mid + 1; else hi = mid - 1;
    }
    return -1;
}

static void *run_decode(job_t *jb)
{
    const int d = jb->d, Hq = jb->Hq, Hkv = jb->Hkv;
    const int G = Hq / Hkv;
    const int64_t n = jb->n, npos = jb->npos;
    int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    double *sc = (double *)malloc(sizeof(double) * (size_t)n);
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    if (!idx || !sc || !o) { jb->status = -2; goto done; }
    const int64_t cnt = swa_oracle_attended(jb->w, jb->s, n, idx);
    if (cnt < 0) { jb->status = -1; goto done; }
    for (int64_t j = 0; j < cnt; ++j) {
        const int64_t r = find_pos(jb->pos, npos, idx[j]);
        if (r < 0) { jb->status = -3; goto done; } /* a member of S_n not supplied */
        idx[j] = r;
    }
    for (int bh = jb->first; bh < jb->last; ++bh) {
        const int b = bh / Hq, h = bh % Hq, hk = h / G;
        const int64_t kstride = (int64_t)Hkv * d;
        const float *kbase = jb->K + ((int64_t)b * npos * Hkv + hk) * d;
        const float *vbase = jb->V + ((int64_t)b * npos * Hkv + hk) * d;
        const float *q = jb->Q + ((int64_t)b * Hq + h) * d;
        const double l = attend_row(q, kbase, vbase, kstride, idx, cnt, d,
                                    jb->sink ? jb->sink[h] : -INFINITY, sc, o);
        double *dst = jb->O + ((int64_t)b * Hq + h) * d;
        for (int c = 0; c < d; ++c) dst[c] = o[c];
        if (jb->lse) jb->lse[(int64_t)b * Hq + h] = l;
    }
done:
    free(idx); free(sc); free(o);
    return NULL;
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    return jb->kind == 0 ? run_prefill(jb) : run_decode(jb);
}

static int run_jobs(job_t proto, int nthreads)
{
    const int rows = proto.B * proto.Hq;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = rows > 0 ? rows : 1;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -2; }
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].first = (int)((int64_t)rows * i / nthreads);
        jobs[i].last = (int)((int64_t)rows * (i + 1) / nthreads);
        jobs[i].status = 0;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &jobs[i]);
    worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    int status = 0;
    for (int i = 0; i < nthreads; ++i) if (jobs[i].status) status = jobs[i].status;
    free(jobs); free(th);
    return status;
}

static int check_dims(int B, int Hq, int Hkv, int d, int64_t w, int64_t s)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv) return -1;
    if (s < 0 || w < 1 || s >= w) return -1;
    return 0;
}

/* Prefill: every row t = 1..L.  Returns 0, or <0 on bad arguments / no memory.
 * sink: NULL, or one learned-sink logit per query head. */
int swa_oracle_prefill_lsink(const float *Q, const float *K, const float *V, double *O,
                             double *lse, const double *sink, int B, int L, int Hq, int Hkv,
                             int d, int64_t w, int64_t s, int nthreads)
{
    if (check_dims(B, Hq, Hkv, d, w, s) || L < 0) return -1;
    job_t jb = {0};
    jb.kind = 0; jb.Q = Q; jb.K = K; jb.V = V; jb.O = O; jb.lse = lse; jb.sink = sink;
    jb.B = B; jb.L = L; jb.Hq = Hq; jb.Hkv = Hkv; jb.d = d; jb.w = w; jb.s = s;
    return run_jobs(jb, nthreads);
}

int swa_oracle_prefill(const float *Q, const float *K, const float *V, double *O,
                       double *lse, int B, int L, int Hq, int Hkv, int d,
                       int64_t w, int64_t s, int nthreads)
{
    return swa_oracle_prefill_lsink(Q, K, V, O, lse, NULL, B, L, Hq, Hkv, d, w, s, nthreads);
}

/* Decode at 1-based position n: the query rows Q attend S_n over the supplied
 * history.  Returns -3 if a member of S_n is missing from pos.  sink: NULL, or
 * one learned-sink logit per query head. */
int swa_oracle_decode_lsink(const float *Q, const int64_t *pos, int64_t npos,
                            const float *Kh, const float *Vh, double *O, double *lse,
                            const double *sink, int B, int Hq, int Hkv, int d, int64_t n,
                            int64_t w, int64_t s, int nthreads)
{
    if (check_dims(B, Hq, Hkv, d, w, s) || n < 1 || npos < 0) return -1;
    for (int64_t j = 1; j < npos; ++j) if (pos[j] <= pos[j - 1]) return -1;
    job_t jb = {0};
    jb.kind = 1; jb.Q = Q; jb.K = Kh; jb.V = Vh; jb.O = O; jb.lse = lse; jb.sink = sink;
    jb.pos = pos; jb.npos = npos; jb.n = n;
    jb.B = B; jb.Hq = Hq; jb.Hkv = Hkv; jb.d = d; jb.w = w; jb.s = s;
    return run_jobs(jb, nthreads);
}

int swa_oracle_decode(const float *Q, const int64_t *pos, int64_t npos,
                      const float *Kh, const float *Vh, double *O, double *lse,
                      int B, int Hq, int Hkv, int d, int64_t n, int64_t w,
                      int64_t s, int nthreads)
{
    return swa_oracle_decode_lsink(Q, pos, npos, Kh, Vh, O, lse, NULL, B, Hq, Hkv, d, n, w, s,
                                   nthreads);
}
