/*
 * oracle.c -- plain, slow, FP64 CPU reference for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * Sources (the lecture pages this follows; cited by title and section):
 *   [FL]  CS349E Lecture 11 shared module "flash_lab.py" (numpy FlashAttention,
 *         flash-decoding and megakernel models):
 *           §1 online softmax  -- softmax_3pass, softmax_online, partial_state,
 *                                 merge_states
 *           §2 standard attention -- _causal_mask, standard_attention
 *           §4 flash-decoding  -- split_kv_decode
 *           §2 backward of standard attention -- standard_attention_bwd
 *   [FF]  CS349E Lecture 11 "02_flash_forward.py", demo 1 (correctness): the
 *         flash forward computes exactly the standard result.
 *
 * What is computed is the *definition* of attention, not the tiled method:
 * the flash forward and flash-decoding reach the standard result exactly (up
 * to rounding order) per [FF] demo 1 and [FL] §3/§4, so the oracle for both
 * GPU entry points is standard attention written out with a materialised
 * score row and a three-pass softmax ([FL] §2, §1).
 *
 * Readings where the pages are silent or inconsistent (each also listed in
 * the design notes):
 *   R1  A query row with no visible key (causal, N > Nk, rows i < N-Nk) gets
 *       O = 0 and LSE = -inf: the identity state (m=-inf, l=0) of
 *       merge_states in [FL] §1.
 *   R4  LSE is the natural log-sum-exp of the *scaled* scores over the
 *       visible keys ([FL] §3 flash_fwd returns L = m + log l).
 *   R5  Causal alignment is bottom-right: query i sits at position Nk-N+i and
 *       sees key j iff j <= Nk-N+i ([FL] §2 _causal_mask with offset Nk-N).
 *   R6  split_kv_decode segment bounds are round-half-even of an evenly
 *       spaced grid 0..S with n_splits+1 points; empty segments are skipped
 *       ([FL] §4).
 *
 * Every function here is pinned by tests that do not re-type its formula:
 * closed forms, hand-derived golden values, invariants, brute force in
 * extended precision and an independent library cross-check.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* [FL] §2 standard attention, one head.                                     */
/*   S_ij = scale * sum_c q_ic k_jc          (masked -> -inf, R5)            */
/*   pass 1: m_i = max_j S_ij                                                */
/*   pass 2: e_ij = exp(S_ij - m_i), l_i = sum_j e_ij                        */
/*   pass 3: P_ij = e_ij / l_i, O_i = sum_j P_ij v_j, LSE_i = m_i + ln l_i   */
/* p (optional) receives the [N, Nk] probability matrix of this head.        */
/* ------------------------------------------------------------------------ */
static void attention_head(const double *q, const double *k, const double *v,
                           double *o, double *lse, double *p, long N, long Nk,
                           long d, long dv, int causal, double scale,
                           double *srow)
{
    for (long i = 0; i < N; ++i) {
        const double *qi = q + i * d;
        long last = Nk - 1;                      /* last visible key index */
        if (causal)
            last = Nk - N + i;                   /* R5: position of query i */
        /* scores of the materialised row; -inf where masked */
        for (long j = 0; j < Nk; ++j) {
            if (j > last) {
                srow[j] = -INFINITY;
                continue;
            }
            const double *kj = k + j * d;
            double acc = 0.0;
            for (long c = 0; c < d; ++c)
                acc += qi[c] * kj[c];
            srow[j] = scale * acc;
        }
        /* pass 1: row maximum */
        double m = -INFINITY;
        for (long j = 0; j < Nk; ++j)
            if (srow[j] > m)
                m = srow[j];
        double *oi = o + i * dv;
        if (m == -INFINITY) {                    /* R1: nothing visible */
            for (long c = 0; c < dv; ++c)
                oi[c] = 0.0;
            lse[i] = -INFINITY;
            if (p)
                for (long j = 0; j < Nk; ++j)
                    p[i * Nk + j] = 0.0;
            continue;
        }
        /* pass 2: exponentials and their sum (exp(-inf) = 0) */
        double l = 0.0;
        for (long j = 0; j < Nk; ++j) {
            srow[j] = exp(srow[j] - m);
            l += srow[j];
        }
        /* pass 3: normalise, then O = P V */
        for (long c = 0; c < dv; ++c)
            oi[c] = 0.0;
        for (long j = 0; j < Nk; ++j) {
            double pij = srow[j] / l;
            if (p)
                p[i * Nk + j] = pij;
            const double *vj = v + j * dv;
            for (long c = 0; c < dv; ++c)
                oi[c] += pij * vj[c];
        }
        lse[i] = m + log(l);
    }
}

typedef struct {
    const double *q, *k, *v;
    double *o, *lse, *p;
    long H, N, Nk, d, dv;
    int causal;
    double scale;
    long head_begin, head_end;
} job_t;

static void *attention_worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    double *srow = (double *)malloc(sizeof(double) * (size_t)(jb->Nk > 0 ? jb->Nk : 1));
    if (!srow)
        return (void *)1;
    for (long h = jb->head_begin; h < jb->head_end; ++h) {
        attention_head(jb->q + h * jb->N * jb->d, jb->k + h * jb->Nk * jb->d,
                       jb->v + h * jb->Nk * jb->dv, jb->o + h * jb->N * jb->dv,
                       jb->lse + h * jb->N,
                       jb->p ? jb->p + h * jb->N * jb->Nk : NULL, jb->N, jb->Nk,
                       jb->d, jb->dv, jb->causal, jb->scale, srow);
    }
    free(srow);
    return NULL;
}

/*
 * Standard attention over contiguous q[B,H,N,d], k[B,H,Nk,d], v[B,H,Nk,dv];
 * writes o[B,H,N,dv], lse[B,H,N] and, if p != NULL, p[B,H,N,Nk].
 * Heads are independent and are spread over `nthreads` POSIX threads; each
 * head is computed by exactly the serial code above, so the result does not
 * depend on the thread count.  Returns 0 on success, -1 on bad arguments,
 * -2 if a thread or buffer could not be created.
 */
int oracle_attention(const double *q, const double *k, const double *v,
                     double *o, double *lse, double *p, long B, long H, long N,
                     long Nk, long d, long dv, int causal, double scale,
                     int nthreads)
{
    if (!q || !k || !v || !o || !lse || B < 1 || H < 1 || N < 1 || Nk < 1 ||
        d < 1 || dv < 1)
        return -1;
    long heads = B * H;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > heads)
        nthreads = (int)heads;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -2;
    }
    int rc = 0;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (job_t){q, k, v, o, lse, p, H, N, Nk, d, dv, causal, scale,
                          heads * t / nthreads, heads * (t + 1) / nthreads};
        if (pthread_create(&th[t], NULL, attention_worker, &jobs[t]) != 0) {
            rc = -2;
            break;
        }
        ++started;
    }
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret)
            rc = -2;
    }
    free(jobs);
    free(th);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* [FL] §1 softmax in three passes over each row: max, sum of exp, divide.   */
/* ------------------------------------------------------------------------ */
void oracle_softmax_3pass(const double *x, double *y, long rows, long n)
{
    for (long r = 0; r < rows; ++r) {
        const double *xr = x + r * n;
        double *yr = y + r * n;
        double m = -INFINITY;
        for (long j = 0; j < n; ++j)
            if (xr[j] > m)
                m = xr[j];
        double s = 0.0;
        for (long j = 0; j < n; ++j)
            s += exp(xr[j] - m);
        for (long j = 0; j < n; ++j)
            yr[j] = exp(xr[j] - m) / s;
    }
}

/* ------------------------------------------------------------------------ */
/* [FL] §1 online softmax: one sweep in blocks keeps a running maximum m and */
/* a running sum l of exp(x - m); when a block raises the maximum, the old   */
/* sum is carried over by the factor exp(m_old - m_new).  A second sweep     */
/* normalises.  `block` need not divide n.                                   */
/* ------------------------------------------------------------------------ */
void oracle_softmax_online(const double *x, double *y, long rows, long n,
                           long block)
{
    if (block < 1)
        block = 1;
    for (long r = 0; r < rows; ++r) {
        const double *xr = x + r * n;
        double *yr = y + r * n;
        double m = -INFINITY, l = 0.0;
        for (long s = 0; s < n; s += block) {
            long e = s + block < n ? s + block : n;
            double mb = -INFINITY;
            for (long j = s; j < e; ++j)
                if (xr[j] > mb)
                    mb = xr[j];
            double m_new = m > mb ? m : mb;
            double carry = (m == -INFINITY) ? 0.0 : exp(m - m_new);
            double add = 0.0;
            for (long j = s; j < e; ++j)
                add += exp(xr[j] - m_new);
            l = l * carry + add;
            m = m_new;
        }
        for (long j = 0; j < n; ++j)
            yr[j] = exp(xr[j] - m) / l;
    }
}

/* ------------------------------------------------------------------------ */
/* [FL] §1 partial state of one segment of a row: m = max, l = sum exp(x-m), */
/* o = sum exp(x-m) v_j (unnormalised).  v may be NULL (then o is unused).   */
/* x[rows, n], v[n, dv] shared by all rows, o[rows, dv].                     */
/* An all -inf row gives m=-inf, l=0, o=0 (the identity state).             */
/* ------------------------------------------------------------------------ */
void oracle_partial_state(const double *x, const double *v, long rows, long n,
                          long dv, double *m, double *l, double *o)
{
    for (long r = 0; r < rows; ++r) {
        const double *xr = x + r * n;
        double mr = -INFINITY;
        for (long j = 0; j < n; ++j)
            if (xr[j] > mr)
                mr = xr[j];
        m[r] = mr;
        double lr = 0.0;
        if (v && o)
            for (long c = 0; c < dv; ++c)
                o[r * dv + c] = 0.0;
        if (mr == -INFINITY) {
            l[r] = 0.0;
            continue;
        }
        for (long j = 0; j < n; ++j) {
            double e = exp(xr[j] - mr);
            lr += e;
            if (v && o)
                for (long c = 0; c < dv; ++c)
                    o[r * dv + c] += e * v[j * dv + c];
        }
        l[r] = lr;
    }
}

/* ------------------------------------------------------------------------ */
/* [FL] §1 merge_states: m = max(ma, mb); each side is rescaled by           */
/* exp(m_side - m), taken as 0 when m_side = -inf; l and o add.              */
/* o arrays may be NULL (dv ignored).  Output may alias an input.            */
/* ------------------------------------------------------------------------ */
void oracle_merge_states(const double *ma, const double *la, const double *oa,
                         const double *mb, const double *lb, const double *ob,
                         long rows, long dv, double *m, double *l, double *o)
{
    for (long r = 0; r < rows; ++r) {
        double a = ma[r], b = mb[r];
        double mm = a > b ? a : b;
        double fa = (a == -INFINITY) ? 0.0 : exp(a - mm);
        double fb = (b == -INFINITY) ? 0.0 : exp(b - mm);
        double lr = la[r] * fa + lb[r] * fb;
        if (oa && ob && o)
            for (long c = 0; c < dv; ++c)
                o[r * dv + c] = oa[r * dv + c] * fa + ob[r * dv + c] * fb;
        m[r] = mm;
        l[r] = lr;
    }
}

/* ------------------------------------------------------------------------ */
/* [FL] §4 split-KV decode of R query rows q[R,d] against one head K[S,d],   */
/* V[S,dv] (no mask).  Segment s covers keys [b_s, b_{s+1}) with            */
/* b_s = round-half-even(s * S / n_splits), b_n = S (R6); empty segments are */
/* skipped.  Each segment yields o_s = softmax(q K_s^T scale) V_s (already   */
/* normalised) and lse_s; then lse = log sum_s exp(lse_s) (taken about the   */
/* largest lse_s) and o = sum_s exp(lse_s - lse) o_s.                        */
/* Returns the number of non-empty segments, or -1 on bad arguments.        */
/* ------------------------------------------------------------------------ */
int oracle_split_kv_decode(const double *q, const double *K, const double *V,
                           long R, long S, long d, long dv, long n_splits,
                           double scale, double *o, double *lse)
{
    if (!q || !K || !V || !o || !lse || R < 1 || S < 1 || d < 1 || dv < 1 ||
        n_splits < 1)
        return -1;
    double *seg_o = (double *)calloc((size_t)(n_splits * R * dv), sizeof(double));
    double *seg_lse = (double *)calloc((size_t)(n_splits * R), sizeof(double));
    double *s = (double *)malloc(sizeof(double) * (size_t)S);
    if (!seg_o || !seg_lse || !s) {
        free(seg_o);
        free(seg_lse);
        free(s);
        return -1;
    }
    long used = 0;
    double step = (double)S / (double)n_splits;
    for (long sp = 0; sp < n_splits; ++sp) {
        long a = (long)nearbyint((double)sp * step);
        long b = (sp + 1 == n_splits) ? S : (long)nearbyint((double)(sp + 1) * step);
        if (b <= a)
            continue;                                  /* empty: skipped */
        for (long r = 0; r < R; ++r) {
            double mr = -INFINITY;
            for (long j = a; j < b; ++j) {
                double acc = 0.0;
                for (long c = 0; c < d; ++c)
                    acc += q[r * d + c] * K[j * d + c];
                s[j] = acc * scale;
                if (s[j] > mr)
                    mr = s[j];
            }
            double lr = 0.0;
            double *os = seg_o + (used * R + r) * dv;
            for (long j = a; j < b; ++j) {
                double e = exp(s[j] - mr);
                lr += e;
                for (long c = 0; c < dv; ++c)
                    os[c] += e * V[j * dv + c];
            }
            for (long c = 0; c < dv; ++c)
                os[c] /= lr;
            seg_lse[used * R + r] = mr + log(lr);
        }
        ++used;
    }
    for (long r = 0; r < R; ++r) {
        double big = -INFINITY;
        for (long u = 0; u < used; ++u)
            if (seg_lse[u * R + r] > big)
                big = seg_lse[u * R + r];
        double tot = 0.0;
        for (long u = 0; u < used; ++u)
            tot += exp(seg_lse[u * R + r] - big);
        lse[r] = log(tot) + big;
        for (long c = 0; c < dv; ++c) {
            double acc = 0.0;
            for (long u = 0; u < used; ++u)
                acc += exp(seg_lse[u * R + r] - lse[r]) * seg_o[(u * R + r) * dv + c];
            o[r * dv + c] = acc;
        }
    }
    free(seg_o);
    free(seg_lse);
    free(s);
    return (int)used;
}

/* ------------------------------------------------------------------------ */
/* [FL] §2 standard attention backward, one head, from the materialised P    */
/* of the forward definition above (a row with no visible key has P = 0):    */
/*   D_i   = sum_c dO_ic O_ic                                                */
/*   dV    = P^T dO                                                          */
/*   dP    = dO V^T                                                          */
/*   dS    = P o (dP - D)          (elementwise; D broadcast along a row)    */
/*   dQ    = scale * dS K                                                    */
/*   dK    = scale * dS^T Q                                                  */
/* p [N, Nk], orow [dv] are caller scratch.                                  */
/* ------------------------------------------------------------------------ */
static void attention_bwd_head(const double *q, const double *k, const double *v,
                               const double *dout, double *dq, double *dk,
                               double *dvv, long N, long Nk, long d, long dv,
                               int causal, double scale, double *p, double *o,
                               double *lse, double *srow)
{
    attention_head(q, k, v, o, lse, p, N, Nk, d, dv, causal, scale, srow);
    for (long x = 0; x < N * d; ++x)
        dq[x] = 0.0;
    for (long x = 0; x < Nk * d; ++x)
        dk[x] = 0.0;
    for (long x = 0; x < Nk * dv; ++x)
        dvv[x] = 0.0;
    for (long i = 0; i < N; ++i) {
        const double *doi = dout + i * dv;
        const double *oi = o + i * dv;
        double Di = 0.0;
        for (long c = 0; c < dv; ++c)
            Di += doi[c] * oi[c];
        for (long j = 0; j < Nk; ++j) {
            double pij = p[i * Nk + j];
            const double *vj = v + j * dv;
            double *dvj = dvv + j * dv;
            for (long c = 0; c < dv; ++c)
                dvj[c] += pij * doi[c];                  /* dV = P^T dO */
            double dpij = 0.0;
            for (long c = 0; c < dv; ++c)
                dpij += doi[c] * vj[c];                  /* dP = dO V^T */
            double dsij = pij * (dpij - Di);             /* dS = P o (dP - D) */
            const double *kj = k + j * d;
            const double *qi = q + i * d;
            double *dqi = dq + i * d;
            double *dkj = dk + j * d;
            for (long c = 0; c < d; ++c) {
                dqi[c] += scale * dsij * kj[c];          /* dQ = scale dS K */
                dkj[c] += scale * dsij * qi[c];          /* dK = scale dS^T Q */
            }
        }
    }
}

typedef struct {
    const double *q, *k, *v, *dout;
    double *dq, *dk, *dv;
    long H, N, Nk, d, dvd;
    int causal;
    double scale;
    long head_begin, head_end;
} bwd_job_t;

static void *attention_bwd_worker(void *arg)
{
    bwd_job_t *jb = (bwd_job_t *)arg;
    size_t np = (size_t)jb->N * (size_t)jb->Nk;
    double *p = (double *)malloc(sizeof(double) * np);
    double *o = (double *)malloc(sizeof(double) * (size_t)(jb->N * jb->dvd));
    double *lse = (double *)malloc(sizeof(double) * (size_t)jb->N);
    double *srow = (double *)malloc(sizeof(double) * (size_t)jb->Nk);
    void *ret = NULL;
    if (!p || !o || !lse || !srow) {
        ret = (void *)1;
    } else {
        for (long h = jb->head_begin; h < jb->head_end; ++h)
            attention_bwd_head(jb->q + h * jb->N * jb->d, jb->k + h * jb->Nk * jb->d,
                               jb->v + h * jb->Nk * jb->dvd, jb->dout + h * jb->N * jb->dvd,
                               jb->dq + h * jb->N * jb->d, jb->dk + h * jb->Nk * jb->d,
                               jb->dv + h * jb->Nk * jb->dvd, jb->N, jb->Nk, jb->d, jb->dvd,
                               jb->causal, jb->scale, p, o, lse, srow);
    }
    free(p);
    free(o);
    free(lse);
    free(srow);
    return ret;
}

/*
 * Backward of standard attention over contiguous q[B,H,N,d], k[B,H,Nk,d],
 * v[B,H,Nk,dv] and the output gradient dout[B,H,N,dv]: writes dq[B,H,N,d],
 * dk[B,H,Nk,d], dv[B,H,Nk,dv].  Threads over heads as oracle_attention; the
 * result does not depend on the thread count.  Returns 0, -1 on bad
 * arguments, -2 if a thread or buffer could not be created.
 */
int oracle_attention_bwd(const double *q, const double *k, const double *v,
                         const double *dout, double *dq, double *dk, double *dv,
                         long B, long H, long N, long Nk, long d, long dvd,
                         int causal, double scale, int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 1 || H < 1 || N < 1 ||
        Nk < 1 || d < 1 || dvd < 1)
        return -1;
    long heads = B * H;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > heads)
        nthreads = (int)heads;
    bwd_job_t *jobs = (bwd_job_t *)calloc((size_t)nthreads, sizeof(bwd_job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -2;
    }
    int rc = 0;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (bwd_job_t){q, k, v, dout, dq, dk, dv, H, N, Nk, d, dvd, causal, scale,
                              heads * t / nthreads, heads * (t + 1) / nthreads};
        if (pthread_create(&th[t], NULL, attention_bwd_worker, &jobs[t]) != 0) {
            rc = -2;
            break;
        }
        ++started;
    }
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret)
            rc = -2;
    }
    free(jobs);
    free(th);
    return rc;
}
