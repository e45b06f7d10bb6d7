/*
 * fab_oracle.c -- plain, slow, f64 CPU oracle for the exact attention backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * library: it restates the definitions from the pages in the most direct form.
 *
 * What it computes (every quantity in double precision, from f32 inputs that
 * are promoted exactly):
 *
 *   Forward, as the ggmlR test file "tests/testthat/test-flash-attn-back.R"
 *   defines it in its plain-R reference `attn_ref`: for batch b, query head h,
 *   key/value head g = h / (H/Hkv) and query n,
 *       s[m] = scale * (q[:,n,h,b] . k[:,m,g,b]) + mask[m,n]   (scale first,
 *              then the additive mask, which is shared by all heads/batches);
 *       a row whose scores are all non-finite is skipped: its output is 0;
 *       otherwise mx = max over the finite scores, e[m] = exp(s[m]-mx) for
 *       finite s[m] and 0 otherwise, P = e / sum(e), O[:,h,n,b] = sum_m P[m] v[:,m,g,b].
 *   The labml "Flash Attention" page, section "Forward pass", gives the same
 *   quantities as S, L and P, and its "Flash Attention Optimization" section
 *   keeps the running max m and sum l; the row log-sum-exp reported here is
 *   LSE = mx + ln(sum e) (natural log), -inf for an all-masked row.
 *
 *   Backward, from the labml page, section "Backward pass":
 *       dV_j = sum_i P_ij dO_i ;  dP_ij = dO_i . V_j ;
 *       D_i  = dO_i . O_i            (equivalently sum_j P_ij dP_ij) ;
 *       dS_ij = P_ij (dP_ij - D_i)   (the page's last form of dsoftmax, with D_i) ;
 *       dQ_i = scale sum_j dS_ij K_j ;  dK_j = scale sum_i dS_ij Q_i .
 *   Here dO_i is the upstream gradient d[:,h,i,b].  Every gradient is the
 *   derivative of sum(d * attn) for the forward above, so an all-masked row
 *   contributes nothing and has zero dQ.
 *
 *   ALiBi (optional; the ggmlR test file names it only through `max_bias`, in its
 *   block "the graph builder rejects attention features it cannot differentiate",
 *   and gives no score function): with per-head slopes alibi[h] (NULL: none) the
 *   score gains the linear bias alibi[h] * (m - n) after the scale, next to the
 *   mask: s[m] = scale * (q . k) + alibi[h] * (m - n) + mask[m,n].  Everything else
 *   (softmax, LSE, backward) is unchanged: the bias is a constant of the inputs,
 *   so it only enters through P.
 *
 *   Result packing, from PowerInfer's "Function ggml_flash_attn_back" (result
 *   sizing) and the ggmlR test's `fab_grads` unpacker: one f32 buffer
 *   [dQ | dK | dV], each slice padded to 16 bytes (4 floats), padding zero.
 *
 * Organisation: a row pass computes, per (b, h, n), the forward row, LSE, D and
 * dQ directly from the formulas; a key pass computes, per (b, g, m), dK and dV
 * as the sums over the rows of the group's query heads that the formulas state,
 * re-evaluating P_ij and dP_ij from the row statistics (mx, sum e, D) of the row
 * pass.  Both passes write disjoint outputs, so the result does not depend on
 * the number of threads.
 *
 * Build: gcc -O2 -std=c11 -shared -fPIC -pthread (no -ffast-math: inf and NaN
 * semantics matter here).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, H, Hkv, N, M, DK, DV;
} oshape;

/* IEEE 754 binary16 -> double, written from the format's definition:
 * sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is
 * subnormal (fraction * 2^-24), exponent 31 is inf (fraction 0) or NaN. */
double fab_oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double x;
    if (e == 0)
        x = ldexp((double)f, -24);
    else if (e == 31)
        x = f ? NAN : INFINITY;
    else
        x = ldexp((double)(f | 0x400), e - 25);
    return sign ? -x : x;
}

static inline int64_t idx_q(const oshape *s, int64_t dk, int64_t n, int64_t h, int64_t b)
{ return dk + s->DK * (n + s->N * (h + s->H * b)); }
static inline int64_t idx_k(const oshape *s, int64_t dk, int64_t m, int64_t g, int64_t b)
{ return dk + s->DK * (m + s->M * (g + s->Hkv * b)); }
static inline int64_t idx_v(const oshape *s, int64_t dv, int64_t m, int64_t g, int64_t b)
{ return dv + s->DV * (m + s->M * (g + s->Hkv * b)); }
static inline int64_t idx_d(const oshape *s, int64_t dv, int64_t h, int64_t n, int64_t b)
{ return dv + s->DV * (h + s->H * (n + s->N * b)); }
static inline int64_t idx_row(const oshape *s, int64_t n, int64_t h, int64_t b)
{ return n + s->N * (h + s->H * b); }

/* score s[m] of query row (b,h,n) against key m: scale first, then the ALiBi
 * bias (when slopes are given) and the mask */
static double score(const oshape *s, const double *q, const double *k, const uint16_t *mask,
                    const double *alibi, double scale, int64_t b, int64_t h, int64_t g, int64_t n,
                    int64_t m)
{
    double acc = 0.0;
    const double *qr = q + idx_q(s, 0, n, h, b);
    const double *kr = k + idx_k(s, 0, m, g, b);
    for (int64_t i = 0; i < s->DK; ++i)
        acc += qr[i] * kr[i];
    acc *= scale;
    if (alibi)
        acc += alibi[h] * (double)(m - n);
    if (mask)
        acc += fab_oracle_half_to_double(mask[m + s->M * n]);
    return acc;
}

typedef struct {
    const oshape *s;
    const double *q, *k, *v, *d;
    const uint16_t *mask;
    const double *alibi;     /* per-head ALiBi slopes [H] or NULL */
    double scale;
    /* row pass outputs (any may be NULL) */
    double *O, *lse, *D, *rmax, *rsum, *dq;
    uint8_t *dead;           /* 1 when the row is all-masked */
    /* key pass outputs */
    double *dk, *dv;
    /* work list: when non-NULL, only these items are processed */
    const int64_t *items;
    int64_t n_items;
    int64_t next;            /* shared counter, guarded by lock */
    pthread_mutex_t lock;
    int check_failed;        /* D self-check */
} job;

static int64_t take(job *j)
{
    pthread_mutex_lock(&j->lock);
    int64_t t = j->next++;
    pthread_mutex_unlock(&j->lock);
    return t;
}

/* One query row (b, h, n): forward, LSE, D and dQ. */
static void row_work(job *j, int64_t r, double *sbuf, double *pbuf, double *dpbuf, double *obuf)
{
    const oshape *s = j->s;
    int64_t n = r % s->N;
    int64_t h = (r / s->N) % s->H;
    int64_t b = r / (s->N * s->H);
    int64_t g = h / (s->H / s->Hkv);
    int64_t row = idx_row(s, n, h, b);

    int any = 0;
    double mx = -INFINITY;
    for (int64_t m = 0; m < s->M; ++m) {
        sbuf[m] = score(s, j->q, j->k, j->mask, j->alibi, j->scale, b, h, g, n, m);
        if (isfinite(sbuf[m])) {
            any = 1;
            if (sbuf[m] > mx)
                mx = sbuf[m];
        }
    }
    if (!any) {
        /* all-masked row: output 0, no gradient, no contribution to dK/dV */
        if (j->O)
            for (int64_t i = 0; i < s->DV; ++i)
                j->O[idx_d(s, i, h, n, b)] = 0.0;
        if (j->lse) j->lse[row] = -INFINITY;
        if (j->D) j->D[row] = 0.0;
        if (j->rmax) j->rmax[row] = -INFINITY;
        if (j->rsum) j->rsum[row] = 0.0;
        if (j->dead) j->dead[row] = 1;
        if (j->dq)
            for (int64_t i = 0; i < s->DK; ++i)
                j->dq[idx_q(s, i, n, h, b)] = 0.0;
        return;
    }
    double L = 0.0;
    for (int64_t m = 0; m < s->M; ++m) {
        pbuf[m] = isfinite(sbuf[m]) ? exp(sbuf[m] - mx) : 0.0;
        L += pbuf[m];
    }
    for (int64_t m = 0; m < s->M; ++m)
        pbuf[m] /= L;
    for (int64_t i = 0; i < s->DV; ++i) {
        double acc = 0.0;
        for (int64_t m = 0; m < s->M; ++m)
            acc += pbuf[m] * j->v[idx_v(s, i, m, g, b)];
        obuf[i] = acc;
    }
    if (j->O)
        for (int64_t i = 0; i < s->DV; ++i)
            j->O[idx_d(s, i, h, n, b)] = obuf[i];
    if (j->lse) j->lse[row] = mx + log(L);
    if (j->rmax) j->rmax[row] = mx;
    if (j->rsum) j->rsum[row] = L;
    if (j->dead) j->dead[row] = 0;

    if (!j->d)
        return;
    const double *dO = j->d + idx_d(s, 0, h, n, b);
    double D = 0.0;
    for (int64_t i = 0; i < s->DV; ++i)
        D += dO[i] * obuf[i];
    double D2 = 0.0;
    for (int64_t m = 0; m < s->M; ++m) {
        double acc = 0.0;
        const double *vr = j->v + idx_v(s, 0, m, g, b);
        for (int64_t i = 0; i < s->DV; ++i)
            acc += dO[i] * vr[i];
        dpbuf[m] = acc;
        D2 += pbuf[m] * acc;
    }
    /* D_i = dO_i . O_i = sum_j P_ij dP_ij (labml page, "Backward pass") */
    if (!(fabs(D - D2) <= 1e-9 * (1.0 + fabs(D))))
        j->check_failed = 1;
    if (j->D) j->D[row] = D;
    if (j->dq) {
        for (int64_t i = 0; i < s->DK; ++i)
            j->dq[idx_q(s, i, n, h, b)] = 0.0;
        for (int64_t m = 0; m < s->M; ++m) {
            double dS = pbuf[m] * (dpbuf[m] - D);
            const double *kr = j->k + idx_k(s, 0, m, g, b);
            for (int64_t i = 0; i < s->DK; ++i)
                j->dq[idx_q(s, i, n, h, b)] += j->scale * dS * kr[i];
        }
    }
}

/* One key (b, g, m): dK and dV (into kacc[DK], vacc[DV]) as the sums over the
 * rows of the group's query heads. */
static void key_work(job *j, int64_t r, double *kacc, double *vacc)
{
    const oshape *s = j->s;
    int64_t m = r % s->M;
    int64_t g = (r / s->M) % s->Hkv;
    int64_t b = r / (s->M * s->Hkv);
    int64_t rk2 = s->H / s->Hkv;
    memset(kacc, 0, sizeof(double) * s->DK);
    memset(vacc, 0, sizeof(double) * s->DV);
    const double *vr = j->v + idx_v(s, 0, m, g, b);
    for (int64_t h = g * rk2; h < (g + 1) * rk2; ++h) {
        for (int64_t n = 0; n < s->N; ++n) {
            int64_t row = idx_row(s, n, h, b);
            if (j->dead[row])
                continue;
            double sc = score(s, j->q, j->k, j->mask, j->alibi, j->scale, b, h, g, n, m);
            if (!isfinite(sc))
                continue;                    /* weight 0 */
            double P = exp(sc - j->rmax[row]) / j->rsum[row];
            const double *dO = j->d + idx_d(s, 0, h, n, b);
            double dP = 0.0;
            for (int64_t i = 0; i < s->DV; ++i)
                dP += dO[i] * vr[i];
            double dS = P * (dP - j->D[row]);
            const double *qr = j->q + idx_q(s, 0, n, h, b);
            for (int64_t i = 0; i < s->DK; ++i)
                kacc[i] += j->scale * dS * qr[i];
            for (int64_t i = 0; i < s->DV; ++i)
                vacc[i] += P * dO[i];
        }
    }
}

static void *row_thread(void *arg)
{
    job *j = (job *)arg;
    const oshape *s = j->s;
    double *sbuf = malloc(sizeof(double) * (s->M + 1));
    double *pbuf = malloc(sizeof(double) * (s->M + 1));
    double *dpbuf = malloc(sizeof(double) * (s->M + 1));
    double *obuf = malloc(sizeof(double) * (s->DV + 1));
    int64_t total = j->items ? j->n_items : s->B * s->H * s->N;
    for (;;) {
        int64_t t = take(j);
        if (t >= total)
            break;
        row_work(j, j->items ? j->items[t] : t, sbuf, pbuf, dpbuf, obuf);
    }
    free(sbuf); free(pbuf); free(dpbuf); free(obuf);
    return NULL;
}

static void *key_thread(void *arg)
{
    job *j = (job *)arg;
    const oshape *s = j->s;
    double *kacc = malloc(sizeof(double) * (s->DK + 1));
    double *vacc = malloc(sizeof(double) * (s->DV + 1));
    int64_t total = j->items ? j->n_items : s->B * s->Hkv * s->M;
    for (;;) {
        int64_t t = take(j);
        if (t >= total)
            break;
        int64_t r = j->items ? j->items[t] : t;
        key_work(j, r, kacc, vacc);
        int64_t m = r % s->M, g = (r / s->M) % s->Hkv, b = r / (s->M * s->Hkv);
        for (int64_t i = 0; i < s->DK; ++i)
            j->dk[idx_k(s, i, m, g, b)] = kacc[i];
        for (int64_t i = 0; i < s->DV; ++i)
            j->dv[idx_v(s, i, m, g, b)] = vacc[i];
    }
    free(kacc); free(vacc);
    return NULL;
}

static void run(job *j, void *(*fn)(void *), int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    j->next = 0;
    for (int i = 0; i < nthreads; ++i)
        pthread_create(&th[i], NULL, fn, j);
    for (int i = 0; i < nthreads; ++i)
        pthread_join(th[i], NULL);
}

static int valid(const oshape *s)
{
    if (s->B < 0 || s->N < 0 || s->M < 0 || s->H < 1 || s->Hkv < 1 || s->DK < 1 || s->DV < 1)
        return 0;
    return s->H % s->Hkv == 0;
}

/* Forward only: O [DV,H,N,B] and LSE [N,H,B]; alibi: per-head slopes [H] or NULL.
 * Returns 0 on success. */
int fab_oracle_forward_alibi(const int64_t *shape7, const double *q, const double *k, const double *v,
                             const uint16_t *mask, const double *alibi, double scale, double *O, double *lse,
                             int nthreads)
{
    oshape s = {shape7[0], shape7[1], shape7[2], shape7[3], shape7[4], shape7[5], shape7[6]};
    if (!valid(&s))
        return -1;
    job j;
    memset(&j, 0, sizeof j);
    pthread_mutex_init(&j.lock, NULL);
    j.s = &s; j.q = q; j.k = k; j.v = v; j.mask = mask; j.alibi = alibi; j.scale = scale;
    j.O = O; j.lse = lse;
    run(&j, row_thread, nthreads);
    pthread_mutex_destroy(&j.lock);
    return 0;
}

int fab_oracle_forward(const int64_t *shape7, const double *q, const double *k, const double *v,
                       const uint16_t *mask, double scale, double *O, double *lse, int nthreads)
{
    return fab_oracle_forward_alibi(shape7, q, k, v, mask, NULL, scale, O, lse, nthreads);
}

/*
 * Full backward: dq [DK,N,H,B], dk [DK,M,Hkv,B], dv [DV,M,Hkv,B]; optionally
 * O, lse and D (row statistics, [N,H,B]); alibi: per-head slopes [H] or NULL.
 * Returns 0, -1 on a bad shape, or -2 when the D = sum P dP self-check failed
 * on some row.
 */
int fab_oracle_backward_alibi(const int64_t *shape7, const double *q, const double *k, const double *v,
                              const uint16_t *mask, const double *alibi, const double *d, double scale,
                              double *dq, double *dk, double *dv, double *O, double *lse, double *D,
                              int nthreads)
{
    oshape s = {shape7[0], shape7[1], shape7[2], shape7[3], shape7[4], shape7[5], shape7[6]};
    if (!valid(&s))
        return -1;
    int64_t rows = s.B * s.H * s.N;
    double *rD = malloc(sizeof(double) * (rows + 1));
    double *rmax = malloc(sizeof(double) * (rows + 1));
    double *rsum = malloc(sizeof(double) * (rows + 1));
    uint8_t *dead = malloc(rows + 1);
    job j;
    memset(&j, 0, sizeof j);
    pthread_mutex_init(&j.lock, NULL);
    j.s = &s; j.q = q; j.k = k; j.v = v; j.d = d; j.mask = mask; j.alibi = alibi; j.scale = scale;
    j.O = O; j.lse = lse; j.D = rD; j.rmax = rmax; j.rsum = rsum; j.dead = dead; j.dq = dq;
    run(&j, row_thread, nthreads);
    j.dk = dk; j.dv = dv;
    run(&j, key_thread, nthreads);
    if (D)
        memcpy(D, rD, sizeof(double) * rows);
    int bad = j.check_failed;
    pthread_mutex_destroy(&j.lock);
    free(rD); free(rmax); free(rsum); free(dead);
    return bad ? -2 : 0;
}

int fab_oracle_backward(const int64_t *shape7, const double *q, const double *k, const double *v,
                        const uint16_t *mask, const double *d, double scale,
                        double *dq, double *dk, double *dv, double *O, double *lse, double *D,
                        int nthreads)
{
    return fab_oracle_backward_alibi(shape7, q, k, v, mask, NULL, d, scale, dq, dk, dv, O, lse, D, nthreads);
}

/*
 * Sampled backward for large problems.
 *   rows  : n_rows flat row ids r = n + N*(h + H*b); dq_out gets DK doubles per row.
 *   keys  : n_keys flat key ids r = m + M*(g + Hkv*b); dk_out / dv_out get DK / DV
 *           doubles per key.
 * The row statistics needed by the keys are computed only for the rows that see
 * a finite score at one of the requested keys.
 */
int fab_oracle_backward_sampled_alibi(const int64_t *shape7, const double *q, const double *k,
                                      const double *v, const uint16_t *mask, const double *alibi,
                                      const double *d, double scale, const int64_t *rows, int64_t n_rows,
                                      double *dq_out, const int64_t *keys, int64_t n_keys, double *dk_out,
                                      double *dv_out, int nthreads)
{
    oshape s = {shape7[0], shape7[1], shape7[2], shape7[3], shape7[4], shape7[5], shape7[6]};
    if (!valid(&s))
        return -1;
    int64_t nrow_all = s.B * s.H * s.N;
    int64_t rk2 = s.H / s.Hkv;
    double *rD = malloc(sizeof(double) * (nrow_all + 1));
    double *rmax = malloc(sizeof(double) * (nrow_all + 1));
    double *rsum = malloc(sizeof(double) * (nrow_all + 1));
    uint8_t *dead = malloc(nrow_all + 1);
    double *dq_full = NULL;
    int64_t *need = malloc(sizeof(int64_t) * (nrow_all + 1));
    uint8_t *flag = calloc(nrow_all + 1, 1);
    int64_t n_need = 0;
    int bad = 0;

    /* rows requested for dQ */
    for (int64_t i = 0; i < n_rows; ++i)
        if (!flag[rows[i]]) { flag[rows[i]] = 1; need[n_need++] = rows[i]; }
    /* rows whose statistics a requested key needs: any row of the key's group
     * with a finite score at that key (its mask entry is not -inf/non-finite). */
    for (int64_t t = 0; t < n_keys; ++t) {
        int64_t m = keys[t] % s.M;
        int64_t g = (keys[t] / s.M) % s.Hkv;
        int64_t b = keys[t] / (s.M * s.Hkv);
        for (int64_t h = g * rk2; h < (g + 1) * rk2; ++h)
            for (int64_t n = 0; n < s.N; ++n) {
                if (mask && !isfinite(fab_oracle_half_to_double(mask[m + s.M * n])))
                    continue;
                int64_t row = idx_row(&s, n, h, b);
                if (!flag[row]) { flag[row] = 1; need[n_need++] = row; }
            }
    }
    /* dq for the needed rows goes to a full-size scratch so row_work can index it */
    dq_full = calloc((size_t)(s.DK * nrow_all + 1), sizeof(double));
    for (int64_t r = 0; r < nrow_all; ++r) dead[r] = 1;

    job j;
    memset(&j, 0, sizeof j);
    pthread_mutex_init(&j.lock, NULL);
    j.s = &s; j.q = q; j.k = k; j.v = v; j.d = d; j.mask = mask; j.alibi = alibi; j.scale = scale;
    j.D = rD; j.rmax = rmax; j.rsum = rsum; j.dead = dead; j.dq = dq_full;
    j.items = need; j.n_items = n_need;
    run(&j, row_thread, nthreads);
    bad |= j.check_failed;
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t r = rows[i];
        int64_t n = r % s.N, h = (r / s.N) % s.H, b = r / (s.N * s.H);
        for (int64_t c = 0; c < s.DK; ++c)
            dq_out[i * s.DK + c] = dq_full[idx_q(&s, c, n, h, b)];
    }
    free(dq_full);

    for (int64_t t = 0; t < n_keys; ++t)
        key_work(&j, keys[t], dk_out + t * s.DK, dv_out + t * s.DV);
    pthread_mutex_destroy(&j.lock);
    free(rD); free(rmax); free(rsum); free(dead); free(need); free(flag);
    return bad ? -2 : 0;
}

int fab_oracle_backward_sampled(const int64_t *shape7, const double *q, const double *k,
                                const double *v, const uint16_t *mask, const double *d,
                                double scale, const int64_t *rows, int64_t n_rows, double *dq_out,
                                const int64_t *keys, int64_t n_keys, double *dk_out,
                                double *dv_out, int nthreads)
{
    return fab_oracle_backward_sampled_alibi(shape7, q, k, v, mask, NULL, d, scale, rows, n_rows, dq_out,
                                             keys, n_keys, dk_out, dv_out, nthreads);
}

/* Blob layout from the pages: offsets in floats, each slice padded to 4 floats. */
static int64_t pad4(int64_t n) { return (n * 4 + 15) / 16 * 16 / 4; }

int fab_oracle_blob_layout(const int64_t *shape7, int64_t *off4)
{
    oshape s = {shape7[0], shape7[1], shape7[2], shape7[3], shape7[4], shape7[5], shape7[6]};
    int64_t nq = s.DK * s.N * s.H * s.B;
    int64_t nk = s.DK * s.M * s.Hkv * s.B;
    int64_t nv = s.DV * s.M * s.Hkv * s.B;
    off4[0] = 0;
    off4[1] = pad4(nq);
    off4[2] = off4[1] + pad4(nk);
    off4[3] = off4[2] + pad4(nv);
    return 0;
}

/* Pack dq | dk | dv into one zero-initialised blob of off4[3] doubles. */
int fab_oracle_pack(const int64_t *shape7, const double *dq, const double *dk, const double *dv,
                    double *blob)
{
    oshape s = {shape7[0], shape7[1], shape7[2], shape7[3], shape7[4], shape7[5], shape7[6]};
    int64_t off[4];
    fab_oracle_blob_layout(shape7, off);
    memset(blob, 0, sizeof(double) * off[3]);
    memcpy(blob + off[0], dq, sizeof(double) * (s.DK * s.N * s.H * s.B));
    memcpy(blob + off[1], dk, sizeof(double) * (s.DK * s.M * s.Hkv * s.B));
    memcpy(blob + off[2], dv, sizeof(double) * (s.DV * s.M * s.Hkv * s.B));
    return 0;
}
