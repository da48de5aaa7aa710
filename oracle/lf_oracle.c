/*
 * lf_oracle.c -- plain fp64 CPU oracle for the Longformer sparse
 * self-attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP library; the two meet only through the seeded inputs.
 *
 * What it computes (sources are the pages' own sections):
 *
 *   Longformer (eightmm.github.io/papers/architectures/longformer),
 *   "Sliding-Window Attention":  N_local(i) = { j : |i - j| <= r },
 *       y_i = sum_{j in N(i)} softmax_j( q_i . k_j / sqrt(d_k) ) v_j .
 *   same page, "Global Attention":  for i in G, N(i) = all positions;
 *       for i not in G, N(i) = N_local(i) U G   (a set union: a global key
 *       that is also inside the window is counted once).
 *   same page, "Mask View": M_ij = 0 on N(i), -inf elsewhere, so the
 *       softmax runs over exactly the allowed set.
 *   Longformer (ciallo.wiki) §2.2.3 and "Longformer长序列处理" (aiqz.cc),
 *       section 膨胀窗口设计: a dilated window samples every delta-th
 *       position (distances delta, 2*delta, ...), same key count, wider
 *       reach.  Reading used here: key j is in N_local(i) iff
 *       |i - j| <= r*delta and (i - j) mod delta == 0.
 *   "Longformer长序列处理", Python 演示 note 3: positions outside the
 *       sequence are dropped (no wrap-around).
 *   same page, HF实践: the window may be given per layer as a list; here a
 *       call may give one radius per head (r_h), the same rule per head.
 *   Longformer (eightmm.github.io), "Implementation Reading" asks whether
 *       windows are one-sided or two-sided.  One-sided reading used here:
 *       key j is in N_local(i) iff 0 <= i - j <= r*delta and
 *       (i - j) mod delta == 0 (the query and the keys before it); global
 *       rows and global keys are as in the two-sided case.
 *   BigBird, as the pages describe it beside Longformer (the mhpn.cn guide
 *       to long-text models, BERT to Longformer, BigBird and RoPE, §2.2.1
 *       and §2.2.2; Longformer (ciallo.wiki) on BigBird): each token also
 *       attends to a few randomly chosen other tokens; the sparse pattern
 *       works in blocks of block_size, usually 64.  Reading used here: the caller draws, for every head
 *       and every query block of 64 positions, n_rand key blocks of 64
 *       positions; a non-global query i also attends to every valid key of
 *       the blocks drawn for its block i / 64 (a set union with the window
 *       and G: each key counts once).  Heads with random blocks have
 *       delta = 1, as in BigBird.
 *   same page, "Implementation Reading" asks that padding be masked:
 *       a padded key leaves every query's set (global rows included);
 *       a padded query row is defined as all zeros.
 *
 * Indices are 0-based (the pages count from 1).  Arithmetic is IEEE fp64;
 * inputs arrive as float32 (bf16 and fp32 inputs are exact in float32) and
 * are widened exactly.  Sums run in ascending key order, so the result is
 * reproducible bit for bit.
 *
 * Gradients (lf_oracle_bwd).  The pages give no backward pass; Longformer
 * (ciallo.wiki) §5.2 only says that training cost grows linearly with the
 * length.  What is computed is the derivative of the forward map above,
 * from the chain rule through the softmax: with P_ij the weights of row i,
 * dP_ij = dy_i . v_j and D_i = sum_j P_ij dP_ij,
 *     dv_j += P_ij dy_i,   dS_ij = P_ij (dP_ij - D_i),
 *     dq_i += dS_ij k_j / sqrt(d_k),   dk_j += dS_ij q_i / sqrt(d_k),
 * summed over the same allowed pairs as the forward.  A padded query row is
 * zero whatever q_i holds, so it passes no gradient.
 *
 * Pins (checked in the CPU test suite): dense brute force with an explicit
 * T x T boolean mask on tiny T; closed-form neighbour counts; v == 1 gives
 * y == 1; q == 0 gives the plain mean of v over N(i); r = 0 with no globals
 * gives y_i = v_i; r >= T-1 equals textbook dense attention; a dilated
 * head equals delta undilated problems on the residue subsequences; keys
 * outside N(i) do not influence row i; global rows equal dense rows.
 * Gradients: float64 autograd of the dense brute force, central finite
 * differences, sum_j dk_j = 0 and sum_j dv_j = sum of dy over valid rows;
 * the gradient at chosen rows and keys (lf_oracle_bwd_rows, _keys) against
 * autograd and, bit for bit, the whole gradient.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* The global set G: sorted, duplicates removed, as a set of positions. */

typedef struct {
    int *pos;  /* sorted, unique */
    int n;
} gset_t;

static int cmp_int(const void *a, const void *b) {
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

static int gset_make(gset_t *g, const int *idx, int n, int T) {
    g->n = 0;
    g->pos = NULL;
    if (n <= 0) return 0;
    g->pos = (int *)malloc(sizeof(int) * (size_t)n);
    if (!g->pos) return -1;
    for (int i = 0; i < n; i++) {
        if (idx[i] < 0 || idx[i] >= T) { free(g->pos); g->pos = NULL; return -1; }
        g->pos[i] = idx[i];
    }
    qsort(g->pos, (size_t)n, sizeof(int), cmp_int);
    int m = 0;
    for (int i = 0; i < n; i++)
        if (m == 0 || g->pos[m - 1] != g->pos[i]) g->pos[m++] = g->pos[i];
    g->n = m;
    return 0;
}

static int gset_has(const gset_t *g, int i) {
    int lo = 0, hi = g->n - 1;
    while (lo <= hi) {
        int mid = (lo + hi) / 2;
        if (g->pos[mid] == i) return 1;
        if (g->pos[mid] < i) lo = mid + 1; else hi = mid - 1;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* N(i) for one query, written out as a sorted list of key positions.
 * Returns |N(i)|; a padded query gets the empty set (its row is zero). */

#define RAND_BLOCK 64

static int neighbours(int T, int r, int delta, int one_sided, const gset_t *G,
                      const unsigned char *pad /* [T] or NULL */, int i, int *out,
                      const int *rblk /* this head's [ceil(T/64)][n_rand] or NULL */, int n_rand,
                      unsigned char *mark /* [T] scratch when rblk is given */) {
    if (pad && pad[i]) return 0;
    int n = 0;
    if (gset_has(G, i)) {
        /* global query: every valid position */
        for (int j = 0; j < T; j++)
            if (!(pad && pad[j])) out[n++] = j;
        return n;
    }
    /* N_local(i): j = i + t*delta for t in [-r, r], inside [0, T) */
    long long tlo = -(long long)r, thi = (long long)r;
    if (one_sided) thi = 0;                              /* keys at or before i only */
    long long tmin = -((long long)i / delta);            /* smallest t with j >= 0 */
    long long tmax = ((long long)(T - 1) - i) / delta;   /* largest t with j < T  */
    if (tlo < tmin) tlo = tmin;
    if (thi > tmax) thi = tmax;
    /* merge the ascending window with the ascending global list (set union) */
    int gi = 0;
    for (long long t = tlo; t <= thi; t++) {
        int j = (int)((long long)i + t * delta);
        while (gi < G->n && G->pos[gi] < j) {
            int g = G->pos[gi++];
            if (!(pad && pad[g])) out[n++] = g;
        }
        if (gi < G->n && G->pos[gi] == j) gi++; /* same key: keep one copy */
        if (!(pad && pad[j])) out[n++] = j;
    }
    while (gi < G->n) {
        int g = G->pos[gi++];
        if (!(pad && pad[g])) out[n++] = g;
    }
    if (rblk && n_rand > 0) {
        /* add the valid keys of the random blocks of i's query block: mark
         * every key of the set so far and of the blocks, then list them in
         * ascending order (a key in both counts once) */
        memset(mark, 0, (size_t)T);
        for (int t = 0; t < n; t++) mark[out[t]] = 1;
        const int *rb = rblk + (size_t)(i / RAND_BLOCK) * n_rand;
        for (int e = 0; e < n_rand; e++) {
            const int j0 = rb[e] * RAND_BLOCK;
            for (int j = j0; j < j0 + RAND_BLOCK && j < T; j++)
                if (!(pad && pad[j])) mark[j] = 1;
        }
        n = 0;
        for (int j = 0; j < T; j++)
            if (mark[j]) out[n++] = j;
    }
    return n;
}

/* ------------------------------------------------------------------ */
/* One output row: softmax over N(i) of q_i . k_j / sqrt(d), weights on v. */

static void attend_row(const float *qi, const float *K, const float *V, int d,
                       const int *nb, int n, double *s, double *yi, double *lse) {
    for (int c = 0; c < d; c++) yi[c] = 0.0;
    if (lse) *lse = -INFINITY;
    if (n == 0) return;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int t = 0; t < n; t++) {
        const float *kj = K + (size_t)nb[t] * d;
        double dot = 0.0;
        for (int c = 0; c < d; c++) dot += (double)qi[c] * (double)kj[c];
        s[t] = dot * inv_sqrt_d;
        if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int t = 0; t < n; t++) {
        s[t] = exp(s[t] - m);
        l += s[t];
    }
    /* log of the softmax denominator: log sum_j exp(s_j) = m + log l */
    if (lse) *lse = m + log(l);
    for (int t = 0; t < n; t++) {
        const float *vj = V + (size_t)nb[t] * d;
        double w = s[t];
        for (int c = 0; c < d; c++) yi[c] += w * (double)vj[c];
    }
    for (int c = 0; c < d; c++) yi[c] /= l;
}

/* ------------------------------------------------------------------ */
/* Threaded driver over a list of rows. */

typedef struct {
    const float *q, *k, *v;
    int B, H, T, d, r;
    const int *rad;         /* [H] radius per head, or NULL: r for every head */
    int one_sided;
    const int *rblk;        /* [H][ceil(T/64)][n_rand] random key blocks, or NULL */
    int n_rand;
    const int *dil;
    const gset_t *G;
    const unsigned char *pad;
    const long long *rows;  /* NULL: all rows in order */
    long long n_rows;
    double *out;
    double *lse;            /* [n_rows] log-sum-exp of each row's scores, or NULL */
    int n_threads, tid;
    int err;
} job_t;

static void *worker(void *arg) {
    job_t *jb = (job_t *)arg;
    int *nb = (int *)malloc(sizeof(int) * (size_t)jb->T);
    double *s = (double *)malloc(sizeof(double) * (size_t)jb->T);
    unsigned char *mark = (unsigned char *)malloc((size_t)jb->T);
    if (!nb || !s || !mark) { jb->err = 1; free(nb); free(s); free(mark); return NULL; }
    const size_t nqb = ((size_t)jb->T + RAND_BLOCK - 1) / RAND_BLOCK;
    const long long chunk = 16;
    for (long long c0 = (long long)jb->tid * chunk; c0 < jb->n_rows;
         c0 += (long long)jb->n_threads * chunk) {
        long long c1 = c0 + chunk < jb->n_rows ? c0 + chunk : jb->n_rows;
        for (long long e = c0; e < c1; e++) {
            long long flat = jb->rows ? jb->rows[e] : e;
            long long bh = flat / jb->T;
            int i = (int)(flat % jb->T);
            int b = (int)(bh / jb->H), h = (int)(bh % jb->H);
            int delta = jb->dil ? jb->dil[h] : 1;
            int rh = jb->rad ? jb->rad[h] : jb->r;
            const unsigned char *padrow = jb->pad ? jb->pad + (size_t)b * jb->T : NULL;
            const int *rb = jb->rblk ? jb->rblk + (size_t)h * nqb * jb->n_rand : NULL;
            int n = neighbours(jb->T, rh, delta, jb->one_sided, jb->G, padrow, i, nb, rb, jb->n_rand, mark);
            const size_t base = (size_t)bh * jb->T * jb->d;
            attend_row(jb->q + base + (size_t)i * jb->d, jb->k + base, jb->v + base,
                       jb->d, nb, n, s, jb->out + (size_t)e * jb->d, jb->lse ? jb->lse + e : NULL);
        }
    }
    free(nb);
    free(s);
    free(mark);
    return NULL;
}

static int host_threads(void) {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int c = CPU_COUNT(&set);
        if (c > 0) return c;
    }
    return 1;
}

static int check_rand(int H, int T, const int *dil, const int *rblk, int n_rand) {
    if (n_rand < 0 || (n_rand > 0 && !rblk)) return -1;
    if (!rblk || n_rand == 0) return 0;
    const long long nqb = ((long long)T + RAND_BLOCK - 1) / RAND_BLOCK;
    for (int h = 0; h < H; h++) {
        if (dil && dil[h] != 1) return -1;
        for (long long e = 0; e < nqb * n_rand; e++) {
            const int x = rblk[(size_t)h * nqb * n_rand + e];
            if (x < 0 || x >= nqb) return -1;
        }
    }
    return 0;
}

static int check_args(int B, int H, int T, int d, int r, const int *rad, int one_sided, const int *dil) {
    if (B < 1 || H < 1 || T < 1 || d < 1 || r < 0) return -1;
    if (one_sided != 0 && one_sided != 1) return -1;
    if (dil)
        for (int h = 0; h < H; h++)
            if (dil[h] < 1) return -1;
    if (rad)
        for (int h = 0; h < H; h++)
            if (rad[h] < 0) return -1;
    return 0;
}

static int run(const float *q, const float *k, const float *v, int B, int H, int T, int d, int r,
               const int *rad, int one_sided, const int *rblk, int n_rand, const int *dil,
               const int *gidx, int ng, const unsigned char *pad, const long long *rows,
               long long n_rows, double *out, double *lse, int n_threads) {
    if (check_args(B, H, T, d, r, rad, one_sided, dil)) return -1;
    if (check_rand(H, T, dil, rblk, n_rand)) return -1;
    if (ng < 0 || (ng > 0 && !gidx)) return -1;
    gset_t G;
    if (gset_make(&G, gidx, ng, T)) return -1;
    if (n_threads <= 0) n_threads = host_threads();
    if ((long long)n_threads > n_rows) n_threads = n_rows > 0 ? (int)n_rows : 1;
    job_t *jobs = (job_t *)calloc((size_t)n_threads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); free(G.pos); return -1; }
    int err = 0;
    for (int t = 0; t < n_threads; t++) {
        job_t j = {q, k, v, B, H, T, d, r, rad, one_sided, rblk, n_rand, dil, &G, pad, rows, n_rows, out, lse,
                   n_threads, t, 0};
        jobs[t] = j;
    }
    for (int t = 1; t < n_threads; t++)
        if (pthread_create(&th[t], NULL, worker, &jobs[t])) { jobs[t].err = 1; th[t] = 0; }
    worker(&jobs[0]);
    for (int t = 1; t < n_threads; t++) if (th[t]) pthread_join(th[t], NULL);
    for (int t = 0; t < n_threads; t++) err |= jobs[t].err;
    free(jobs);
    free(th);
    free(G.pos);
    return err ? -1 : n_threads;
}

/* ------------------------------------------------------------------ */
/* Gradients: one thread per (b, h) at a time, so that the key-side sums of
 * a head stay in one thread. */

typedef struct {
    job_t base;             /* shapes, sets and inputs; rows unused */
    const float *dy;
    double *dq, *dk, *dv;
    long long n_bh;
} bjob_t;

/* Row i's weights P_ij = softmax_j(s_ij) over N(i), into s (in the order of
 * nb), and D_i = sum_j P_ij dP_ij with dP_ij = dy_i . v_j. */
static double row_weights(const float *qi, const float *dyi, const float *K, const float *V, int d,
                          const int *nb, int n, double *s) {
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int t = 0; t < n; t++) {
        const float *kj = K + (size_t)nb[t] * d;
        double dot = 0.0;
        for (int c = 0; c < d; c++) dot += (double)qi[c] * (double)kj[c];
        s[t] = dot * inv_sqrt_d;
        if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int t = 0; t < n; t++) {
        s[t] = exp(s[t] - m);
        l += s[t];
    }
    double D = 0.0;
    for (int t = 0; t < n; t++) {
        s[t] /= l;
        const float *vj = V + (size_t)nb[t] * d;
        double dp = 0.0;
        for (int c = 0; c < d; c++) dp += (double)dyi[c] * (double)vj[c];
        D += s[t] * dp;
    }
    return D;
}

/* dS_ij = P_ij (dP_ij - D_i) for the key at position t of row i's list. */
static double row_ds(const float *dyi, const float *V, int d, const int *nb, const double *s, double D,
                     int t) {
    const float *vj = V + (size_t)nb[t] * d;
    double dp = 0.0;
    for (int c = 0; c < d; c++) dp += (double)dyi[c] * (double)vj[c];
    return s[t] * (dp - D);
}

/* Row i's contributions: dq_i, and (when dK, dV are given) its terms of
 * dk_j and dv_j for every j in N(i). */
static void grad_row(const float *qi, const float *dyi, const float *K, const float *V, int d,
                     const int *nb, int n, double *s, double *dqi, double *dK, double *dV) {
    if (n == 0) return;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    const double D = row_weights(qi, dyi, K, V, d, nb, n, s);
    for (int t = 0; t < n; t++) {
        const int j = nb[t];
        const float *kj = K + (size_t)j * d;
        const double ds = row_ds(dyi, V, d, nb, s, D, t);
        for (int c = 0; c < d; c++) {
            dqi[c] += ds * inv_sqrt_d * (double)kj[c];
            if (dK) {
                dK[(size_t)j * d + c] += ds * inv_sqrt_d * (double)qi[c];
                dV[(size_t)j * d + c] += s[t] * (double)dyi[c];
            }
        }
    }
}

static void *bworker(void *arg) {
    bjob_t *bj = (bjob_t *)arg;
    job_t *jb = &bj->base;
    int *nb = (int *)malloc(sizeof(int) * (size_t)jb->T);
    double *s = (double *)malloc(sizeof(double) * (size_t)jb->T);
    unsigned char *mark = (unsigned char *)malloc((size_t)jb->T);
    if (!nb || !s || !mark) { jb->err = 1; free(nb); free(s); free(mark); return NULL; }
    const size_t nqb = ((size_t)jb->T + RAND_BLOCK - 1) / RAND_BLOCK;
    for (long long bh = jb->tid; bh < bj->n_bh; bh += jb->n_threads) {
        int b = (int)(bh / jb->H), h = (int)(bh % jb->H);
        int delta = jb->dil ? jb->dil[h] : 1;
        int rh = jb->rad ? jb->rad[h] : jb->r;
        const unsigned char *padrow = jb->pad ? jb->pad + (size_t)b * jb->T : NULL;
        const int *rb = jb->rblk ? jb->rblk + (size_t)h * nqb * jb->n_rand : NULL;
        const size_t base = (size_t)bh * jb->T * jb->d;
        for (size_t e = 0; e < (size_t)jb->T * jb->d; e++)
            bj->dq[base + e] = bj->dk[base + e] = bj->dv[base + e] = 0.0;
        for (int i = 0; i < jb->T; i++) {
            int n = neighbours(jb->T, rh, delta, jb->one_sided, jb->G, padrow, i, nb, rb, jb->n_rand, mark);
            grad_row(jb->q + base + (size_t)i * jb->d, bj->dy + base + (size_t)i * jb->d, jb->k + base,
                     jb->v + base, jb->d, nb, n, s, bj->dq + base + (size_t)i * jb->d, bj->dk + base,
                     bj->dv + base);
        }
    }
    free(nb);
    free(s);
    free(mark);
    return NULL;
}

/* ------------------------------------------------------------------ */
/* Gradients at chosen positions, for checks at sizes where the whole
 * gradient would take too long: dq of chosen query rows, dk and dv of chosen
 * key positions.  The arithmetic is lf_oracle_bwd's: a row's weights and dS
 * come from row_weights and row_ds, and a key's sums run over the rows i that
 * attend to it in ascending order, the order in which the whole gradient
 * adds them, so both give the same bits. */

typedef struct {
    job_t base;             /* shapes, sets and inputs; rows = the chosen positions */
    const float *dy;
    double *o1, *o2;        /* dq of the rows; or dk and dv of the keys */
    int keys;               /* 0: query rows, 1: key positions */
} sjob_t;

/* Position of key j in row i's sorted list, or -1 when j is not in N(i). */
static int find_key(const int *nb, int n, int j) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = lo + (hi - lo) / 2;
        if (nb[mid] < j) lo = mid + 1;
        else hi = mid;
    }
    return lo < n && nb[lo] == j ? lo : -1;
}

static void *sworker(void *arg) {
    sjob_t *sj = (sjob_t *)arg;
    job_t *jb = &sj->base;
    const int T = jb->T, d = jb->d;
    int *nb = (int *)malloc(sizeof(int) * (size_t)T);
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    unsigned char *mark = (unsigned char *)malloc((size_t)T);
    if (!nb || !s || !mark) { jb->err = 1; free(nb); free(s); free(mark); return NULL; }
    const size_t nqb = ((size_t)T + RAND_BLOCK - 1) / RAND_BLOCK;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    for (long long e = jb->tid; e < jb->n_rows; e += jb->n_threads) {
        const long long flat = jb->rows[e];
        const long long bh = flat / T;
        const int x = (int)(flat % T);
        const int b = (int)(bh / jb->H), h = (int)(bh % jb->H);
        const int delta = jb->dil ? jb->dil[h] : 1;
        const int rh = jb->rad ? jb->rad[h] : jb->r;
        const unsigned char *padrow = jb->pad ? jb->pad + (size_t)b * T : NULL;
        const int *rb = jb->rblk ? jb->rblk + (size_t)h * nqb * jb->n_rand : NULL;
        const size_t base = (size_t)bh * T * d;
        const float *Q = jb->q + base, *K = jb->k + base, *V = jb->v + base, *DY = sj->dy + base;
        if (!sj->keys) {
            double *dqi = sj->o1 + (size_t)e * d;
            for (int c = 0; c < d; c++) dqi[c] = 0.0;
            const int n = neighbours(T, rh, delta, jb->one_sided, jb->G, padrow, x, nb, rb, jb->n_rand, mark);
            grad_row(Q + (size_t)x * d, DY + (size_t)x * d, K, V, d, nb, n, s, dqi, NULL, NULL);
            continue;
        }
        double *dkj = sj->o1 + (size_t)e * d, *dvj = sj->o2 + (size_t)e * d;
        for (int c = 0; c < d; c++) dkj[c] = dvj[c] = 0.0;
        for (int i = 0; i < T; i++) {
            const int n = neighbours(T, rh, delta, jb->one_sided, jb->G, padrow, i, nb, rb, jb->n_rand, mark);
            const int t = find_key(nb, n, x);
            if (t < 0) continue;
            const float *qi = Q + (size_t)i * d, *dyi = DY + (size_t)i * d;
            const double D = row_weights(qi, dyi, K, V, d, nb, n, s);
            const double ds = row_ds(dyi, V, d, nb, s, D, t);
            for (int c = 0; c < d; c++) {
                dkj[c] += ds * inv_sqrt_d * (double)qi[c];
                dvj[c] += s[t] * (double)dyi[c];
            }
        }
    }
    free(nb);
    free(s);
    free(mark);
    return NULL;
}

static int srun(const float *q, const float *k, const float *v, const float *dy, int B, int H, int T, int d,
                int r, const int *rad, int one_sided, const int *rblk, int n_rand, const int *dil,
                const int *gidx, int ng, const unsigned char *pad, const long long *pos, long long n_pos,
                double *o1, double *o2, int keys, int n_threads) {
    if (check_args(B, H, T, d, r, rad, one_sided, dil)) return -1;
    if (check_rand(H, T, dil, rblk, n_rand)) return -1;
    if (ng < 0 || (ng > 0 && !gidx) || n_pos < 0 || (n_pos > 0 && !pos)) return -1;
    for (long long e = 0; e < n_pos; e++)
        if (pos[e] < 0 || pos[e] >= (long long)B * H * T) return -1;
    gset_t G;
    if (gset_make(&G, gidx, ng, T)) return -1;
    if (n_threads <= 0) n_threads = host_threads();
    if ((long long)n_threads > n_pos) n_threads = n_pos > 0 ? (int)n_pos : 1;
    sjob_t *jobs = (sjob_t *)calloc((size_t)n_threads, sizeof(sjob_t));
    pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); free(G.pos); return -1; }
    for (int t = 0; t < n_threads; t++) {
        job_t j = {q, k, v, B, H, T, d, r, rad, one_sided, rblk, n_rand, dil, &G, pad, pos, n_pos, NULL, NULL,
                   n_threads, t, 0};
        jobs[t].base = j;
        jobs[t].dy = dy;
        jobs[t].o1 = o1;
        jobs[t].o2 = o2;
        jobs[t].keys = keys;
    }
    for (int t = 1; t < n_threads; t++)
        if (pthread_create(&th[t], NULL, sworker, &jobs[t])) { jobs[t].base.err = 1; th[t] = 0; }
    sworker(&jobs[0]);
    int err = 0;
    for (int t = 1; t < n_threads; t++) if (th[t]) pthread_join(th[t], NULL);
    for (int t = 0; t < n_threads; t++) err |= jobs[t].base.err;
    free(jobs);
    free(th);
    free(G.pos);
    return err ? -1 : n_threads;
}

/* ------------------------------------------------------------------ */
/* Exported entry points (plain C ABI for ctypes). */

/* Gradients of the full forward (same arguments as lf_oracle_fwd2) for the
 * upstream gradient dy[B][H][T][d]: dq, dk, dv [B][H][T][d] in fp64.
 * Returns the thread count used, or -1 on invalid arguments. */
int lf_oracle_bwd(const float *q, const float *k, const float *v, const float *dy, int B, int H, int T,
                  int d, int r, const int *radius, int one_sided, const int *rand_blocks, int n_rand,
                  const int *dilation, const int *global_idx, int n_global,
                  const unsigned char *key_padding_mask, double *dq, double *dk, double *dv,
                  int n_threads) {
    if (check_args(B, H, T, d, r, radius, one_sided, dilation)) return -1;
    if (check_rand(H, T, dilation, rand_blocks, n_rand)) return -1;
    if (n_global < 0 || (n_global > 0 && !global_idx)) return -1;
    gset_t G;
    if (gset_make(&G, global_idx, n_global, T)) return -1;
    const long long n_bh = (long long)B * H;
    if (n_threads <= 0) n_threads = host_threads();
    if ((long long)n_threads > n_bh) n_threads = (int)n_bh;
    bjob_t *jobs = (bjob_t *)calloc((size_t)n_threads, sizeof(bjob_t));
    pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); free(G.pos); return -1; }
    for (int t = 0; t < n_threads; t++) {
        job_t j = {q, k, v, B, H, T, d, r, radius, one_sided, rand_blocks, n_rand, dilation, &G,
                   key_padding_mask, NULL, 0, NULL, NULL, n_threads, t, 0};
        jobs[t].base = j;
        jobs[t].dy = dy;
        jobs[t].dq = dq;
        jobs[t].dk = dk;
        jobs[t].dv = dv;
        jobs[t].n_bh = n_bh;
    }
    for (int t = 1; t < n_threads; t++)
        if (pthread_create(&th[t], NULL, bworker, &jobs[t])) { jobs[t].base.err = 1; th[t] = 0; }
    bworker(&jobs[0]);
    int err = 0;
    for (int t = 1; t < n_threads; t++) if (th[t]) pthread_join(th[t], NULL);
    for (int t = 0; t < n_threads; t++) err |= jobs[t].base.err;
    free(jobs);
    free(th);
    free(G.pos);
    return err ? -1 : n_threads;
}


/* dq of chosen query rows (same arguments as lf_oracle_bwd): rows[e] =
 * (b*H + h)*T + i -> dq_rows[e][d].  Returns the thread count used, or -1 on
 * invalid arguments. */
int lf_oracle_bwd_rows(const float *q, const float *k, const float *v, const float *dy, int B, int H,
                       int T, int d, int r, const int *radius, int one_sided, const int *rand_blocks,
                       int n_rand, const int *dilation, const int *global_idx, int n_global,
                       const unsigned char *key_padding_mask, const long long *rows, long long n_rows,
                       double *dq_rows, int n_threads) {
    return srun(q, k, v, dy, B, H, T, d, r, radius, one_sided, rand_blocks, n_rand, dilation, global_idx,
                n_global, key_padding_mask, rows, n_rows, dq_rows, NULL, 0, n_threads);
}

/* dk and dv of chosen key positions: keys[e] = (b*H + h)*T + j ->
 * dk_keys[e][d], dv_keys[e][d]. */
int lf_oracle_bwd_keys(const float *q, const float *k, const float *v, const float *dy, int B, int H,
                       int T, int d, int r, const int *radius, int one_sided, const int *rand_blocks,
                       int n_rand, const int *dilation, const int *global_idx, int n_global,
                       const unsigned char *key_padding_mask, const long long *keys, long long n_keys,
                       double *dk_keys, double *dv_keys, int n_threads) {
    return srun(q, k, v, dy, B, H, T, d, r, radius, one_sided, rand_blocks, n_rand, dilation, global_idx,
                n_global, key_padding_mask, keys, n_keys, dk_keys, dv_keys, 1, n_threads);
}

/* Full forward: out[B][H][T][d] in fp64.  radius: [H] per-head radii or
 * NULL (then r for every head); one_sided: 0 two-sided, 1 one-sided.
 * Returns the thread count used, or -1 on invalid arguments. */
int lf_oracle_fwd2(const float *q, const float *k, const float *v, int B, int H, int T, int d,
                   int r, const int *radius, int one_sided, const int *rand_blocks, int n_rand,
                   const int *dilation, const int *global_idx, int n_global,
                   const unsigned char *key_padding_mask, double *out, int n_threads) {
    long long n = (long long)B * H * T;
    return run(q, k, v, B, H, T, d, r, radius, one_sided, rand_blocks, n_rand, dilation, global_idx,
               n_global, key_padding_mask, NULL, n, out, NULL, n_threads);
}

/* The same forward, also writing lse[(b*H + h)*T + i] = log sum_{j in N(i)}
 * exp(q_i . k_j / sqrt(d)), the natural log of row i's softmax denominator
 * (-inf for a padded query, whose set is empty). */
int lf_oracle_fwd_lse(const float *q, const float *k, const float *v, int B, int H, int T, int d,
                      int r, const int *radius, int one_sided, const int *rand_blocks, int n_rand,
                      const int *dilation, const int *global_idx, int n_global,
                      const unsigned char *key_padding_mask, double *out, double *lse, int n_threads) {
    long long n = (long long)B * H * T;
    return run(q, k, v, B, H, T, d, r, radius, one_sided, rand_blocks, n_rand, dilation, global_idx,
               n_global, key_padding_mask, NULL, n, out, lse, n_threads);
}

int lf_oracle_fwd(const float *q, const float *k, const float *v, int B, int H, int T, int d,
                  int r, const int *dilation, const int *global_idx, int n_global,
                  const unsigned char *key_padding_mask, double *out, int n_threads) {
    return lf_oracle_fwd2(q, k, v, B, H, T, d, r, NULL, 0, NULL, 0, dilation, global_idx, n_global,
                          key_padding_mask, out, n_threads);
}

/* Selected rows only: rows[e] = (b*H + h)*T + i; out_rows[e][d]. */
int lf_oracle_rows2(const float *q, const float *k, const float *v, int B, int H, int T, int d,
                    int r, const int *radius, int one_sided, const int *rand_blocks, int n_rand,
                    const int *dilation, const int *global_idx, int n_global,
                    const unsigned char *key_padding_mask, const long long *rows, long long n_rows,
                    double *out_rows, int n_threads) {
    for (long long e = 0; e < n_rows; e++)
        if (rows[e] < 0 || rows[e] >= (long long)B * H * T) return -1;
    return run(q, k, v, B, H, T, d, r, radius, one_sided, rand_blocks, n_rand, dilation, global_idx,
               n_global, key_padding_mask, rows, n_rows, out_rows, NULL, n_threads);
}

int lf_oracle_rows(const float *q, const float *k, const float *v, int B, int H, int T, int d,
                   int r, const int *dilation, const int *global_idx, int n_global,
                   const unsigned char *key_padding_mask, const long long *rows, long long n_rows,
                   double *out_rows, int n_threads) {
    return lf_oracle_rows2(q, k, v, B, H, T, d, r, NULL, 0, NULL, 0, dilation, global_idx, n_global,
                           key_padding_mask, rows, n_rows, out_rows, n_threads);
}

/* N(i) of one query of sequence b, head radius r and stride delta: sorted
 * positions into idx (capacity T).  Returns |N(i)|, or -1 on invalid
 * arguments. */
int lf_oracle_neighbours2(int T, int r, int delta, int one_sided, const int *rand_blocks, int n_rand,
                          const int *global_idx, int n_global, const unsigned char *pad_row, int i,
                          int *idx) {
    if (T < 1 || r < 0 || delta < 1 || i < 0 || i >= T || (one_sided != 0 && one_sided != 1)) return -1;
    const int one_delta = delta;
    if (check_rand(1, T, &one_delta, rand_blocks, n_rand)) return -1;
    gset_t G;
    if (gset_make(&G, global_idx, n_global, T)) return -1;
    unsigned char *mark = (unsigned char *)malloc((size_t)T);
    if (!mark) { free(G.pos); return -1; }
    int n = neighbours(T, r, delta, one_sided, &G, pad_row, i, idx, rand_blocks, n_rand, mark);
    free(mark);
    free(G.pos);
    return n;
}

int lf_oracle_neighbours(int T, int r, int delta, const int *global_idx, int n_global,
                         const unsigned char *pad_row, int i, int *idx) {
    return lf_oracle_neighbours2(T, r, delta, 0, NULL, 0, global_idx, n_global, pad_row, i, idx);
}

/* Sum over all (b, h, i) of |N(i)|: the number of (query, key) pairs the
 * softmax runs over.  Returns -1 on invalid arguments. */
long long lf_oracle_count_pairs2(int B, int H, int T, int r, const int *radius, int one_sided,
                                 const int *rand_blocks, int n_rand, const int *dilation,
                                 const int *global_idx, int n_global,
                                 const unsigned char *key_padding_mask) {
    if (check_args(B, H, T, 1, r, radius, one_sided, dilation)) return -1;
    if (check_rand(H, T, dilation, rand_blocks, n_rand)) return -1;
    gset_t G;
    if (gset_make(&G, global_idx, n_global, T)) return -1;
    int *nb = (int *)malloc(sizeof(int) * (size_t)T);
    unsigned char *mark = (unsigned char *)malloc((size_t)T);
    if (!nb || !mark) { free(nb); free(mark); free(G.pos); return -1; }
    const size_t nqb = ((size_t)T + RAND_BLOCK - 1) / RAND_BLOCK;
    long long total = 0;
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            int delta = dilation ? dilation[h] : 1;
            int rh = radius ? radius[h] : r;
            const unsigned char *padrow = key_padding_mask ? key_padding_mask + (size_t)b * T : NULL;
            const int *rb = rand_blocks ? rand_blocks + (size_t)h * nqb * n_rand : NULL;
            for (int i = 0; i < T; i++)
                total += neighbours(T, rh, delta, one_sided, &G, padrow, i, nb, rb, n_rand, mark);
        }
    free(nb);
    free(mark);
    free(G.pos);
    return total;
}

long long lf_oracle_count_pairs(int B, int H, int T, int r, const int *dilation,
                                const int *global_idx, int n_global,
                                const unsigned char *key_padding_mask) {
    return lf_oracle_count_pairs2(B, H, T, r, NULL, 0, NULL, 0, dilation, global_idx, n_global,
                                  key_padding_mask);
}
