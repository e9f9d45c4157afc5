/*
 * hstu_ref.c -- fp64 CPU oracle for HSTU pointwise attention over jagged sequences.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's CPU-baseline leg
 * may call this code; the product path never does.  It shares no code, header or table with the
 * HIP implementation.
 *
 * What it computes (plain definitions, no tiling, no skipping, fp64 throughout):
 *
 *  HSTU spatial aggregation (page 1 "Generative recommendation: algorithm evolution to
 *  engineering", section 2.1.2, the HSTU paragraph around equation (2)): pointwise attention with
 *  a relative attention bias built from positions and timestamps, and no softmax:
 *      S_ij = alpha * <q_i, k_j> + Wp[h, bucket(|i - j|)] + Wt[h, bucket(|t_i - t_j|)]
 *      P_ij = vis(i, j) ? SiLU(S_ij) / N : 0,        O_i = sum_j P_ij v_j
 *  N is the max_seqlen argument (page 1 section 2.1.3 writes N for the maximum length).
 *
 *  Composite mask (page 2 "RecSDK supports generative recommendation", section on the HSTU
 *  acceleration operator: causal plus context/target masks; page 1 section 2.1.2, ranking task:
 *  candidates appended at the end must not interact with each other).  Per sequence of length
 *  n with num_contexts C and num_targets Tg:
 *      nc = min(C, n), nt = min(max(Tg, 0), n - nc), nh = n - nt
 *      vis(i, j) = j < nc  or  (i < nh and j <= i)  or  (i >= nh and (j < nh or j == i))
 *
 *  Bucket of a non-negative distance x (the pages call the bias "position and time" aware and
 *  give no bucketing; the reading used here is 16 exact buckets, then 4 buckets per octave,
 *  saturating at 127):
 *      bucket(x) = x                                             for x < 16
 *                = min(127, 16 + 4 (e - 4) + ((x >> (e - 2)) & 3))  with e = floor(log2 x)
 *
 *  Backward: the derivative of the definitions above, written out per pair.
 *
 *  Full layer (page 1 section 2.1.2, equations (1)-(3): pointwise projection with SiLU giving
 *  Q, K, V and a gate U; spatial aggregation; pointwise transformation gated by U; layers joined
 *  by residual connections):
 *      Z = SiLU(X W1), columns [U | V | Q | K], each head-major;  A = attention(Q, K, V)
 *      G = LayerNorm(A) * U  (per token over all H*d features, biased variance, no affine)
 *      Y = G W2 + X
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define NB 128

/* ---- definitions -------------------------------------------------------------------------- */

int hstu_ref_bucket(int64_t x) {
    if (x < 16) return (int)x;
    int e = 63 - __builtin_clzll((unsigned long long)x);
    int64_t b = 16 + 4 * (int64_t)(e - 4) + ((x >> (e - 2)) & 3);
    return b < 127 ? (int)b : 127;
}

static void seq_split(int64_t n, int64_t num_contexts, int64_t num_targets, int64_t* nc,
                      int64_t* nt, int64_t* nh) {
    *nc = num_contexts < n ? num_contexts : n;
    if (*nc < 0) *nc = 0;
    int64_t t = num_targets > 0 ? num_targets : 0;
    *nt = t < n - *nc ? t : n - *nc;
    *nh = n - *nt;
}

static int vis(int64_t i, int64_t j, int64_t nc, int64_t nh) {
    if (j < nc) return 1;
    if (i < nh) return j <= i;
    return j < nh || j == i;
}

int hstu_ref_visible(int64_t n, int64_t num_contexts, int64_t num_targets, int64_t i, int64_t j) {
    int64_t nc, nt, nh;
    seq_split(n, num_contexts, num_targets, &nc, &nt, &nh);
    if (i < 0 || j < 0 || i >= n || j >= n) return 0;
    return vis(i, j, nc, nh);
}

static int64_t absdiff64(int64_t a, int64_t b) { return a >= b ? a - b : b - a; }

typedef struct {
    int64_t B, H, dqk, dv;
    const int64_t* off;
    int64_t N;
    int64_t nc_arg;
    const int32_t* nt_arr;
    const int64_t* ts;
    const double* rp;
    const double* rt;
    double alpha;
    const double* q;
    const double* k;
    const double* v;
} prob_t;

static int64_t targets_of(const prob_t* p, int64_t b) { return p->nt_arr ? p->nt_arr[b] : 0; }

/* S_ij for absolute token rows ti = s + i and tj = s + j, head h. */
static double score(const prob_t* p, int64_t s, int64_t h, int64_t i, int64_t j) {
    const double* qi = p->q + ((s + i) * p->H + h) * p->dqk;
    const double* kj = p->k + ((s + j) * p->H + h) * p->dqk;
    double dot = 0.0;
    for (int64_t c = 0; c < p->dqk; ++c) dot += qi[c] * kj[c];
    double x = p->alpha * dot;
    if (p->rp) x += p->rp[h * NB + hstu_ref_bucket(i >= j ? i - j : j - i)];
    if (p->rt) x += p->rt[h * NB + hstu_ref_bucket(absdiff64(p->ts[s + i], p->ts[s + j]))];
    return x;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static double dot_rows(const double* a, const double* b, int64_t d);

/* ---- scheduling helper: (b, h) units, longest first --------------------------------------- */

typedef struct { int64_t n, b, h; } unit_t;

static int unit_cmp(const void* a, const void* b) {
    const unit_t* x = (const unit_t*)a;
    const unit_t* y = (const unit_t*)b;
    if (x->n != y->n) return x->n > y->n ? -1 : 1;
    if (x->b != y->b) return x->b < y->b ? -1 : 1;
    return x->h < y->h ? -1 : (x->h > y->h);
}

static unit_t* make_units(const prob_t* p) {
    unit_t* u = (unit_t*)malloc(sizeof(unit_t) * (size_t)(p->B * p->H + 1));
    for (int64_t b = 0; b < p->B; ++b)
        for (int64_t h = 0; h < p->H; ++h)
            u[b * p->H + h] = (unit_t){p->off[b + 1] - p->off[b], b, h};
    qsort(u, (size_t)(p->B * p->H), sizeof(unit_t), unit_cmp);
    return u;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* ---- forward ------------------------------------------------------------------------------ */

static void fwd_row(const prob_t* p, int64_t b, int64_t h, int64_t i, double* o) {
    int64_t s = p->off[b], n = p->off[b + 1] - s, nc, nt, nh;
    seq_split(n, p->nc_arg, targets_of(p, b), &nc, &nt, &nh);
    for (int64_t c = 0; c < p->dv; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        if (!vis(i, j, nc, nh)) continue;
        double x = score(p, s, h, i, j);
        double w = x * sigmoid(x) / (double)p->N;
        const double* vj = p->v + ((s + j) * p->H + h) * p->dv;
        for (int64_t c = 0; c < p->dv; ++c) o[c] += w * vj[c];
    }
}

void hstu_ref_attn_fwd(int64_t B, int64_t H, int64_t dqk, int64_t dv, const int64_t* off,
                       int64_t N, int64_t num_contexts, const int32_t* num_targets,
                       const int64_t* ts, const double* rab_pos, const double* rab_ts,
                       double alpha, const double* q, const double* k, const double* v,
                       double* out, int nthreads) {
    prob_t p = {B, H, dqk, dv, off, N, num_contexts, num_targets, ts, rab_pos, rab_ts, alpha,
                q, k, v};
    unit_t* u = make_units(&p);
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t x = 0; x < B * H; ++x) {
        int64_t b = u[x].b, h = u[x].h, s = off[b], n = off[b + 1] - s;
        for (int64_t i = 0; i < n; ++i) fwd_row(&p, b, h, i, out + ((s + i) * H + h) * dv);
    }
    free(u);
}

static int64_t seq_of(const int64_t* off, int64_t B, int64_t tok) {
    int64_t lo = 0, hi = B - 1;  /* last b with off[b] <= tok and a non-empty sequence */
    while (lo < hi) {
        int64_t mid = (lo + hi + 1) / 2;
        if (off[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* Forward for selected (token, head) rows only: out_rows is nrows x dv. */
void hstu_ref_attn_fwd_rows(int64_t B, int64_t H, int64_t dqk, int64_t dv, const int64_t* off,
                            int64_t N, int64_t num_contexts, const int32_t* num_targets,
                            const int64_t* ts, const double* rab_pos, const double* rab_ts,
                            double alpha, const double* q, const double* k, const double* v,
                            int64_t nrows, const int64_t* row_tok, const int64_t* row_head,
                            double* out_rows, int nthreads) {
    prob_t p = {B, H, dqk, dv, off, N, num_contexts, num_targets, ts, rab_pos, rab_ts, alpha,
                q, k, v};
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t b = seq_of(off, B, row_tok[r]);
        fwd_row(&p, b, row_head[r], row_tok[r] - off[b], out_rows + r * dv);
    }
}

/* ---- candidate scoring against cached history -------------------------------------------- */

/* Ranking with a key/value cache (page 2 "RecSDK supports generative recommendation", HSTU
 * acceleration operator: KV-cache support; page 1 section 2.1.2, ranking: candidates appended
 * after the history see the whole history and themselves, never each other).  User b has nh
 * history tokens held in the cache (rows cache_off[b] .. cache_off[b + 1] of kc / vc, positions
 * 0 .. nh - 1, times ts_cache) and m candidates (rows cand_off[b] .. of q / k / v, positions
 * nh + c, times ts_cand).  For candidate c and head h:
 *     S_cj = alpha <q_c, k_j> + Wp[h, bucket(nh + c - j)] + Wt[h, bucket(|t_c - t_j|)]  (j < nh)
 *     S_cc = alpha <q_c, k_c> + Wp[h, bucket(0)] + Wt[h, bucket(0)]
 *     O_c  = sum_{j < nh} SiLU(S_cj) / N v_j + SiLU(S_cc) / N v_c
 * These are the candidate rows of the full forward over [history | candidates] with the
 * candidates as targets.  out is (T_cand, H, d). */
void hstu_ref_attn_fwd_cached(int64_t B, int64_t H, int64_t d, const int64_t* cand_off,
                              const int64_t* cache_off, int64_t N, const int64_t* ts_cand,
                              const int64_t* ts_cache, const double* rab_pos,
                              const double* rab_ts, double alpha, const double* q,
                              const double* k, const double* v, const double* kc,
                              const double* vc, double* out, int nthreads) {
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t x = 0; x < B * H; ++x) {
        int64_t b = x / H, h = x % H;
        int64_t s = cand_off[b], m = cand_off[b + 1] - s;
        int64_t sc = cache_off[b], nh = cache_off[b + 1] - sc;
        for (int64_t c = 0; c < m; ++c) {
            const double* qc = q + ((s + c) * H + h) * d;
            double* o = out + ((s + c) * H + h) * d;
            for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
            for (int64_t j = 0; j <= nh; ++j) {  /* j == nh stands for the candidate itself */
                int self = j == nh;
                const double* kj = self ? k + ((s + c) * H + h) * d : kc + ((sc + j) * H + h) * d;
                const double* vj = self ? v + ((s + c) * H + h) * d : vc + ((sc + j) * H + h) * d;
                double xs = alpha * dot_rows(qc, kj, d);
                if (rab_pos) xs += rab_pos[h * NB + hstu_ref_bucket(self ? 0 : nh + c - j)];
                if (rab_ts)
                    xs += rab_ts[h * NB + hstu_ref_bucket(self ? 0 : absdiff64(ts_cand[s + c], ts_cache[sc + j]))];
                double w = xs * sigmoid(xs) / (double)N;
                for (int64_t e = 0; e < d; ++e) o[e] += w * vj[e];
            }
        }
    }
}

/* ---- backward ----------------------------------------------------------------------------- */

/* d/dS of SiLU(S)/N, times dP. */
static double dscore(double x, double dp, double N) {
    double sg = sigmoid(x);
    return dp * sg * (1.0 + x * (1.0 - sg)) / N;
}

static double dot_rows(const double* a, const double* b, int64_t d) {
    double r = 0.0;
    for (int64_t c = 0; c < d; ++c) r += a[c] * b[c];
    return r;
}

/* Full backward.  dq, dk, dv are (T, H, d) and are overwritten.  drab_pos / drab_ts are (H, 128),
 * overwritten, may be NULL.  Per (b, h) partial bias gradients are reduced in (b, h) order so the
 * result does not depend on the thread count. */
void hstu_ref_attn_bwd(int64_t B, int64_t H, int64_t dqk, int64_t dv, const int64_t* off,
                       int64_t N, int64_t num_contexts, const int32_t* num_targets,
                       const int64_t* ts, const double* rab_pos, const double* rab_ts,
                       double alpha, const double* q, const double* k, const double* v,
                       const double* dout, double* dq, double* dk, double* dvv, double* drab_pos,
                       double* drab_ts, int nthreads) {
    prob_t p = {B, H, dqk, dv, off, N, num_contexts, num_targets, ts, rab_pos, rab_ts, alpha,
                q, k, v};
    int64_t T = off[B];
    memset(dq, 0, sizeof(double) * (size_t)(T * H * dqk));
    memset(dk, 0, sizeof(double) * (size_t)(T * H * dqk));
    memset(dvv, 0, sizeof(double) * (size_t)(T * H * dv));
    double* part = (double*)calloc((size_t)(B * H * 2 * NB + 1), sizeof(double));
    unit_t* u = make_units(&p);
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t x = 0; x < B * H; ++x) {
        int64_t b = u[x].b, h = u[x].h, s = off[b], n = off[b + 1] - s, nc, nt, nh;
        seq_split(n, num_contexts, targets_of(&p, b), &nc, &nt, &nh);
        double* gp = part + (b * H + h) * 2 * NB;
        double* gt = gp + NB;
        for (int64_t i = 0; i < n; ++i) {
            const double* qi = q + ((s + i) * H + h) * dqk;
            const double* doi = dout + ((s + i) * H + h) * dv;
            double* dqi = dq + ((s + i) * H + h) * dqk;
            for (int64_t j = 0; j < n; ++j) {
                if (!vis(i, j, nc, nh)) continue;
                const double* kj = k + ((s + j) * H + h) * dqk;
                const double* vj = v + ((s + j) * H + h) * dv;
                double* dkj = dk + ((s + j) * H + h) * dqk;
                double* dvj = dvv + ((s + j) * H + h) * dv;
                double xs = score(&p, s, h, i, j);
                double w = xs * sigmoid(xs) / (double)N;
                double dp = dot_rows(doi, vj, dv);
                double ds = dscore(xs, dp, (double)N);
                for (int64_t c = 0; c < dv; ++c) dvj[c] += w * doi[c];
                for (int64_t c = 0; c < dqk; ++c) {
                    dqi[c] += alpha * ds * kj[c];
                    dkj[c] += alpha * ds * qi[c];
                }
                gp[hstu_ref_bucket(i >= j ? i - j : j - i)] += ds;
                if (ts) gt[hstu_ref_bucket(absdiff64(ts[s + i], ts[s + j]))] += ds;
            }
        }
    }
    if (drab_pos) memset(drab_pos, 0, sizeof(double) * (size_t)(H * NB));
    if (drab_ts) memset(drab_ts, 0, sizeof(double) * (size_t)(H * NB));
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t e = 0; e < NB; ++e) {
                if (drab_pos && rab_pos) drab_pos[h * NB + e] += part[(b * H + h) * 2 * NB + e];
                if (drab_ts && rab_ts) drab_ts[h * NB + e] += part[(b * H + h) * 2 * NB + NB + e];
            }
    free(part);
    free(u);
}

/* Backward for selected rows: dq of the rows as queries, dk and dv of the rows as keys.
 * Each output is nrows x d. */
void hstu_ref_attn_bwd_rows(int64_t B, int64_t H, int64_t dqk, int64_t dv, const int64_t* off,
                            int64_t N, int64_t num_contexts, const int32_t* num_targets,
                            const int64_t* ts, const double* rab_pos, const double* rab_ts,
                            double alpha, const double* q, const double* k, const double* v,
                            const double* dout, int64_t nrows, const int64_t* row_tok,
                            const int64_t* row_head, double* dq_rows, double* dk_rows,
                            double* dv_rows, int nthreads) {
    prob_t p = {B, H, dqk, dv, off, N, num_contexts, num_targets, ts, rab_pos, rab_ts, alpha,
                q, k, v};
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t b = seq_of(off, B, row_tok[r]), h = row_head[r];
        int64_t s = off[b], n = off[b + 1] - s, nc, nt, nh;
        int64_t m = row_tok[r] - s;
        seq_split(n, num_contexts, targets_of(&p, b), &nc, &nt, &nh);
        double* gq = dq_rows + r * dqk;
        double* gk = dk_rows + r * dqk;
        double* gv = dv_rows + r * dv;
        for (int64_t c = 0; c < dqk; ++c) gq[c] = gk[c] = 0.0;
        for (int64_t c = 0; c < dv; ++c) gv[c] = 0.0;
        /* row m as a query */
        const double* dom = dout + ((s + m) * H + h) * dv;
        for (int64_t j = 0; j < n; ++j) {
            if (!vis(m, j, nc, nh)) continue;
            const double* vj = v + ((s + j) * H + h) * dv;
            const double* kj = k + ((s + j) * H + h) * dqk;
            double xs = score(&p, s, h, m, j);
            double ds = dscore(xs, dot_rows(dom, vj, dv), (double)N);
            for (int64_t c = 0; c < dqk; ++c) gq[c] += alpha * ds * kj[c];
        }
        /* row m as a key */
        const double* vm = v + ((s + m) * H + h) * dv;
        for (int64_t i = 0; i < n; ++i) {
            if (!vis(i, m, nc, nh)) continue;
            const double* qi = q + ((s + i) * H + h) * dqk;
            const double* doi = dout + ((s + i) * H + h) * dv;
            double xs = score(&p, s, h, i, m);
            double w = xs * sigmoid(xs) / (double)N;
            double ds = dscore(xs, dot_rows(doi, vm, dv), (double)N);
            for (int64_t c = 0; c < dv; ++c) gv[c] += w * doi[c];
            for (int64_t c = 0; c < dqk; ++c) gk[c] += alpha * ds * qi[c];
        }
    }
}

/* ---- full layer --------------------------------------------------------------------------- */

/* x (T, D), w1 (D, 4*H*d), w2 (H*d, D), y (T, D).  attn_out (T, H*d) may be NULL; if given it
 * receives the attention output A before the LayerNorm. */
void hstu_ref_layer_fwd(int64_t B, int64_t H, int64_t d, int64_t D, const int64_t* off, int64_t N,
                        int64_t num_contexts, const int32_t* num_targets, const int64_t* ts,
                        const double* rab_pos, const double* rab_ts, double alpha,
                        const double* x, const double* w1, const double* w2, double eps,
                        double* y, double* attn_out, int nthreads) {
    int64_t T = off[B], Hd = H * d, W = 4 * Hd;
    double* z = (double*)malloc(sizeof(double) * (size_t)(T * W + 1));
    double* u = (double*)malloc(sizeof(double) * (size_t)(T * Hd + 1));
    double* qq = (double*)malloc(sizeof(double) * (size_t)(T * Hd + 1));
    double* kk = (double*)malloc(sizeof(double) * (size_t)(T * Hd + 1));
    double* vv = (double*)malloc(sizeof(double) * (size_t)(T * Hd + 1));
    double* a = (double*)malloc(sizeof(double) * (size_t)(T * Hd + 1));
    set_threads(nthreads);
    /* Z = SiLU(X W1) */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* zt = z + t * W;
        for (int64_t c = 0; c < W; ++c) zt[c] = 0.0;
        for (int64_t e = 0; e < D; ++e) {
            double xe = x[t * D + e];
            const double* wr = w1 + e * W;
            for (int64_t c = 0; c < W; ++c) zt[c] += xe * wr[c];
        }
        for (int64_t c = 0; c < W; ++c) zt[c] = zt[c] * sigmoid(zt[c]);
        for (int64_t c = 0; c < Hd; ++c) {
            u[t * Hd + c] = zt[c];
            vv[t * Hd + c] = zt[Hd + c];
            qq[t * Hd + c] = zt[2 * Hd + c];
            kk[t * Hd + c] = zt[3 * Hd + c];
        }
    }
    hstu_ref_attn_fwd(B, H, d, d, off, N, num_contexts, num_targets, ts, rab_pos, rab_ts, alpha,
                      qq, kk, vv, a, nthreads);
    if (attn_out) memcpy(attn_out, a, sizeof(double) * (size_t)(T * Hd));
    /* G = LayerNorm(A) * U, then Y = G W2 + X */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* at = a + t * Hd;
        double mean = 0.0, var = 0.0;
        for (int64_t c = 0; c < Hd; ++c) mean += at[c];
        mean /= (double)Hd;
        for (int64_t c = 0; c < Hd; ++c) var += (at[c] - mean) * (at[c] - mean);
        var /= (double)Hd;
        double rstd = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < Hd; ++c) at[c] = (at[c] - mean) * rstd * u[t * Hd + c];
        double* yt = y + t * D;
        for (int64_t c = 0; c < D; ++c) yt[c] = x[t * D + c];
        for (int64_t e = 0; e < Hd; ++e) {
            double g = at[e];
            const double* wr = w2 + e * D;
            for (int64_t c = 0; c < D; ++c) yt[c] += g * wr[c];
        }
    }
    free(z); free(u); free(qq); free(kk); free(vv); free(a);
}

/* Layer backward: gradients of sum(dy * Y) for Y = layer_fwd(x, w1, w2), by the chain rule through
 * the steps of the forward in reverse (page 1 section 2.1.2, equations (1)-(3)):
 *   H = X W1, Z = SiLU(H) = [U | V | Q | K], A = attention(Q, K, V),
 *   xh = (A - mean) / sqrt(var + eps) per token, G = xh * U, Y = G W2 + X.
 * Backward:
 *   dW2 = G^T dy,  dG = dy W2^T,  dU = dG * xh,  dxh = dG * U,
 *   dA = (dxh - mean(dxh) - xh * mean(dxh * xh)) / sqrt(var + eps)      (per token, over H*d)
 *   (dQ, dK, dV, d rab) = attention backward with dout = dA,
 *   dH = [dU | dV | dQ | dK] * SiLU'(H),  SiLU'(h) = s (1 + h (1 - s)), s = sigmoid(h),
 *   dW1 = X^T dH,  dX = dy + dH W1^T.
 * Outputs: dx (T x D), dw1 (D x 4Hd), dw2 (Hd x D); drab_* (H x 128) when the table is given. */
void hstu_ref_layer_bwd(int64_t B, int64_t H, int64_t d, int64_t D, const int64_t* off, int64_t N,
                        int64_t num_contexts, const int32_t* num_targets, const int64_t* ts,
                        const double* rab_pos, const double* rab_ts, double alpha,
                        const double* x, const double* w1, const double* w2, const double* dy,
                        double eps, double* dx, double* dw1, double* dw2, double* drab_pos,
                        double* drab_ts, int nthreads) {
    int64_t T = off[B], Hd = H * d, W = 4 * Hd;
    size_t nz = (size_t)(T * W + 1), na = (size_t)(T * Hd + 1);
    double* hpre = (double*)malloc(sizeof(double) * nz);
    double* u = (double*)malloc(sizeof(double) * na);
    double* qq = (double*)malloc(sizeof(double) * na);
    double* kk = (double*)malloc(sizeof(double) * na);
    double* vv = (double*)malloc(sizeof(double) * na);
    double* a = (double*)malloc(sizeof(double) * na);
    double* xh = (double*)malloc(sizeof(double) * na);
    double* rstd = (double*)malloc(sizeof(double) * (size_t)(T + 1));
    double* g = (double*)malloc(sizeof(double) * na);
    double* da = (double*)malloc(sizeof(double) * na);
    double* du = (double*)malloc(sizeof(double) * na);
    double* dq = (double*)malloc(sizeof(double) * na);
    double* dk = (double*)malloc(sizeof(double) * na);
    double* dv = (double*)malloc(sizeof(double) * na);
    double* dh = (double*)malloc(sizeof(double) * nz);
    set_threads(nthreads);
    /* forward, keeping H (before SiLU), xh and 1/sqrt(var + eps) */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* ht = hpre + t * W;
        for (int64_t c = 0; c < W; ++c) ht[c] = 0.0;
        for (int64_t e = 0; e < D; ++e) {
            double xe = x[t * D + e];
            const double* wr = w1 + e * W;
            for (int64_t c = 0; c < W; ++c) ht[c] += xe * wr[c];
        }
        for (int64_t c = 0; c < Hd; ++c) {
            u[t * Hd + c] = ht[c] * sigmoid(ht[c]);
            vv[t * Hd + c] = ht[Hd + c] * sigmoid(ht[Hd + c]);
            qq[t * Hd + c] = ht[2 * Hd + c] * sigmoid(ht[2 * Hd + c]);
            kk[t * Hd + c] = ht[3 * Hd + c] * sigmoid(ht[3 * Hd + c]);
        }
    }
    hstu_ref_attn_fwd(B, H, d, d, off, N, num_contexts, num_targets, ts, rab_pos, rab_ts, alpha,
                      qq, kk, vv, a, nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* at = a + t * Hd;
        double mean = 0.0, var = 0.0;
        for (int64_t c = 0; c < Hd; ++c) mean += at[c];
        mean /= (double)Hd;
        for (int64_t c = 0; c < Hd; ++c) var += (at[c] - mean) * (at[c] - mean);
        var /= (double)Hd;
        rstd[t] = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < Hd; ++c) {
            xh[t * Hd + c] = (at[c] - mean) * rstd[t];
            g[t * Hd + c] = xh[t * Hd + c] * u[t * Hd + c];
        }
    }
    /* dW2 = G^T dy (rows of W2 independent) */
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < Hd; ++e) {
        double* wr = dw2 + e * D;
        for (int64_t c = 0; c < D; ++c) wr[c] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double ge = g[t * Hd + e];
            for (int64_t c = 0; c < D; ++c) wr[c] += ge * dy[t * D + c];
        }
    }
    /* dG = dy W2^T, then the gate and LayerNorm backward, per token */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* dxh = da + t * Hd;  /* dxh first, turned into dA in place */
        double m1 = 0.0, m2 = 0.0;
        for (int64_t e = 0; e < Hd; ++e) {
            double dg = 0.0;
            for (int64_t c = 0; c < D; ++c) dg += dy[t * D + c] * w2[e * D + c];
            du[t * Hd + e] = dg * xh[t * Hd + e];
            dxh[e] = dg * u[t * Hd + e];
            m1 += dxh[e];
            m2 += dxh[e] * xh[t * Hd + e];
        }
        m1 /= (double)Hd;
        m2 /= (double)Hd;
        for (int64_t e = 0; e < Hd; ++e) dxh[e] = (dxh[e] - m1 - xh[t * Hd + e] * m2) * rstd[t];
    }
    hstu_ref_attn_bwd(B, H, d, d, off, N, num_contexts, num_targets, ts, rab_pos, rab_ts, alpha,
                      qq, kk, vv, da, dq, dk, dv, drab_pos, drab_ts, nthreads);
    /* dH = [dU | dV | dQ | dK] * SiLU'(H) */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t c = 0; c < W; ++c) {
            int64_t blk = c / Hd, e = c % Hd;
            double dz = blk == 0 ? du[t * Hd + e] : blk == 1 ? dv[t * Hd + e]
                      : blk == 2 ? dq[t * Hd + e] : dk[t * Hd + e];
            double h = hpre[t * W + c], s = sigmoid(h);
            dh[t * W + c] = dz * s * (1.0 + h * (1.0 - s));
        }
    }
    /* dW1 = X^T dH */
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < D; ++e) {
        double* wr = dw1 + e * W;
        for (int64_t c = 0; c < W; ++c) wr[c] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double xe = x[t * D + e];
            for (int64_t c = 0; c < W; ++c) wr[c] += xe * dh[t * W + c];
        }
    }
    /* dX = dy + dH W1^T */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t e = 0; e < D; ++e) {
            double acc = dy[t * D + e];
            for (int64_t c = 0; c < W; ++c) acc += dh[t * W + c] * w1[e * W + c];
            dx[t * D + e] = acc;
        }
    free(hpre); free(u); free(qq); free(kk); free(vv); free(a); free(xh); free(rstd); free(g);
    free(da); free(du); free(dq); free(dk); free(dv); free(dh);
}

/* ---- counting ----------------------------------------------------------------------------- */

/* Number of visible (i, j) pairs of the batch for one head, by enumerating vis(). */
int64_t hstu_ref_count_pairs(int64_t B, const int64_t* off, int64_t num_contexts,
                             const int32_t* num_targets) {
    int64_t total = 0;
    for (int64_t b = 0; b < B; ++b) {
        int64_t n = off[b + 1] - off[b], nc, nt, nh;
        seq_split(n, num_contexts, num_targets ? num_targets[b] : 0, &nc, &nt, &nh);
        for (int64_t i = 0; i < n; ++i)
            for (int64_t j = 0; j < n; ++j) total += vis(i, j, nc, nh);
    }
    return total;
}

int hstu_ref_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
