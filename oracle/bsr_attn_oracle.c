/*
 * Oracle for block-sparse (BSR) softmax attention, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path never
 * calls it and shares no code with it.
 *
 * Plain, slow, obviously correct: every value is computed in fp64 straight
 * from the definition of masked softmax attention and its exact gradient, one
 * query row at a time, with no tiling, fusion or reordering.
 *
 * What is computed (sources: the two trnsparse release-diff pages,
 * "trnsparse 0.7.0 -> 0.9.0" and "trnsparse 0.4.1 -> 0.6.0"):
 *
 *  - The mask is block-granular: query row r attends to every key c whose
 *    128-wide key block is a stored block of r's block row. The attention
 *    benchmark builds its dense reference by expanding the block mask by the
 *    block size on both axes and running dense softmax attention with that
 *    boolean mask ("trnsparse 0.7.0 -> 0.9.0", benchmarks/bench_native_trn2.py,
 *    attention section).
 *  - s_rc = scale * <q_r, k_c>;  m_r = max_c s_rc;  l_r = sum_c exp(s_rc - m_r);
 *    P_rc = exp(s_rc - m_r) / l_r;  O_r = sum_c P_rc v_c.  The row statistics
 *    m (row_max) and l (row_denom) are the ones the forward returns
 *    ("trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.4.3 and 0.4.4: per-row max and
 *    sum-of-exponentials, then a stable softmax; CHANGELOG 0.5.1:
 *    return_stats gives (out, row_max, row_denom)).
 *  - Backward with the delta identity D_r = <dO_r, O_r>
 *    ("trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.5.0):
 *    dP_rc = <dO_r, v_c>;  dS_rc = P_rc (dP_rc - D_r);
 *    dQ_r = scale * sum_c dS_rc k_c;  dK_c = scale * sum_r dS_rc q_r;
 *    dV_c = sum_r P_rc dO_r  ("trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.5.1:
 *    dQ row-first, dK/dV column-first over the transposed structure).
 *  - A block row with no stored block has O = 0, row_max = -inf,
 *    row_denom = 0 and dQ = 0; keys no row attends to get dK = dV = 0
 *    (a reading: the pages never build such a structure).
 *
 * Layout: q, k, v, dout, o, dq, dk, dv are [BH][S][D] row-major doubles
 * (BH = batch * heads); row_max, row_denom are [BH][S]. The structure
 * (row_ptr[nb + 1], col_idx[nnzb], block size b, S = nb * b) is shared by
 * every (batch, head). Inputs are not validated beyond what the loops need;
 * the caller passes a well-formed structure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t BH, S, D, b, nb;
    const int32_t *row_ptr, *col_idx;
    double scale;
    const double *q, *k, *v, *dout;
} problem;

/* Everything the definition gives for one query row. */
typedef struct {
    int64_t n;       /* number of keys attended, |C(r)| */
    int64_t *keys;   /* the attended key indices, ascending */
    double *p;       /* P_rc for those keys */
    double *ds;      /* dS_rc for those keys (backward only) */
    double m, l, delta;
    double *o;       /* O_r, length D */
} row_result;

static void row_alloc(row_result *rr, int64_t S, int64_t D) {
    rr->keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)S);
    rr->p = (double *)malloc(sizeof(double) * (size_t)S);
    rr->ds = (double *)malloc(sizeof(double) * (size_t)S);
    rr->o = (double *)malloc(sizeof(double) * (size_t)D);
}

static void row_free(row_result *rr) {
    free(rr->keys); free(rr->p); free(rr->ds); free(rr->o);
}

static double dot(const double *a, const double *b, int64_t D) {
    double s = 0.0;
    for (int64_t d = 0; d < D; ++d) s += a[d] * b[d];
    return s;
}

/* Query row r of (batch, head) bh: scores, softmax, output and, when the
 * problem carries dout, the delta and dS of that row. */
static void row_pass(const problem *pb, int64_t bh, int64_t r, row_result *rr) {
    const int64_t S = pb->S, D = pb->D, b = pb->b;
    const double *qr = pb->q + (bh * S + r) * D;
    const double *kb = pb->k + bh * S * D;
    const double *vb = pb->v + bh * S * D;
    const int64_t I = r / b;

    rr->n = 0;
    for (int32_t p = pb->row_ptr[I]; p < pb->row_ptr[I + 1]; ++p) {
        const int64_t J = pb->col_idx[p];
        for (int64_t c = J * b; c < (J + 1) * b; ++c) rr->keys[rr->n++] = c;
    }
    for (int64_t d = 0; d < D; ++d) rr->o[d] = 0.0;
    if (rr->n == 0) {
        rr->m = -INFINITY; rr->l = 0.0; rr->delta = 0.0;
        return;
    }
    /* scores s_rc, kept in p[] until normalised */
    double m = -INFINITY;
    for (int64_t i = 0; i < rr->n; ++i) {
        const double s = pb->scale * dot(qr, kb + rr->keys[i] * D, D);
        rr->p[i] = s;
        if (s > m) m = s;
    }
    double l = 0.0;
    for (int64_t i = 0; i < rr->n; ++i) l += exp(rr->p[i] - m);
    for (int64_t i = 0; i < rr->n; ++i) rr->p[i] = exp(rr->p[i] - m) / l;
    for (int64_t i = 0; i < rr->n; ++i) {
        const double *vc = vb + rr->keys[i] * D;
        for (int64_t d = 0; d < D; ++d) rr->o[d] += rr->p[i] * vc[d];
    }
    rr->m = m;
    rr->l = l;
    if (!pb->dout) return;
    const double *dor = pb->dout + (bh * S + r) * D;
    rr->delta = dot(dor, rr->o, D);
    for (int64_t i = 0; i < rr->n; ++i) {
        const double dp = dot(dor, vb + rr->keys[i] * D, D);
        rr->ds[i] = rr->p[i] * (dp - rr->delta);
    }
}

/* Is key block J attended by query block I? (own scan of the BSR row) */
static int block_stored(const problem *pb, int64_t I, int64_t J) {
    for (int32_t p = pb->row_ptr[I]; p < pb->row_ptr[I + 1]; ++p)
        if (pb->col_idx[p] == J) return 1;
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Forward over every (bh, row): O, row_max, row_denom. */
void oracle_fwd(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb,
                const int32_t *row_ptr, const int32_t *col_idx, double scale,
                const double *q, const double *k, const double *v,
                double *o, double *row_max, double *row_denom) {
    problem pb = {BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, NULL};
    #pragma omp parallel
    {
        row_result rr;
        row_alloc(&rr, S, D);
        #pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < BH * S; ++t) {
            const int64_t bh = t / S, r = t % S;
            row_pass(&pb, bh, r, &rr);
            memcpy(o + t * D, rr.o, sizeof(double) * (size_t)D);
            row_max[t] = rr.m;
            row_denom[t] = rr.l;
        }
        row_free(&rr);
    }
}

/* Forward for a list of flat rows t = bh * S + r only. */
void oracle_fwd_rows(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb,
                     const int32_t *row_ptr, const int32_t *col_idx, double scale,
                     const double *q, const double *k, const double *v,
                     int64_t n_rows, const int64_t *rows,
                     double *o, double *row_max, double *row_denom) {
    problem pb = {BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, NULL};
    #pragma omp parallel
    {
        row_result rr;
        row_alloc(&rr, S, D);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            const int64_t t = rows[i];
            row_pass(&pb, t / S, t % S, &rr);
            memcpy(o + i * D, rr.o, sizeof(double) * (size_t)D);
            row_max[i] = rr.m;
            row_denom[i] = rr.l;
        }
        row_free(&rr);
    }
}

/* Backward over everything: dq, dk, dv (each [BH][S][D]). dK/dV are gathered
 * per key: for key c, every query row whose block row stores c's block. */
void oracle_bwd(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb,
                const int32_t *row_ptr, const int32_t *col_idx, double scale,
                const double *q, const double *k, const double *v, const double *dout,
                double *dq, double *dk, double *dv) {
    problem pb = {BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, dout};
    const double *kall = k, *qall = q;
    /* dQ, row by row */
    #pragma omp parallel
    {
        row_result rr;
        row_alloc(&rr, S, D);
        #pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < BH * S; ++t) {
            const int64_t bh = t / S, r = t % S;
            row_pass(&pb, bh, r, &rr);
            double *dqr = dq + t * D;
            for (int64_t d = 0; d < D; ++d) dqr[d] = 0.0;
            for (int64_t i = 0; i < rr.n; ++i) {
                const double *kc = kall + (bh * S + rr.keys[i]) * D;
                for (int64_t d = 0; d < D; ++d) dqr[d] += scale * rr.ds[i] * kc[d];
            }
        }
        row_free(&rr);
    }
    /* dK, dV, key block by key block: every query row of every block row
     * that stores this key block contributes, in ascending row order. */
    #pragma omp parallel
    {
        row_result rr;
        row_alloc(&rr, S, D);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < BH * nb; ++u) {
            const int64_t bh = u / nb, J = u % nb;
            double *dkb = dk + (bh * S + J * b) * D;
            double *dvb = dv + (bh * S + J * b) * D;
            for (int64_t x = 0; x < b * D; ++x) { dkb[x] = 0.0; dvb[x] = 0.0; }
            for (int64_t I = 0; I < nb; ++I) {
                if (!block_stored(&pb, I, J)) continue;
                for (int64_t r = I * b; r < (I + 1) * b; ++r) {
                    row_pass(&pb, bh, r, &rr);
                    const double *qr = qall + (bh * S + r) * D;
                    const double *dor = dout + (bh * S + r) * D;
                    for (int64_t i = 0; i < rr.n; ++i) {
                        const int64_t c = rr.keys[i];
                        if (c / b != J) continue;
                        double *dkc = dkb + (c - J * b) * D;
                        double *dvc = dvb + (c - J * b) * D;
                        for (int64_t d = 0; d < D; ++d) {
                            dkc[d] += scale * rr.ds[i] * qr[d];
                            dvc[d] += rr.p[i] * dor[d];
                        }
                    }
                }
            }
        }
        row_free(&rr);
    }
}

/* dQ for a list of flat query rows t = bh * S + r. */
void oracle_bwd_rows(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb,
                     const int32_t *row_ptr, const int32_t *col_idx, double scale,
                     const double *q, const double *k, const double *v, const double *dout,
                     int64_t n_rows, const int64_t *rows, double *dq) {
    problem pb = {BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, dout};
    #pragma omp parallel
    {
        row_result rr;
        row_alloc(&rr, S, D);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            const int64_t t = rows[i], bh = t / S;
            row_pass(&pb, bh, t % S, &rr);
            double *dqr = dq + i * D;
            for (int64_t d = 0; d < D; ++d) dqr[d] = 0.0;
            for (int64_t j = 0; j < rr.n; ++j) {
                const double *kc = k + (bh * S + rr.keys[j]) * D;
                for (int64_t d = 0; d < D; ++d) dqr[d] += scale * rr.ds[j] * kc[d];
            }
        }
        row_free(&rr);
    }
}

/* dK and dV for a list of flat keys t = bh * S + c. Every query row that
 * attends to c contributes; rows are visited in ascending order and their
 * contributions summed in that order. */
void oracle_bwd_cols(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb,
                     const int32_t *row_ptr, const int32_t *col_idx, double scale,
                     const double *q, const double *k, const double *v, const double *dout,
                     int64_t n_cols, const int64_t *cols, double *dk, double *dv) {
    problem pb = {BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, dout};
    for (int64_t i = 0; i < n_cols; ++i) {
        const int64_t t = cols[i], bh = t / S, c = t % S, J = c / b;
        double *dkc = dk + i * D, *dvc = dv + i * D;
        /* per query row contributions, computed in parallel, summed in order */
        double *ck = (double *)calloc((size_t)(S * D), sizeof(double));
        double *cv = (double *)calloc((size_t)(S * D), sizeof(double));
        unsigned char *hit = (unsigned char *)calloc((size_t)S, 1);
        #pragma omp parallel
        {
            row_result rr;
            row_alloc(&rr, S, D);
            #pragma omp for schedule(dynamic, 8)
            for (int64_t r = 0; r < S; ++r) {
                if (!block_stored(&pb, r / b, J)) continue;
                row_pass(&pb, bh, r, &rr);
                const double *qr = q + (bh * S + r) * D;
                const double *dor = dout + (bh * S + r) * D;
                for (int64_t j = 0; j < rr.n; ++j) {
                    if (rr.keys[j] != c) continue;
                    for (int64_t d = 0; d < D; ++d) {
                        ck[r * D + d] = scale * rr.ds[j] * qr[d];
                        cv[r * D + d] = rr.p[j] * dor[d];
                    }
                    hit[r] = 1;
                }
            }
            row_free(&rr);
        }
        for (int64_t d = 0; d < D; ++d) { dkc[d] = 0.0; dvc[d] = 0.0; }
        for (int64_t r = 0; r < S; ++r) {
            if (!hit[r]) continue;
            for (int64_t d = 0; d < D; ++d) { dkc[d] += ck[r * D + d]; dvc[d] += cv[r * D + d]; }
        }
        free(ck); free(cv); free(hit);
    }
}

/*
 * Block-sparse times dense (the pages' other operation on the same BSR
 * structure; page "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.8.0: bsr_spmm
 * walks exactly the stored blocks and addresses B by block column).
 *
 * A is given by its stored b x b blocks in BSR order (blocks[p] is the block
 * at (block row of p, col_idx[p]), row-major); B is dense [nb*b, n]
 * row-major; C is dense [nb*b, n]:
 *   C[i][j] = sum over stored blocks (I = i / b, J) of
 *             sum_k A_IJ[i - I*b][k] * B[J*b + k][j].
 * A block row with no stored block gives zero rows.
 */
void oracle_spmm(int64_t nb, int64_t b, int64_t n, const int32_t *row_ptr, const int32_t *col_idx,
                 const double *blocks, const double *B, double *C) {
    const int64_t M = nb * b;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < M; ++i) {
        const int64_t I = i / b, ii = i - I * b;
        double *crow = C + i * n;
        for (int64_t j = 0; j < n; ++j) crow[j] = 0.0;
        for (int32_t p = row_ptr[I]; p < row_ptr[I + 1]; ++p) {
            const int64_t J = col_idx[p];
            const double *arow = blocks + ((int64_t)p * b + ii) * b;
            for (int64_t k = 0; k < b; ++k) {
                const double aik = arow[k];
                const double *brow = B + (J * b + k) * n;
                for (int64_t j = 0; j < n; ++j) crow[j] += aik * brow[j];
            }
        }
    }
}
