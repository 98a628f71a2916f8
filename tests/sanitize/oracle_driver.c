/*
 * Driver for the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (CPU only; built by tests/test_sanitizers.py with gcc). It runs every
 * oracle entry point on small seeded inputs over several structures,
 * including empty block rows and columns and a structure with no stored
 * block; any invalid memory access or undefined behaviour aborts the run
 * with a sanitizer report. The values are checked elsewhere (test_oracle.py).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_fwd(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb, const int32_t *row_ptr,
                const int32_t *col_idx, double scale, const double *q, const double *k, const double *v, double *o,
                double *row_max, double *row_denom);
void oracle_fwd_rows(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb, const int32_t *row_ptr,
                     const int32_t *col_idx, double scale, const double *q, const double *k, const double *v,
                     int64_t n_rows, const int64_t *rows, double *o, double *row_max, double *row_denom);
void oracle_bwd(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb, const int32_t *row_ptr,
                const int32_t *col_idx, double scale, const double *q, const double *k, const double *v,
                const double *dout, double *dq, double *dk, double *dv);
void oracle_bwd_rows(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb, const int32_t *row_ptr,
                     const int32_t *col_idx, double scale, const double *q, const double *k, const double *v,
                     const double *dout, int64_t n_rows, const int64_t *rows, double *dq);
void oracle_bwd_cols(int64_t BH, int64_t S, int64_t D, int64_t b, int64_t nb, const int32_t *row_ptr,
                     const int32_t *col_idx, double scale, const double *q, const double *k, const double *v,
                     const double *dout, int64_t n_cols, const int64_t *cols, double *dk, double *dv);
void oracle_spmm(int64_t nb, int64_t b, int64_t n, const int32_t *row_ptr, const int32_t *col_idx,
                 const double *blocks, const double *bmat, double *c);

static uint64_t state = 88172645463325252ull;
static double uniform(void) { /* xorshift64 */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double *filled(int64_t n) {
    double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = uniform();
    return p;
}

/* one structure of nb block rows of block size b, given as a mask */
static void run(int64_t nb, int64_t b, int64_t BH, int64_t D, const unsigned char *mask) {
    int32_t *row_ptr = (int32_t *)calloc((size_t)nb + 1, sizeof(int32_t));
    int32_t *col_idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nb * nb > 0 ? nb * nb : 1));
    int32_t nnzb = 0;
    for (int64_t i = 0; i < nb; ++i) {
        for (int64_t j = 0; j < nb; ++j)
            if (mask[i * nb + j]) col_idx[nnzb++] = (int32_t)j;
        row_ptr[i + 1] = nnzb;
    }
    const int64_t S = nb * b, n = BH * S * D;
    double *q = filled(n), *k = filled(n), *v = filled(n), *d = filled(n);
    double *o = filled(n), *dq = filled(n), *dk = filled(n), *dv = filled(n);
    double *m = filled(BH * S), *l = filled(BH * S);
    const double scale = 0.25;
    oracle_fwd(BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, o, m, l);
    oracle_bwd(BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, d, dq, dk, dv);
    int64_t rows[3] = {0, BH * S / 2, BH * S - 1};
    double *o3 = filled(3 * D), *m3 = filled(3), *l3 = filled(3), *dq3 = filled(3 * D), *dk3 = filled(3 * D),
           *dv3 = filled(3 * D);
    oracle_fwd_rows(BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, 3, rows, o3, m3, l3);
    oracle_bwd_rows(BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, d, 3, rows, dq3);
    oracle_bwd_cols(BH, S, D, b, nb, row_ptr, col_idx, scale, q, k, v, d, 3, rows, dk3, dv3);
    double *blocks = filled((int64_t)nnzb * b * b), *bm = filled(S * 8), *c = filled(S * 8);
    oracle_spmm(nb, b, 8, row_ptr, col_idx, blocks, bm, c);
    free(q); free(k); free(v); free(d); free(o); free(dq); free(dk); free(dv); free(m); free(l);
    free(o3); free(m3); free(l3); free(dq3); free(dk3); free(dv3); free(blocks); free(bm); free(c);
    free(row_ptr); free(col_idx);
}

int main(void) {
    const int64_t nb = 4, b = 8;
    unsigned char mask[16];
    for (int kind = 0; kind < 5; ++kind) {
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 4; ++j) {
                int keep = 0;
                if (kind == 0) keep = 1;                                   /* every block */
                if (kind == 1) keep = (i - j <= 1 && j - i <= 1) || !i || !j; /* global */
                if (kind == 2) keep = (i == 0 && j == 3) || (i == 2 && j <= 2); /* empty rows and columns */
                if (kind == 3) keep = 0;                                   /* nothing stored */
                if (kind == 4) keep = i == j;                              /* diagonal */
                mask[i * 4 + j] = (unsigned char)keep;
            }
        run(nb, b, 2, 4, mask);
    }
    printf("oracle driver: ok\n");
    return 0;
}
