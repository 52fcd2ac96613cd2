/*
 * CPU oracle for the shard GEMMs of a 3D-parallel FC layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and
 * the benchmark's CPU-baseline leg may load this library. It shares no source,
 * header or helper with the GPU path (sharded_fc_layer_amd/csrc).
 *
 * What it computes: the plain definitions of the three products of one fully
 * connected layer on one GPU's shard (sciencestack.ai/paper/2502.08145,
 * Figure 1: the matrix multiply of an FC layer, split over a virtual grid):
 *
 *   forward          Y[m][n]  = sum_k X[m][k] * W[k][n]
 *   backward-data    dX[m][k] = sum_n dY[m][n] * W[k][n]      (dY . W^T)
 *   backward-weight  dW[k][n] = sum_m X[m][k] * dY[m][n]      (X^T . dY)
 *
 * Operands are bf16 (mlsanity.com/paper/2502.08145, Abstract: bf16 training):
 * each input element is the exact value of its 16-bit pattern (the high half
 * of an IEEE binary32). Every bf16 x bf16 product is exact in binary64 and
 * the sums are carried in binary64. Alongside each output the oracle returns
 * the tolerance scale S = sum |a|*|b| over the same terms.
 *
 * Storage orders: X and W each come row-major (order 0) or column-major
 * (order 1); dY is always row-major. The caller selects which output rows
 * and columns to compute (all of them, or a sample), so large shapes can be
 * checked one element at a time.
 *
 * Loops run output row -> reduction index -> output column, with OpenMP over
 * output rows. No blocking, no reordering of the sum beyond that.
 *
 * Parity pins: tests/test_oracle_pins.py (exact rational brute force, closed
 * forms, invariants, a library fp64 product, the virtual-grid reassembly) and
 * tests/test_golden.py (a hand-computed worked example, tests/golden/).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORDER_ROW 0
#define ORDER_COL 1

/* exact value of a bf16 bit pattern */
static double bf16_value(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* element (i, j) of a logical R x C bf16 matrix in the given storage order */
static double at(const uint16_t* p, int order, int64_t R, int64_t C, int64_t i, int64_t j) {
    return bf16_value(order == ORDER_ROW ? p[i * C + j] : p[j * R + i]);
}

/*
 * Generic plain product O[a][b] = sum_r A(I[a], r) * B(r, J[b]) for the
 * selected output rows I (n_i of them) and columns J (n_j), with S alongside.
 * A is a logical nI_total x R matrix, B a logical R x nJ_total matrix; both
 * are read through `at` in their storage orders. O and S are n_i x n_j,
 * row-major, overwritten.
 */
static int plain_product(const uint16_t* A, int a_order, int64_t a_rows,
                         const uint16_t* B, int b_order, int64_t b_cols, int64_t R,
                         const int64_t* I, int64_t n_i, const int64_t* J, int64_t n_j,
                         double* O, double* S) {
    /* the operand values that the selected outputs touch, decoded once */
    double* Bsel = (double*)malloc((size_t)(R > 0 ? R : 1) * (size_t)(n_j > 0 ? n_j : 1) * sizeof(double));
    if (!Bsel) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t b = 0; b < n_j; ++b)
            Bsel[r * n_j + b] = at(B, b_order, R, b_cols, r, J[b]);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t a = 0; a < n_i; ++a) {
        double* o = O + a * n_j;
        double* s = S + a * n_j;
        for (int64_t b = 0; b < n_j; ++b) { o[b] = 0.0; s[b] = 0.0; }
        for (int64_t r = 0; r < R; ++r) {
            const double x = at(A, a_order, a_rows, R, I[a], r);
            const double ax = fabs(x);
            const double* brow = Bsel + r * n_j;
            for (int64_t b = 0; b < n_j; ++b) {
                o[b] += x * brow[b];
                s[b] += ax * fabs(brow[b]);
            }
        }
    }
    free(Bsel);
    return 0;
}

/* forward: Y = X . W; rows index m (of M), cols index n (of N) */
int oracle_fc_fwd(const uint16_t* X, int x_order, const uint16_t* W, int w_order,
                  int64_t M, int64_t K, int64_t N,
                  const int64_t* rows, int64_t n_rows, const int64_t* cols, int64_t n_cols,
                  double* Y, double* S) {
    if (M < 0 || K < 0 || N < 0) return 2;
    /* A(m, k) = X[m][k]; B(k, n) = W[k][n] */
    return plain_product(X, x_order, M, W, w_order, N, K, rows, n_rows, cols, n_cols, Y, S);
}

/*
 * backward-data: dX = dY . W^T; rows index m (of M), cols index k (of K).
 * The reduction runs over n, the output features of the layer. B(n, k) is
 * W[k][n], i.e. the logical N x K matrix W^T, whose storage order is the
 * opposite of W's.
 */
int oracle_fc_bwd_data(const uint16_t* dY, const uint16_t* W, int w_order,
                       int64_t M, int64_t K, int64_t N,
                       const int64_t* rows, int64_t n_rows, const int64_t* cols, int64_t n_cols,
                       double* dX, double* S) {
    if (M < 0 || K < 0 || N < 0) return 2;
    const int wt_order = (w_order == ORDER_ROW) ? ORDER_COL : ORDER_ROW;
    return plain_product(dY, ORDER_ROW, M, W, wt_order, K, N, rows, n_rows, cols, n_cols, dX, S);
}

/*
 * backward-weight: dW = X^T . dY; rows index k (of K), cols index n (of N).
 * The reduction runs over m, the tokens. A(k, m) is X[m][k], i.e. the logical
 * K x M matrix X^T, whose storage order is the opposite of X's.
 */
int oracle_fc_bwd_weight(const uint16_t* X, int x_order, const uint16_t* dY,
                         int64_t M, int64_t K, int64_t N,
                         const int64_t* rows, int64_t n_rows, const int64_t* cols, int64_t n_cols,
                         double* dW, double* S) {
    if (M < 0 || K < 0 || N < 0) return 2;
    const int xt_order = (x_order == ORDER_ROW) ? ORDER_COL : ORDER_ROW;
    return plain_product(X, xt_order, K, dY, ORDER_ROW, N, M, rows, n_rows, cols, n_cols, dW, S);
}

/*
 * bf16 output rounding of an exact binary64 value: round to the nearest
 * bf16 (8 significant bits), ties to even, computed from the value itself
 * (never through binary32, so there is no double rounding). Overflow beyond
 * the largest finite bf16 gives infinity. Writes bit patterns.
 */
void oracle_round_bf16(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) {
        const double x = v[i];
        const int neg = signbit(x) ? 1 : 0;
        double a = fabs(x);
        uint16_t bits;
        if (isnan(x)) {
            bits = 0x7FC0;
        } else if (a == 0.0) {
            bits = 0;
        } else {
            int e;
            frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
            int qexp = e - 8;             /* spacing of 8-bit significands */
            if (qexp < -133) qexp = -133; /* bf16 subnormal spacing 2^-133 */
            const double q = nearbyint(ldexp(a, -qexp)); /* ties to even */
            const double r = ldexp(q, qexp);
            if (r > 3.3895313892515355e38) { /* largest finite bf16 */
                bits = 0x7F80;
            } else {
                float f = (float)r;       /* exact: r has <= 8 significant bits */
                uint32_t u;
                memcpy(&u, &f, sizeof u);
                bits = (uint16_t)(u >> 16);
            }
        }
        out[i] = (uint16_t)(bits | (neg ? 0x8000 : 0));
    }
}
