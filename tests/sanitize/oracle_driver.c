/*
 * Host sanitizer run of the CPU oracle (oracle/oracle.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize_cpu.py
 * (without OpenMP: the pragmas are ignored and every loop runs in order).
 *
 * It drives each entry point over every storage order, on shapes with
 * dimensions of 0, 1 and ragged sizes, with full and sampled (unsorted,
 * repeated, boundary) output selections, and checks each value against a
 * naive sum written here in the same order, so a read or write outside the
 * buffers, an overflow or a wrong value all fail the run. It also rounds
 * special and random values to bf16 and checks the patterns the format fixes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_fc_fwd(const uint16_t*, int, const uint16_t*, int, int64_t, int64_t, int64_t, const int64_t*, int64_t,
                  const int64_t*, int64_t, double*, double*);
int oracle_fc_bwd_data(const uint16_t*, const uint16_t*, int, int64_t, int64_t, int64_t, const int64_t*, int64_t,
                       const int64_t*, int64_t, double*, double*);
int oracle_fc_bwd_weight(const uint16_t*, int, const uint16_t*, int64_t, int64_t, int64_t, const int64_t*, int64_t,
                         const int64_t*, int64_t, double*, double*);
void oracle_round_bf16(const double*, int64_t, uint16_t*);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}

static double bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* a finite bf16 with a small exponent range, so sums stay exact-ish */
static uint16_t rand_bf16(void) {
    const uint32_t r = next_u32();
    const uint16_t sign = (uint16_t)((r & 1u) << 15);
    const uint16_t exp = (uint16_t)(120 + (r >> 1) % 12);
    const uint16_t man = (uint16_t)((r >> 5) & 0x7F);
    return (uint16_t)(sign | (exp << 7) | man);
}

/* logical (i, j) of an R x C matrix stored row-major (0) or column-major (1) */
static double el(const uint16_t* p, int order, int64_t R, int64_t C, int64_t i, int64_t j) {
    return bf16(order == 0 ? p[i * C + j] : p[j * R + i]);
}

static int failures = 0;
#define CHECK(cond, ...)                      \
    do {                                      \
        if (!(cond)) {                        \
            fprintf(stderr, __VA_ARGS__);     \
            fputc('\n', stderr);              \
            ++failures;                       \
        }                                     \
    } while (0)

/* selection: all indices, or a sample with the first, the last, repeats and
   an unsorted order */
static int64_t* selection(int64_t n, int sampled, int64_t* count) {
    if (!sampled || n == 0) {
        int64_t* s = (int64_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
        for (int64_t i = 0; i < n; ++i) s[i] = i;
        *count = n;
        return s;
    }
    const int64_t c = 5;
    int64_t* s = (int64_t*)malloc((size_t)c * sizeof(int64_t));
    s[0] = n - 1;
    s[1] = 0;
    s[2] = (int64_t)(next_u32() % (uint32_t)n);
    s[3] = s[2];
    s[4] = n / 2;
    *count = c;
    return s;
}

static void run_case(int64_t M, int64_t K, int64_t N, int xo, int wo, int sampled) {
    uint16_t* X = (uint16_t*)malloc((size_t)(M * K > 0 ? M * K : 1) * 2);
    uint16_t* W = (uint16_t*)malloc((size_t)(K * N > 0 ? K * N : 1) * 2);
    uint16_t* dY = (uint16_t*)malloc((size_t)(M * N > 0 ? M * N : 1) * 2);
    for (int64_t i = 0; i < M * K; ++i) X[i] = rand_bf16();
    for (int64_t i = 0; i < K * N; ++i) W[i] = rand_bf16();
    for (int64_t i = 0; i < M * N; ++i) dY[i] = rand_bf16();
    for (int op = 0; op < 3; ++op) {
        const int64_t R = op == 0 ? M : op == 1 ? M : K;  /* output rows */
        const int64_t C = op == 0 ? N : op == 1 ? K : N;  /* output cols */
        const int64_t red = op == 0 ? K : op == 1 ? N : M;
        int64_t nr, nc;
        int64_t* rows = selection(R, sampled, &nr);
        int64_t* cols = selection(C, sampled, &nc);
        /* exact-size outputs, so any write past them is caught */
        double* O = (double*)malloc((size_t)(nr * nc > 0 ? nr * nc : 1) * sizeof(double));
        double* S = (double*)malloc((size_t)(nr * nc > 0 ? nr * nc : 1) * sizeof(double));
        int rc;
        if (op == 0)
            rc = oracle_fc_fwd(X, xo, W, wo, M, K, N, rows, nr, cols, nc, O, S);
        else if (op == 1)
            rc = oracle_fc_bwd_data(dY, W, wo, M, K, N, rows, nr, cols, nc, O, S);
        else
            rc = oracle_fc_bwd_weight(X, xo, dY, M, K, N, rows, nr, cols, nc, O, S);
        CHECK(rc == 0, "op %d M %lld K %lld N %lld: status %d", op, (long long)M, (long long)K, (long long)N, rc);
        for (int64_t a = 0; a < nr && rc == 0; ++a)
            for (int64_t b = 0; b < nc; ++b) {
                double o = 0.0, s = 0.0;
                for (int64_t r = 0; r < red; ++r) {
                    double x, y;
                    if (op == 0) {
                        x = el(X, xo, M, K, rows[a], r);
                        y = el(W, wo, K, N, r, cols[b]);
                    } else if (op == 1) {
                        x = el(dY, 0, M, N, rows[a], r);
                        y = el(W, wo, K, N, cols[b], r);
                    } else {
                        x = el(X, xo, M, K, r, rows[a]);
                        y = el(dY, 0, M, N, r, cols[b]);
                    }
                    o += x * y;
                    s += fabs(x) * fabs(y);
                }
                CHECK(O[a * nc + b] == o && S[a * nc + b] == s,
                      "op %d M %lld K %lld N %lld orders %d %d: value (%lld, %lld) %.17g vs %.17g", op, (long long)M,
                      (long long)K, (long long)N, xo, wo, (long long)rows[a], (long long)cols[b], O[a * nc + b], o);
            }
        free(rows);
        free(cols);
        free(O);
        free(S);
    }
    free(X);
    free(W);
    free(dY);
}

static void rounding(void) {
    const double v[] = {0.0, -0.0, 1.0, -2.0, 1.0 + 1.0 / 256, 1.0 + 3.0 / 256, INFINITY, -INFINITY, NAN,
                        3.3895313892515355e38, 3.4e38, 1e300, ldexp(1.0, -133), ldexp(1.0, -134),
                        ldexp(3.0, -136), ldexp(1.0, -126), -ldexp(1.0, -140), 5e-324, ldexp(3.0, -135)};
    const int n = (int)(sizeof v / sizeof v[0]);
    uint16_t out[sizeof v / sizeof v[0]];
    oracle_round_bf16(v, n, out);
    CHECK(out[0] == 0x0000 && out[1] == 0x8000, "signed zeros: %04x %04x", out[0], out[1]);
    CHECK(out[2] == 0x3F80 && out[3] == 0xC000, "1, -2: %04x %04x", out[2], out[3]);
    CHECK(out[4] == 0x3F80, "1 + 2^-8 ties to even (down): %04x", out[4]);
    CHECK(out[5] == 0x3F82, "1 + 3 * 2^-8 ties to even (up): %04x", out[5]);
    CHECK(out[6] == 0x7F80 && out[7] == 0xFF80, "infinities: %04x %04x", out[6], out[7]);
    CHECK((out[8] & 0x7F80) == 0x7F80 && (out[8] & 0x7F) != 0, "NaN: %04x", out[8]);
    CHECK(out[9] == 0x7F7F, "largest finite: %04x", out[9]);
    CHECK(out[10] == 0x7F80 && out[11] == 0x7F80, "overflow: %04x %04x", out[10], out[11]);
    CHECK(out[12] == 0x0001, "smallest subnormal: %04x", out[12]);
    CHECK(out[13] == 0x0000, "half the smallest subnormal ties to even (zero): %04x", out[13]);
    CHECK(out[14] == 0x0000, "3/8 of the smallest subnormal rounds to zero: %04x", out[14]);
    CHECK(out[15] == 0x0080, "smallest normal: %04x", out[15]);
    CHECK(out[16] == 0x8000, "tiny negative rounds to -0: %04x", out[16]);
    CHECK(out[17] == 0x0000, "smallest double: %04x", out[17]);
    CHECK(out[18] == 0x0001, "3/4 of the smallest subnormal rounds up to it: %04x", out[18]);
    /* random doubles: the pattern decodes to a value within half a bf16 ulp */
    enum { R = 4096 };
    static double rv[R];
    static uint16_t ro[R];
    for (int i = 0; i < R; ++i) {
        const double m = (double)next_u32() / 4294967296.0 + 0.5;
        rv[i] = ldexp(i % 2 ? -m : m, (int)(next_u32() % 200) - 100);
    }
    oracle_round_bf16(rv, R, ro);
    for (int i = 0; i < R; ++i) {
        const double back = bf16(ro[i]);
        int e;
        frexp(rv[i], &e);
        CHECK(fabs(back - rv[i]) <= ldexp(1.0, e - 9), "random %d: %.17g -> %04x", i, rv[i], ro[i]);
    }
    oracle_round_bf16(v, 0, out); /* an empty call touches nothing */
}

int main(void) {
    const int64_t dims[] = {0, 1, 2, 7, 33};
    int cases = 0;
    for (int a = 0; a < 5; ++a)
        for (int b = 0; b < 5; ++b)
            for (int c = 0; c < 5; ++c)
                for (int orders = 0; orders < 4; ++orders)
                    for (int sampled = 0; sampled < 2; ++sampled) {
                        run_case(dims[a], dims[b], dims[c], orders & 1, orders >> 1, sampled);
                        ++cases;
                    }
    run_case(65, 130, 67, 1, 0, 1);
    /* negative sizes are refused before anything is read */
    double o[1], s[1];
    int64_t idx[1] = {0};
    CHECK(oracle_fc_fwd(NULL, 0, NULL, 0, -1, 1, 1, idx, 0, idx, 0, o, s) != 0, "negative M accepted");
    CHECK(oracle_fc_bwd_data(NULL, NULL, 0, 1, -1, 1, idx, 0, idx, 0, o, s) != 0, "negative K accepted");
    CHECK(oracle_fc_bwd_weight(NULL, 0, NULL, 1, 1, -1, idx, 0, idx, 0, o, s) != 0, "negative N accepted");
    rounding();
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("sanitized oracle run: ok (%d product cases)\n", cases + 1);
    return 0;
}
