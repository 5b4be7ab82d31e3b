/* driver_oracle.c -- runs oracle/oracle.c under the host sanitizers: all
 * rows and row subsets, key ranges (empty included), causal with Sq > Sk
 * (rows without keys), GQA, 1 and 3 threads, and each class of bad argument.
 * Besides the return codes it checks two facts that hold for any input: a
 * row without allowed keys gives O = 0 and LSE = -inf, and a constant V gives
 * O equal to that constant.  Exits 0 when every check holds; the sanitizers
 * abort it on any memory error or undefined behaviour. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int Hq,
                    int Hkv, int Sq, int Sk, int D, int causal, float scale, int key_begin,
                    int key_end, const int64_t *rows, int64_t n_rows, double *o, double *lse,
                    int nthreads);
int64_t oracle_allowed_pairs(int Sq, int Sk, int causal);

static int g_fail = 0;
static uint32_t g_state = 12345u;

static uint16_t rand_bf16(void)
{
    /* a bf16 with a random sign and mantissa, magnitude in [2^-3, 2^1) */
    g_state = g_state * 1664525u + 1013904223u;
    const uint32_t r = g_state >> 8;
    const uint16_t exp = (uint16_t)(124 + (r & 3));
    return (uint16_t)(((r >> 2) & 1u) << 15 | exp << 7 | ((r >> 3) & 0x7f));
}

static void check(int cond, const char *what)
{
    if (!cond) {
        fprintf(stderr, "FAIL %s\n", what);
        ++g_fail;
    }
}

static void run_case(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int threads)
{
    const size_t qn = (size_t)B * Sq * Hq * D, kn = (size_t)B * Sk * Hkv * D;
    uint16_t *q = malloc(qn * 2), *k = malloc(kn * 2), *v = malloc(kn * 2);
    /* room for every row, or for the 5-row subsets below */
    const size_t nrow = (size_t)B * Hq * Sq > 5 ? (size_t)B * Hq * Sq : 5;
    double *o = malloc(nrow * D * sizeof(double)), *lse = malloc(nrow * sizeof(double));
    for (size_t i = 0; i < qn; ++i) q[i] = rand_bf16();
    for (size_t i = 0; i < kn; ++i) { k[i] = rand_bf16(); v[i] = 0x3fc0; /* 1.5 */ }
    check(oracle_attn_fwd(q, k, v, B, Hq, Hkv, Sq, Sk, D, causal, 0.125f, 0, Sk, NULL, 0, o, lse,
                          threads) == 0, "all rows");
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < Sq; ++i)
            for (int h = 0; h < Hq; ++h) {
                const int empty = causal && i + Sk - Sq < 0;
                const double l = lse[((size_t)b * Hq + h) * Sq + i];
                const double *row = o + (((size_t)b * Sq + i) * Hq + h) * D;
                check(empty ? isinf(l) && l < 0 : isfinite(l), "LSE finite unless the row is empty");
                for (int d = 0; d < D; ++d)
                    check(fabs(row[d] - (empty ? 0.0 : 1.5)) < 1e-12, "constant V gives constant O");
            }
    /* a subset of rows, and a key range that cuts the keys */
    int64_t rows[3 * 5];
    for (int r = 0; r < 5; ++r) {
        rows[3 * r] = r % B;
        rows[3 * r + 1] = (r * 7) % Hq;
        rows[3 * r + 2] = (r * 13) % Sq;
    }
    check(oracle_attn_fwd(q, k, v, B, Hq, Hkv, Sq, Sk, D, causal, 0.125f, 0, Sk, rows, 5, o, lse,
                          threads) == 0, "row subset");
    check(oracle_attn_fwd(q, k, v, B, Hq, Hkv, Sq, Sk, D, causal, -0.5f, Sk / 3, Sk, rows, 5, o,
                          lse, threads) == 0, "key range");
    check(oracle_attn_fwd(q, k, v, B, Hq, Hkv, Sq, Sk, D, causal, 0.125f, 2, 2, rows, 5, o, lse,
                          threads) == 0, "empty key range");
    for (int r = 0; r < 5; ++r) check(isinf(lse[r]) && lse[r] < 0, "empty key range gives -inf");
    free(q); free(k); free(v); free(o); free(lse);
}

int main(void)
{
    run_case(2, 4, 2, 37, 53, 64, 1, 1);
    run_case(2, 4, 2, 37, 53, 64, 0, 3);
    run_case(1, 2, 1, 40, 9, 128, 1, 3);     /* Sq > Sk: the first rows have no keys */
    run_case(1, 1, 1, 1, 300, 256, 0, 2);
    uint16_t x[64] = {0};
    double o[64], l[1];
    int64_t bad_row[3] = {0, 0, 5};
    check(oracle_attn_fwd(NULL, x, x, 1, 1, 1, 1, 1, 64, 0, 1.0f, 0, 1, NULL, 0, o, l, 1) < 0, "null q");
    check(oracle_attn_fwd(x, x, x, 1, 3, 2, 1, 1, 64, 0, 1.0f, 0, 1, NULL, 0, o, l, 1) < 0, "Hq % Hkv");
    check(oracle_attn_fwd(x, x, x, 1, 1, 1, 1, 1, 64, 0, 1.0f, 0, 2, NULL, 0, o, l, 1) < 0, "key_end > Sk");
    check(oracle_attn_fwd(x, x, x, 1, 1, 1, 1, 1, 64, 0, 1.0f, 0, 1, bad_row, 1, o, l, 1) < 0, "row out of range");
    check(oracle_allowed_pairs(4096, 4096, 1) == 4096LL * 4097 / 2, "causal pairs");
    check(oracle_allowed_pairs(40, 9, 1) == 45, "causal pairs with Sq > Sk");
    check(oracle_allowed_pairs(5, 7, 0) == 35, "non-causal pairs");
    printf("oracle: %d failures\n", g_fail);
    return g_fail ? 1 : 0;
}
