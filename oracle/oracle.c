/*
 * oracle.c -- plain, slow, double-precision CPU reference for the attention
 * forward pass.  TEST INFRASTRUCTURE ONLY: the tests, the smoke entry and the
 * benchmark's CPU-baseline leg may call it; the library never does.  It shares
 * no code, header or constant with the GPU path.
 *
 * What it computes is the plain definition, not the tiled algorithm:
 *
 *   s_ij   = scale * sum_d q[b,i,hq,d] * k[b,j,g,d]        for allowed j
 *   m_i    = max_j s_ij
 *   w_ij   = exp(s_ij - m_i),  l_i = sum_j w_ij
 *   O[b,i,hq,:] = sum_j w_ij * v[b,j,g,:] / l_i
 *   LSE[b,hq,i] = m_i + ln(l_i)            (natural log of sum_j exp(s_ij))
 *
 * Sources.  The components and their order (scores QK^T, row max, exp, row
 * sum, rescale, causal masking, then PV) are the ones listed for prefill
 * attention in "从 Volta/Turing、Ampere、Ada 到 Hopper：硬件、PTX 与 Kernel 编程
 * 范式演进" (tom-jerr.github.io), section "Attention 的瓶颈会在 Tensor Core 与
 * CUDA Core 之间迁移", and the loop they replace is the SM80 main loop of
 * "SM80 内核实现对比" (Inference Cookbook, FlashAttention), section 4.1.  The
 * online-softmax recurrence the kernels use is an exact rewrite of this
 * two-pass definition, so the definition is what the oracle writes out.
 *
 * Readings where the pages say nothing (each is listed in the design notes):
 *   - LSE is the natural log of the sum of exp of the *scaled* scores, laid
 *     out [B][Hq][Sq].
 *   - causal: key j is allowed for query i iff j <= i + (Sk - Sq)
 *     (bottom-right alignment; equals "j <= i" whenever Sq == Sk).
 *   - GQA: query head hq reads KV head g = hq / (Hq / Hkv).
 *   - a row with no allowed key has O = 0 and LSE = -inf.
 *   - layouts: q, o [B][Sq][Hq][D]; k, v [B][Sk][Hkv][D], D innermost.
 *
 * Inputs are the bf16 bit patterns the GPU receives; each is widened to
 * double exactly.  scale is the float32 the GPU receives, widened to double.
 * Everything after that is double precision; libm exp/log only.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v;
    int B, Hq, Hkv, Sq, Sk, D, causal;
    double scale;
    int key_begin, key_end;
    const int64_t *rows; /* NULL: every (b, hq, i); else triples (b, hq, i) */
    int64_t n_rows;
    double *o, *lse;
    int64_t first, last; /* this worker's row range [first, last) */
    int status;
} job_t;

/* One output row: the plain two-pass definition. */
static int one_row(const job_t *J, int b, int hq, int i, double *o_row, double *lse_out,
                   double *score)
{
    const int D = J->D;
    const int g = hq / (J->Hq / J->Hkv);
    /* allowed keys: [key_begin, key_end) and, when causal, j <= i + Sk - Sq */
    int64_t hi = J->key_end;
    if (J->causal) {
        int64_t lim = (int64_t)i + J->Sk - J->Sq + 1;
        if (lim < hi) hi = lim;
    }
    const int64_t lo = J->key_begin;

    for (int d = 0; d < D; ++d) o_row[d] = 0.0;
    if (hi <= lo) {
        *lse_out = -INFINITY;
        return 0;
    }

    const uint16_t *qrow = J->q + (((int64_t)b * J->Sq + i) * J->Hq + hq) * D;
    double m = -INFINITY;
    for (int64_t j = lo; j < hi; ++j) {
        const uint16_t *krow = J->k + (((int64_t)b * J->Sk + j) * J->Hkv + g) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += bf16_bits_to_double(qrow[d]) * bf16_bits_to_double(krow[d]);
        double s = J->scale * dot;
        score[j - lo] = s;
        if (s > m) m = s;
    }
    if (!isfinite(m)) return 1;

    double l = 0.0;
    for (int64_t j = lo; j < hi; ++j) {
        double w = exp(score[j - lo] - m);
        score[j - lo] = w;
        l += w;
    }
    for (int64_t j = lo; j < hi; ++j) {
        const uint16_t *vrow = J->v + (((int64_t)b * J->Sk + j) * J->Hkv + g) * D;
        const double w = score[j - lo];
        for (int d = 0; d < D; ++d) o_row[d] += w * bf16_bits_to_double(vrow[d]);
    }
    /* internal check: the normalised weights sum to one */
    double wsum = 0.0;
    for (int64_t j = lo; j < hi; ++j) wsum += score[j - lo] / l;
    if (fabs(wsum - 1.0) > 1e-12) return 2;

    for (int d = 0; d < D; ++d) {
        o_row[d] /= l;
        if (!isfinite(o_row[d])) return 3;
    }
    *lse_out = m + log(l);
    return 0;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *score = (double *)malloc(sizeof(double) * (size_t)(J->Sk > 0 ? J->Sk : 1));
    if (!score) {
        J->status = 4;
        return NULL;
    }
    for (int64_t r = J->first; r < J->last && J->status == 0; ++r) {
        int b, hq, i;
        double *o_row, *lse_out;
        if (J->rows) {
            b = (int)J->rows[3 * r];
            hq = (int)J->rows[3 * r + 1];
            i = (int)J->rows[3 * r + 2];
            o_row = J->o + r * J->D;
            lse_out = J->lse + r;
        } else {
            /* r enumerates (b, hq, i) with i fastest */
            i = (int)(r % J->Sq);
            hq = (int)((r / J->Sq) % J->Hq);
            b = (int)(r / ((int64_t)J->Sq * J->Hq));
            o_row = J->o + (((int64_t)b * J->Sq + i) * J->Hq + hq) * J->D;
            lse_out = J->lse + ((int64_t)b * J->Hq + hq) * J->Sq + i;
        }
        J->status = one_row(J, b, hq, i, o_row, lse_out, score);
    }
    free(score);
    return NULL;
}

/*
 * oracle_attn_fwd: returns 0 on success, a positive code on a failed internal
 * check, negative on bad arguments.
 *   rows == NULL: o is [B][Sq][Hq][D] and lse is [B][Hq][Sq] (all rows).
 *   rows != NULL: n_rows triples (b, hq, i); o is [n_rows][D], lse [n_rows].
 *   [key_begin, key_end) restricts the keys (pass 0, Sk for all of them).
 */
int oracle_attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int Hq,
                    int Hkv, int Sq, int Sk, int D, int causal, float scale, int key_begin,
                    int key_end, const int64_t *rows, int64_t n_rows, double *o, double *lse,
                    int nthreads)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || D < 1) return -2;
    if (Hq % Hkv != 0) return -3;
    if (key_begin < 0 || key_end > Sk || key_begin > key_end) return -4;
    const int64_t total = rows ? n_rows : (int64_t)B * Hq * Sq;
    if (rows) {
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 ||
                rows[3 * r + 1] >= Hq || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= Sq)
                return -5;
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (total < nthreads) nthreads = total > 0 ? (int)total : 1;

    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return 4;
    }
    int rc = 0;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        job_t *J = &jobs[t];
        J->q = q; J->k = k; J->v = v;
        J->B = B; J->Hq = Hq; J->Hkv = Hkv; J->Sq = Sq; J->Sk = Sk; J->D = D;
        J->causal = causal;
        J->scale = (double)scale;
        J->key_begin = key_begin; J->key_end = key_end;
        J->rows = rows; J->n_rows = n_rows;
        J->o = o; J->lse = lse;
        J->first = total * t / nthreads;
        J->last = total * (t + 1) / nthreads;
        J->status = 0;
        if (pthread_create(&tids[t], NULL, worker, J) != 0) {
            worker(J); /* run inline if a thread cannot be started */
        } else {
            ++started;
            continue;
        }
        tids[t] = 0;
    }
    for (int t = 0; t < nthreads; ++t) {
        if (tids[t]) pthread_join(tids[t], NULL);
        if (jobs[t].status && !rc) rc = jobs[t].status;
    }
    (void)started;
    free(jobs);
    free(tids);
    return rc;
}

/* number of allowed (query, key) pairs for one (b, hq): the algorithmic work
 * unit, 4*D flops each (QK^T and PV), used by the benchmark's CPU leg. */
int64_t oracle_allowed_pairs(int Sq, int Sk, int causal)
{
    if (!causal) return (int64_t)Sq * Sk;
    int64_t n = 0;
    for (int64_t i = 0; i < Sq; ++i) {
        int64_t hi = i + Sk - Sq + 1;
        if (hi > Sk) hi = Sk;
        if (hi > 0) n += hi;
    }
    return n;
}
