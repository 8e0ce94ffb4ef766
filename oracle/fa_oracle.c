/*
 * Attention oracle: plain, slow, fp64, CPU only.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do. It shares no code, header or table with the GPU
 * library.
 *
 * What it computes (the definition, written out):
 *   s_j  = scale * (q_i . k_j)             for every allowed key j
 *   a_j  = exp(s_j) / sum_t exp(s_t)        (softmax weights, sum to 1)
 *   o_i  = sum_j a_j v_j
 *   lse_i = ln sum_j exp(s_j)
 * Sources: "FlashAttention tiles exact softmax without materializing the
 * score matrix" (nalar.dev), opening definition S = QK^T/sqrt(d),
 * P = softmax(S), O = PV; "transformer math: flash attention math"
 * (aicassindra.com), section "What we must compute, and why storage is the
 * problem" (per-query form s_j, a_j, o).
 *
 * How: the safe-softmax route of the same aicassindra.com page, section
 * "Safe softmax: the max-subtraction we cannot give up": subtracting the
 * row maximum m leaves the weights unchanged, and the evaluation takes three
 * passes over the score row -- one for m, one for the denominator l, one for
 * the weighted sum. Then o = (weighted sum) / l and lse = m + ln l.
 *
 * Allowed keys: all j in [0, N); with causal != 0 only j <= i (a key after
 * the query is excluded, nalar.dev section "Causal masking fits inside the
 * tiled computation"). There is no tiling, blocking or reordering here: one
 * N-length fp64 score buffer per row, summed in ascending key order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the parallel loop below uses. */
int fa_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * q, k, v : [B, H, N, d] fp64, contiguous.
 * rows    : NULL for every row, else [B*H, n_rows] row indices (each in [0, N)).
 * o       : [B, H, N, d] when rows == NULL, else [B*H, n_rows, d].
 * lse     : [B, H, N]    when rows == NULL, else [B*H, n_rows].
 * Returns 0 on success, 1 on a bad argument, 2 on allocation failure.
 */
int fa_oracle_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
                  int64_t B, int64_t H, int64_t N, int64_t d, double scale, int causal,
                  const int64_t* rows, int64_t n_rows) {
    if (!q || !k || !v || !o || !lse || B < 1 || H < 1 || N < 1 || d < 1) return 1;
    int64_t per_head = rows ? n_rows : N;
    if (per_head < 1) return 1;
    if (rows) {
        for (int64_t t = 0; t < B * H * n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= N) return 1;
    }
    int64_t total = B * H * per_head;
    int nthreads = fa_oracle_threads();
    /* one score row and one accumulator per thread */
    double* s_all = (double*)malloc((size_t)nthreads * (size_t)N * sizeof(double));
    double* acc_all = (double*)malloc((size_t)nthreads * (size_t)d * sizeof(double));
    if (!s_all || !acc_all) {
        free(s_all);
        free(acc_all);
        return 2;
    }

#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t t = 0; t < total; ++t) {
#ifdef _OPENMP
        int tid = omp_get_thread_num();
#else
        int tid = 0;
#endif
        double* s = s_all + (size_t)tid * (size_t)N;
        double* acc = acc_all + (size_t)tid * (size_t)d;
        int64_t bh = t / per_head;
        int64_t r = t % per_head;
        int64_t i = rows ? rows[bh * n_rows + r] : r;
        const double* qi = q + (bh * N + i) * d;
        const double* kh = k + bh * N * d;
        const double* vh = v + bh * N * d;
        int64_t n_allowed = causal ? i + 1 : N;

        /* scores */
        for (int64_t j = 0; j < n_allowed; ++j) {
            const double* kj = kh + j * d;
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
            s[j] = scale * dot;
        }
        /* pass 1: the row maximum */
        double m = -INFINITY;
        for (int64_t j = 0; j < n_allowed; ++j)
            if (s[j] > m) m = s[j];
        /* pass 2: the denominator; every exponent s_j - m is <= 0 */
        double l = 0.0;
        for (int64_t j = 0; j < n_allowed; ++j) {
            s[j] = exp(s[j] - m);
            l += s[j];
        }
        /* pass 3: the weighted sum of values */
        for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
        for (int64_t j = 0; j < n_allowed; ++j) {
            const double* vj = vh + j * d;
            double w = s[j];
            for (int64_t c = 0; c < d; ++c) acc[c] += w * vj[c];
        }
        double* oi = o + (bh * per_head + r) * d;
        for (int64_t c = 0; c < d; ++c) oi[c] = acc[c] / l;
        lse[bh * per_head + r] = m + log(l);
    }
    free(s_all);
    free(acc_all);
    return 0;
}
