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
 *
 * fa_oracle_fwd_masked and fa_oracle_fwd_blocksparse restrict the allowed keys
 * further (windows, key padding, a mask over blocks of the score matrix).
 * fa_oracle_bwd, at the end of the file, gives the gradients of the same
 * definition with respect to q, k and v by the chain rule; fa_oracle_bwd_masked and
 * fa_oracle_bwd_blocksparse the same under the window / key-length and block masks.
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

/*
 * Gradients of the loss L = sum_i dO_i . o_i with respect to q, k and v (fp64).
 *
 * The pages give the backward pass only as a dataflow: keep the per-row
 * softmax statistics and recompute score tiles rather than store them
 * ("Decoding flash attention" (bibekananda.in), section "The backward pass";
 * nalar.dev, section "Backward computation can trade recomputation for stored
 * intermediates"). The values are the chain rule applied to the definition at
 * the top of this file, written out with no tiling:
 *   a_ij  = softmax weights of row i (three-pass route, as above)
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j a_ij dP_ij                 (the row's weighted mean of dP)
 *   dS_ij = a_ij (dP_ij - D_i)               (Jacobian of softmax applied to dP)
 *   dV_j  = sum_i a_ij dO_i
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 * Sums over i run over the rows that allow key j (all rows, or i >= j when
 * causal); sums over j over the keys row i allows.
 *
 * q, k, v, dout : [G, N, d] fp64 (G heads), contiguous.
 * rows          : NULL for every row, else [G, n_rows] row indices; dq is [G, n_rows or N, d].
 * keys          : NULL for every key, else [G, n_keys] key indices; dk, dv are [G, n_keys or N, d].
 * lse, delta    : NULL or [G, N]; receive m_i + ln l_i and D_i of every row.
 * Returns 0 on success, 1 on a bad argument, 2 on allocation failure.
 */
int fa_oracle_bwd(const double* q, const double* k, const double* v, const double* dout,
                  double* dq, double* dk, double* dv, double* lse, double* delta,
                  int64_t G, int64_t N, int64_t d, double scale, int causal,
                  const int64_t* rows, int64_t n_rows, const int64_t* keys, int64_t n_keys) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || G < 1 || N < 1 || d < 1) return 1;
    int64_t R = rows ? n_rows : N;
    int64_t C = keys ? n_keys : N;
    if (R < 1 || C < 1) return 1;
    for (int64_t t = 0; rows && t < G * n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= N) return 1;
    for (int64_t t = 0; keys && t < G * n_keys; ++t)
        if (keys[t] < 0 || keys[t] >= N) return 1;
    int nthreads = fa_oracle_threads();
    double* m_all = (double*)malloc((size_t)(G * N) * sizeof(double));
    double* l_all = (double*)malloc((size_t)(G * N) * sizeof(double));
    double* D_all = (double*)malloc((size_t)(G * N) * sizeof(double));
    double* s_all = (double*)malloc((size_t)nthreads * (size_t)N * sizeof(double));
    double* dp_all = (double*)malloc((size_t)nthreads * (size_t)N * sizeof(double));
    if (!m_all || !l_all || !D_all || !s_all || !dp_all) {
        free(m_all); free(l_all); free(D_all); free(s_all); free(dp_all);
        return 2;
    }

    /* pass 1, every row: m_i, l_i (three-pass route) and D_i */
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t t = 0; t < G * N; ++t) {
#ifdef _OPENMP
        int tid = omp_get_thread_num();
#else
        int tid = 0;
#endif
        double* s = s_all + (size_t)tid * (size_t)N;
        int64_t g = t / N, i = t % N;
        const double* qi = q + t * d;
        const double* doi = dout + t * d;
        const double* kh = k + g * N * d;
        const double* vh = v + g * N * d;
        int64_t n_allowed = causal ? i + 1 : N;
        for (int64_t j = 0; j < n_allowed; ++j) {
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
            s[j] = scale * dot;
        }
        double m = -INFINITY;
        for (int64_t j = 0; j < n_allowed; ++j)
            if (s[j] > m) m = s[j];
        double l = 0.0;
        for (int64_t j = 0; j < n_allowed; ++j) l += exp(s[j] - m);
        double D = 0.0;
        for (int64_t j = 0; j < n_allowed; ++j) {
            double dp = 0.0;
            for (int64_t c = 0; c < d; ++c) dp += doi[c] * vh[j * d + c];
            D += (exp(s[j] - m) / l) * dp;
        }
        m_all[t] = m;
        l_all[t] = l;
        D_all[t] = D;
        if (lse) lse[t] = m + log(l);
        if (delta) delta[t] = D;
    }

    /* pass 2, requested rows: dQ_i = scale * sum_j a_ij (dP_ij - D_i) k_j */
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t t = 0; t < G * R; ++t) {
#ifdef _OPENMP
        int tid = omp_get_thread_num();
#else
        int tid = 0;
#endif
        double* s = s_all + (size_t)tid * (size_t)N;
        double* dp = dp_all + (size_t)tid * (size_t)N;
        int64_t g = t / R, r = t % R;
        int64_t i = rows ? rows[g * n_rows + r] : r;
        const double* qi = q + (g * N + i) * d;
        const double* doi = dout + (g * N + i) * d;
        const double* kh = k + g * N * d;
        const double* vh = v + g * N * d;
        int64_t n_allowed = causal ? i + 1 : N;
        double m = m_all[g * N + i], l = l_all[g * N + i], D = D_all[g * N + i];
        for (int64_t j = 0; j < n_allowed; ++j) {
            double dot = 0.0, dpv = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
            for (int64_t c = 0; c < d; ++c) dpv += doi[c] * vh[j * d + c];
            s[j] = exp(scale * dot - m) / l;
            dp[j] = dpv;
        }
        double* out = dq + t * d;
        for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
        for (int64_t j = 0; j < n_allowed; ++j) {
            double ds = s[j] * (dp[j] - D);
            for (int64_t c = 0; c < d; ++c) out[c] += ds * kh[j * d + c];
        }
        for (int64_t c = 0; c < d; ++c) out[c] *= scale;
    }

    /* pass 3, requested keys: dV_j = sum_i a_ij dO_i, dK_j = scale * sum_i a_ij (dP_ij - D_i) q_i */
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
    for (int64_t t = 0; t < G * C; ++t) {
        int64_t g = t / C, r = t % C;
        int64_t j = keys ? keys[g * n_keys + r] : r;
        const double* kj = k + (g * N + j) * d;
        const double* vj = v + (g * N + j) * d;
        double* ok = dk + t * d;
        double* ov = dv + t * d;
        for (int64_t c = 0; c < d; ++c) ok[c] = ov[c] = 0.0;
        for (int64_t i = causal ? j : 0; i < N; ++i) {
            const double* qi = q + (g * N + i) * d;
            const double* doi = dout + (g * N + i) * d;
            double dot = 0.0, dpv = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
            for (int64_t c = 0; c < d; ++c) dpv += doi[c] * vj[c];
            double a = exp(scale * dot - m_all[g * N + i]) / l_all[g * N + i];
            double ds = a * (dpv - D_all[g * N + i]);
            for (int64_t c = 0; c < d; ++c) {
                ov[c] += a * doi[c];
                ok[c] += ds * qi[c];
            }
        }
        for (int64_t c = 0; c < d; ++c) ok[c] *= scale;
    }
    free(m_all); free(l_all); free(D_all); free(s_all); free(dp_all);
    return 0;
}

/*
 * The definition above with a general mask: key j is allowed for query i when
 *   (window_left  < 0 or j >= i - window_left)  and
 *   (window_right < 0 or j <= i + window_right) and
 *   j < kv_len_b,   kv_len_b = seqlens_k ? seqlens_k[b] : N.
 * Masked keys carry no probability mass, which is how the pages admit masks other
 * than the causal one ("Causal masking fits inside the tiled computation", nalar.dev,
 * last paragraph; aicassindra.com, "Pitfalls in implementing the recurrence": masked
 * scores are -inf before the max, "for causal or padded attention"). window_right = 0
 * with window_left = -1 is the causal mask; seqlens_k is key padding.
 * A row with no allowed key has no softmax; its output is 0 and its lse is -inf.
 *
 * Arguments as fa_oracle_fwd, with causal replaced by window_left, window_right and
 * seqlens_k (host pointer, [B], or NULL). Same return codes.
 */
int fa_oracle_fwd_masked(const double* q, const double* k, const double* v, double* o, double* lse,
                         int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                         int64_t window_left, int64_t window_right, const int64_t* seqlens_k,
                         const int64_t* rows, int64_t n_rows) {
    if (!q || !k || !v || !o || !lse || B < 1 || H < 1 || N < 1 || d < 1) return 1;
    if (window_left < -1 || window_right < -1) return 1;
    int64_t per_head = rows ? n_rows : N;
    if (per_head < 1) return 1;
    for (int64_t t = 0; rows && t < B * H * n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= N) return 1;
    for (int64_t b = 0; seqlens_k && b < B; ++b)
        if (seqlens_k[b] < 0 || seqlens_k[b] > N) return 1;
    int64_t total = B * H * per_head;
    int nthreads = fa_oracle_threads();
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
        int64_t kv_len = seqlens_k ? seqlens_k[bh / H] : N;
        /* the allowed keys form one interval [lo, hi) */
        int64_t lo = window_left >= 0 ? i - window_left : 0;
        int64_t hi = window_right >= 0 ? i + window_right + 1 : N;
        if (lo < 0) lo = 0;
        if (hi > kv_len) hi = kv_len;
        const double* qi = q + (bh * N + i) * d;
        const double* kh = k + bh * N * d;
        const double* vh = v + bh * N * d;
        double* oi = o + (bh * per_head + r) * d;
        if (hi <= lo) {
            for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
            lse[bh * per_head + r] = -INFINITY;
            continue;
        }
        for (int64_t j = lo; j < hi; ++j) {
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
            s[j] = scale * dot;
        }
        /* the three passes of the safe softmax, over the allowed keys */
        double m = -INFINITY;
        for (int64_t j = lo; j < hi; ++j)
            if (s[j] > m) m = s[j];
        double l = 0.0;
        for (int64_t j = lo; j < hi; ++j) {
            s[j] = exp(s[j] - m);
            l += s[j];
        }
        for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
        for (int64_t j = lo; j < hi; ++j)
            for (int64_t c = 0; c < d; ++c) acc[c] += s[j] * vh[j * d + c];
        for (int64_t c = 0; c < d; ++c) oi[c] = acc[c] / l;
        lse[bh * per_head + r] = m + log(l);
    }
    free(s_all);
    free(acc_all);
    return 0;
}

/*
 * Block-sparse attention: the general mask of fa_oracle_fwd_masked and, on top of it, a
 * mask over blocks of the score matrix. Query i lies in query block i / block_q, key j in
 * key block j / block_k; the pair is allowed only when the byte
 *   block_mask[b * stride_b + h * stride_h + (i / block_q) * n_kb + j / block_k]
 * is non-zero, with n_kb = ceil(N / block_k) bytes per mask row (a stride of 0 shares one
 * mask across batches or heads). Any mask applied to the scores before the max is
 * admitted by the pages ("Causal masking fits inside the tiled computation", nalar.dev,
 * last paragraph; aicassindra.com, "Pitfalls in implementing the recurrence"); a mask given
 * per block is the plainest such mask that decides whole tiles at once.
 * A row with no allowed key has no softmax; its output is 0 and its lse is -inf.
 *
 * Arguments as fa_oracle_fwd_masked, plus block_mask (host pointer), block_q, block_k >= 1,
 * stride_b, stride_h >= 0. Same return codes.
 */
int fa_oracle_fwd_blocksparse(const double* q, const double* k, const double* v, double* o, double* lse,
                              int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                              int64_t window_left, int64_t window_right, const int64_t* seqlens_k,
                              const uint8_t* block_mask, int64_t block_q, int64_t block_k,
                              int64_t stride_b, int64_t stride_h, const int64_t* rows, int64_t n_rows) {
    if (!q || !k || !v || !o || !lse || !block_mask || B < 1 || H < 1 || N < 1 || d < 1) return 1;
    if (window_left < -1 || window_right < -1 || block_q < 1 || block_k < 1 || stride_b < 0 || stride_h < 0)
        return 1;
    int64_t per_head = rows ? n_rows : N;
    if (per_head < 1) return 1;
    for (int64_t t = 0; rows && t < B * H * n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= N) return 1;
    for (int64_t b = 0; seqlens_k && b < B; ++b)
        if (seqlens_k[b] < 0 || seqlens_k[b] > N) return 1;
    const int64_t n_kb = (N + block_k - 1) / block_k;
    int64_t total = B * H * per_head;
    int nthreads = fa_oracle_threads();
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
        int64_t kv_len = seqlens_k ? seqlens_k[bh / H] : N;
        int64_t lo = window_left >= 0 ? i - window_left : 0;
        int64_t hi = window_right >= 0 ? i + window_right + 1 : N;
        if (lo < 0) lo = 0;
        if (hi > kv_len) hi = kv_len;
        const uint8_t* mrow = block_mask + (bh / H) * stride_b + (bh % H) * stride_h + (i / block_q) * n_kb;
        const double* qi = q + (bh * N + i) * d;
        const double* kh = k + bh * N * d;
        const double* vh = v + bh * N * d;
        double* oi = o + (bh * per_head + r) * d;
        /* scores of the allowed keys; the others stay out of every pass */
        double m = -INFINITY;
        int64_t allowed = 0;
        for (int64_t j = lo; j < hi; ++j) {
            if (!mrow[j / block_k]) continue;
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
            s[j] = scale * dot;
            if (s[j] > m) m = s[j];
            ++allowed;
        }
        if (allowed == 0) {
            for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
            lse[bh * per_head + r] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int64_t j = lo; j < hi; ++j) {
            if (!mrow[j / block_k]) continue;
            s[j] = exp(s[j] - m);
            l += s[j];
        }
        for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
        for (int64_t j = lo; j < hi; ++j) {
            if (!mrow[j / block_k]) continue;
            for (int64_t c = 0; c < d; ++c) acc[c] += s[j] * vh[j * d + c];
        }
        for (int64_t c = 0; c < d; ++c) oi[c] = acc[c] / l;
        lse[bh * per_head + r] = m + log(l);
    }
    free(s_all);
    free(acc_all);
    return 0;
}

/*
 * The gradients of fa_oracle_bwd under a general mask. Key j is allowed for query i of batch b
 * when j >= i - window_left (window_left >= 0), j <= i + window_right (window_right >= 0),
 * j < seqlens_k[b] (seqlens_k given) and, with a block mask, the byte of query block
 * i / block_q and key block j / block_k is non-zero (the layout of fa_oracle_fwd_blocksparse).
 * The chain rule is unchanged; every sum runs over the allowed pairs only (masked scores carry
 * no probability, so they contribute nothing to any gradient). A row with no allowed key has
 * lse = -inf, D = 0 and dq = 0, and adds nothing to dk or dv; a key no row allows gets
 * dk = dv = 0.
 */
typedef struct {
    int64_t H, N, window_left, window_right, block_q, block_k, n_kb, stride_b, stride_h;
    const int64_t* seqlens_k;
    const uint8_t* block_mask; /* NULL: no block mask */
} mask_spec;

/* the allowed keys of row i of head g lie in [lo, hi) (and pass allowed_block) */
static void key_range(const mask_spec* ms, int64_t g, int64_t i, int64_t* lo, int64_t* hi) {
    int64_t a = ms->window_left >= 0 ? i - ms->window_left : 0;
    int64_t b = ms->window_right >= 0 ? i + ms->window_right + 1 : ms->N;
    const int64_t kv_len = ms->seqlens_k ? ms->seqlens_k[g / ms->H] : ms->N;
    *lo = a < 0 ? 0 : a;
    *hi = b > kv_len ? kv_len : b;
}
static int allowed_block(const mask_spec* ms, int64_t g, int64_t i, int64_t j) {
    if (!ms->block_mask) return 1;
    return ms->block_mask[(g / ms->H) * ms->stride_b + (g % ms->H) * ms->stride_h +
                          (i / ms->block_q) * ms->n_kb + j / ms->block_k] != 0;
}

static int bwd_general(const double* q, const double* k, const double* v, const double* dout,
                       double* dq, double* dk, double* dv, double* lse, double* delta,
                       int64_t B, int64_t H, int64_t N, int64_t d, double scale, const mask_spec* ms,
                       const int64_t* rows, int64_t n_rows, const int64_t* keys, int64_t n_keys) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 1 || H < 1 || N < 1 || d < 1) return 1;
    if (ms->window_left < -1 || ms->window_right < -1) return 1;
    const int64_t G = B * H;
    int64_t R = rows ? n_rows : N;
    int64_t C = keys ? n_keys : N;
    if (R < 1 || C < 1) return 1;
    for (int64_t t = 0; rows && t < G * n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= N) return 1;
    for (int64_t t = 0; keys && t < G * n_keys; ++t)
        if (keys[t] < 0 || keys[t] >= N) return 1;
    for (int64_t b = 0; ms->seqlens_k && b < B; ++b)
        if (ms->seqlens_k[b] < 0 || ms->seqlens_k[b] > N) return 1;
    int nthreads = fa_oracle_threads();
    double* m_all = (double*)malloc((size_t)(G * N) * sizeof(double));
    double* l_all = (double*)malloc((size_t)(G * N) * sizeof(double));
    double* D_all = (double*)malloc((size_t)(G * N) * sizeof(double));
    double* s_all = (double*)malloc((size_t)nthreads * (size_t)N * sizeof(double));
    if (!m_all || !l_all || !D_all || !s_all) {
        free(m_all); free(l_all); free(D_all); free(s_all);
        return 2;
    }

    /* pass 1, every row: m_i, l_i (three-pass route over the allowed keys) and D_i */
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t t = 0; t < G * N; ++t) {
#ifdef _OPENMP
        int tid = omp_get_thread_num();
#else
        int tid = 0;
#endif
        double* s = s_all + (size_t)tid * (size_t)N;
        int64_t g = t / N, i = t % N, lo, hi;
        key_range(ms, g, i, &lo, &hi);
        const double* qi = q + t * d;
        const double* doi = dout + t * d;
        const double* kh = k + g * N * d;
        const double* vh = v + g * N * d;
        double m = -INFINITY, l = 0.0, D = 0.0;
        int64_t n_allowed = 0;
        for (int64_t j = lo; j < hi; ++j) {
            if (!allowed_block(ms, g, i, j)) continue;
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
            s[j] = scale * dot;
            if (s[j] > m) m = s[j];
            ++n_allowed;
        }
        for (int64_t j = lo; j < hi; ++j)
            if (allowed_block(ms, g, i, j)) l += exp(s[j] - m);
        for (int64_t j = lo; j < hi; ++j) {
            if (!allowed_block(ms, g, i, j)) continue;
            double dp = 0.0;
            for (int64_t c = 0; c < d; ++c) dp += doi[c] * vh[j * d + c];
            D += (exp(s[j] - m) / l) * dp;
        }
        m_all[t] = m;
        l_all[t] = l;
        D_all[t] = D;
        if (lse) lse[t] = n_allowed > 0 ? m + log(l) : -INFINITY;
        if (delta) delta[t] = D;
    }

    /* pass 2, requested rows: dQ_i = scale * sum_j a_ij (dP_ij - D_i) k_j over the allowed j */
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t t = 0; t < G * R; ++t) {
        int64_t g = t / R, r = t % R;
        int64_t i = rows ? rows[g * n_rows + r] : r, lo, hi;
        key_range(ms, g, i, &lo, &hi);
        const double* qi = q + (g * N + i) * d;
        const double* doi = dout + (g * N + i) * d;
        const double* kh = k + g * N * d;
        const double* vh = v + g * N * d;
        double m = m_all[g * N + i], l = l_all[g * N + i], D = D_all[g * N + i];
        double* out = dq + t * d;
        for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
        for (int64_t j = lo; j < hi; ++j) {
            if (!allowed_block(ms, g, i, j)) continue;
            double dot = 0.0, dpv = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * kh[j * d + c];
            for (int64_t c = 0; c < d; ++c) dpv += doi[c] * vh[j * d + c];
            double ds = exp(scale * dot - m) / l * (dpv - D);
            for (int64_t c = 0; c < d; ++c) out[c] += ds * kh[j * d + c];
        }
        for (int64_t c = 0; c < d; ++c) out[c] *= scale;
    }

    /* pass 3, requested keys: dV_j = sum_i a_ij dO_i, dK_j = scale * sum_i a_ij (dP_ij - D_i) q_i
       over the rows i that allow key j */
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
    for (int64_t t = 0; t < G * C; ++t) {
        int64_t g = t / C, r = t % C;
        int64_t j = keys ? keys[g * n_keys + r] : r;
        const double* kj = k + (g * N + j) * d;
        const double* vj = v + (g * N + j) * d;
        double* ok = dk + t * d;
        double* ov = dv + t * d;
        for (int64_t c = 0; c < d; ++c) ok[c] = ov[c] = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            int64_t lo, hi;
            key_range(ms, g, i, &lo, &hi);
            if (j < lo || j >= hi || !allowed_block(ms, g, i, j)) continue;
            const double* qi = q + (g * N + i) * d;
            const double* doi = dout + (g * N + i) * d;
            double dot = 0.0, dpv = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
            for (int64_t c = 0; c < d; ++c) dpv += doi[c] * vj[c];
            double a = exp(scale * dot - m_all[g * N + i]) / l_all[g * N + i];
            double ds = a * (dpv - D_all[g * N + i]);
            for (int64_t c = 0; c < d; ++c) {
                ov[c] += a * doi[c];
                ok[c] += ds * qi[c];
            }
        }
        for (int64_t c = 0; c < d; ++c) ok[c] *= scale;
    }
    free(m_all); free(l_all); free(D_all); free(s_all);
    return 0;
}

/*
 * fa_oracle_bwd_masked: the gradients under the window / key-length mask. Arguments as
 * fa_oracle_bwd, with G replaced by B, H (rows and keys are [B*H, ...]) and causal by
 * window_left, window_right and seqlens_k (host pointer, [B], or NULL). Same return codes.
 */
int fa_oracle_bwd_masked(const double* q, const double* k, const double* v, const double* dout,
                         double* dq, double* dk, double* dv, double* lse, double* delta,
                         int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                         int64_t window_left, int64_t window_right, const int64_t* seqlens_k,
                         const int64_t* rows, int64_t n_rows, const int64_t* keys, int64_t n_keys) {
    mask_spec ms = {H, N, window_left, window_right, 1, 1, 0, 0, 0, seqlens_k, NULL};
    return bwd_general(q, k, v, dout, dq, dk, dv, lse, delta, B, H, N, d, scale, &ms, rows, n_rows, keys,
                       n_keys);
}

/*
 * fa_oracle_bwd_blocksparse: the gradients under the block mask of fa_oracle_fwd_blocksparse
 * on top of the window / key-length mask. Arguments as fa_oracle_bwd_masked, plus block_mask
 * (host pointer), block_q, block_k >= 1 and stride_b, stride_h >= 0. Same return codes.
 */
int fa_oracle_bwd_blocksparse(const double* q, const double* k, const double* v, const double* dout,
                              double* dq, double* dk, double* dv, double* lse, double* delta,
                              int64_t B, int64_t H, int64_t N, int64_t d, double scale,
                              int64_t window_left, int64_t window_right, const int64_t* seqlens_k,
                              const uint8_t* block_mask, int64_t block_q, int64_t block_k,
                              int64_t stride_b, int64_t stride_h,
                              const int64_t* rows, int64_t n_rows, const int64_t* keys, int64_t n_keys) {
    if (!block_mask || block_q < 1 || block_k < 1 || stride_b < 0 || stride_h < 0) return 1;
    mask_spec ms = {H, N, window_left, window_right, block_q, block_k, (N + block_k - 1) / block_k,
                    stride_b, stride_h, seqlens_k, block_mask};
    return bwd_general(q, k, v, dout, dq, dk, dv, lse, delta, B, H, N, d, scale, &ms, rows, n_rows, keys,
                       n_keys);
}
