// Attention forward on the host CPU (fa_cpu.h): the tiled online-softmax recurrence of
// "transformer math: flash attention math" (aicassindra.com, "The block-wise update, and the full
// algorithm"), run, as that page's "Why the same math matters on a CPU" describes, so that one
// query tile's scores and running state stay in cache while key and value blocks stream through.
//
// Per (head, tile of 32 query rows), one thread keeps in fp32: the query rows pre-multiplied by
// scale * log2(e) (scores come out in log2 units), the running max m, denominator l and
// unnormalised output o~ of each row, and one block of 64 keys and values converted from f16/bf16.
// For each block: S = Q K^T, mask, then per row m_new = max(m, max_j s), alpha = 2^(m - m_new),
// p = 2^(s - m_new), l = alpha l + sum p, o~ = alpha o~ + p V, m = m_new (the loop of the page,
// in base 2). At the end o = o~ / l and lse = (m + log2 l) ln 2. Every loop over d or over the
// block runs in SIMD lanes; an AVX-512 or AVX2/FMA/F16C build of the tile loop is chosen at run
// time.

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <exception>
#include <thread>
#include <vector>

#include <immintrin.h>

#include "fa_cpu.h"

namespace {

constexpr int kBQ = 32;  // query rows per tile
constexpr int kBK = 64;  // keys per block

inline float bits_to_f32(uint32_t b) {
    float f;
    memcpy(&f, &b, 4);
    return f;
}
inline uint32_t f32_to_bits(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    return b;
}

// Exact widening of IEEE binary16 (normal, subnormal, inf, nan).
inline float f16_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    if (e == 0) {
        const float f = (float)m * 5.9604644775390625e-8f;  // m * 2^-24, exact
        return sign ? -f : f;
    }
    if (e == 31) return bits_to_f32(sign | 0x7f800000u | (m << 13));
    return bits_to_f32(sign | ((e + 112u) << 23) | (m << 13));
}
inline float bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

// fp32 -> binary16, round to nearest even (overflow to inf, subnormals kept).
inline uint16_t f32_to_f16(float f) {
    const uint32_t x = f32_to_bits(f);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u) return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
    if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  // >= 65520 rounds to inf
    if (ax < 0x38800000u) {                                      // below 2^-14: subnormal or 0
        const uint32_t m = (uint32_t)nearbyintf(bits_to_f32(ax) * 16777216.0f);  // / 2^-24, RNE
        return (uint16_t)(sign | m);
    }
    uint32_t r = (((ax >> 23) - 112u) << 10) | ((ax & 0x7fffffu) >> 13);
    const uint32_t rem = ax & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) r += 1u;  // a carry moves the exponent
    return (uint16_t)(sign | r);
}
// fp32 -> bfloat16, round to nearest even (nan stays nan).
inline uint16_t f32_to_bf16(float f) {
    const uint32_t x = f32_to_bits(f);
    if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
    return (uint16_t)((x + 0x7fffu + ((x >> 16) & 1u)) >> 16);
}

// 2^x for x <= 0 (x = -inf gives 0): x = n + f with n = round(x), |f| <= 1/2, and
// 2^f = e^t, t = f ln 2, by its Taylor series to t^7 (truncation below 6e-9 for |t| <= 0.35);
// 2^n is built in the exponent field. Below 2^-126 the result is flushed to 0.
inline float exp2_nonpos(float x) {
    const float xc = x < -126.0f ? -126.0f : x;
    const float n = nearbyintf(xc);
    const float t = (xc - n) * 0.693147180559945309f;
    float p = 1.0f + t * (1.0f / 7.0f);
    p = 1.0f + t * (1.0f / 6.0f) * p;
    p = 1.0f + t * (1.0f / 5.0f) * p;
    p = 1.0f + t * (1.0f / 4.0f) * p;
    p = 1.0f + t * (1.0f / 3.0f) * p;
    p = 1.0f + t * (1.0f / 2.0f) * p;
    p = 1.0f + t * p;
    const float two_n = bits_to_f32((uint32_t)((int32_t)n + 127) << 23);
    return x < -126.0f ? 0.0f : p * two_n;
}

struct Scratch {
    std::vector<float> q, kt, vf, s, acc;  // kt: the key block transposed, [d][kBK]
    float m[kBQ], l[kBQ];
    explicit Scratch(int d) : q((size_t)kBQ * d), kt((size_t)kBK * d), vf((size_t)kBK * d), s((size_t)kBQ * kBK),
                              acc((size_t)kBQ * d) {}
};

// n binary16 values (n a multiple of 8) -> fp32, times mul, with the F16C conversion
__attribute__((target("avx2,fma,f16c"))) inline void widen_f16_f16c(const uint16_t* in, float* out, int n, float mul) {
    for (int c = 0; c < n; c += 8) {
        const __m256 w = _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i*>(in + c)));
        _mm256_storeu_ps(out + c, _mm256_mul_ps(w, _mm256_set1_ps(mul)));
    }
}

// rows [r0, r0 + n) of one [N, D] tensor of one head -> fp32 rows of `dst` (missing rows zero)
template <int D, bool BF16, bool F16C>
__attribute__((always_inline)) inline void widen_rows(const uint16_t* src, int r0, int n, int N, float* dst, float mul) {
    for (int r = 0; r < n; ++r) {
        float* out = dst + (size_t)r * D;
        if (r0 + r >= N) {
            for (int c = 0; c < D; ++c) out[c] = 0.0f;
            continue;
        }
        const uint16_t* in = src + (size_t)(r0 + r) * D;
        if constexpr (BF16) {
#pragma omp simd
            for (int c = 0; c < D; ++c) out[c] = bf16_to_f32(in[c]) * mul;
        } else if constexpr (F16C) {
            widen_f16_f16c(in, out, D, mul);
        } else {
            for (int c = 0; c < D; ++c) out[c] = f16_to_f32(in[c]) * mul;
        }
    }
}

// the same rows written transposed: dst[c * kBK + r] (missing rows zero)
template <int D, bool BF16, bool F16C>
__attribute__((always_inline)) inline void widen_rows_t(const uint16_t* src, int r0, int n, int N, float* dst,
                                                        float* row_buf) {
    widen_rows<D, BF16, F16C>(src, r0, n, N, row_buf, 1.0f);
    for (int r = n; r < kBK; ++r)
        for (int c = 0; c < D; ++c) row_buf[(size_t)r * D + c] = 0.0f;
    for (int r = 0; r < kBK; ++r)
        for (int c = 0; c < D; ++c) dst[(size_t)c * kBK + r] = row_buf[(size_t)r * D + c];
}

// One (head, query tile): rows q0 .. q0 + 31 of head `bh`.
template <int D, bool BF16, bool CAUSAL, bool F16C>
__attribute__((always_inline)) inline void tile(const uint16_t* Q, const uint16_t* K, const uint16_t* V, uint16_t* O,
                                                float* LSE, int64_t bh, int q0, int N, float c, Scratch& w) {
    const int64_t head = bh * (int64_t)N * D;
    const int nq = std::min(kBQ, N - q0);
    widen_rows<D, BF16, F16C>(Q + head, q0, nq, N, w.q.data(), c);  // scores come out in log2 units
    for (int i = 0; i < kBQ; ++i) {
        w.m[i] = -INFINITY;
        w.l[i] = 0.0f;
    }
    std::fill(w.acc.begin(), w.acc.end(), 0.0f);
    const int kv_end = CAUSAL ? std::min(N, q0 + nq) : N;
    for (int k0 = 0; k0 < kv_end; k0 += kBK) {
        const int nk = std::min(kBK, kv_end - k0);
        widen_rows_t<D, BF16, F16C>(K + head, k0, nk, N, w.kt.data(), w.vf.data());  // vf as staging
        widen_rows<D, BF16, F16C>(V + head, k0, nk, N, w.vf.data(), 1.0f);
        // S = Q K^T for the block, two rows at a time, vectorised over the 64 keys: each column of
        // K^T feeds both rows (no horizontal sums)
        for (int i = 0; i < nq; i += 2) {
            const float* q0r = w.q.data() + (size_t)i * D;
            const float* q1r = w.q.data() + (size_t)std::min(i + 1, kBQ - 1) * D;
            float a0[kBK], a1[kBK];
#pragma omp simd
            for (int j = 0; j < kBK; ++j) a0[j] = a1[j] = 0.0f;
            for (int cc = 0; cc < D; ++cc) {
                const float x0 = q0r[cc], x1 = q1r[cc];
                const float* kc = w.kt.data() + (size_t)cc * kBK;
#pragma omp simd
                for (int j = 0; j < kBK; ++j) {
                    a0[j] += x0 * kc[j];
                    a1[j] += x1 * kc[j];
                }
            }
            float* s0 = w.s.data() + (size_t)i * kBK;
#pragma omp simd
            for (int j = 0; j < kBK; ++j) s0[j] = a0[j];
            if (i + 1 < kBQ) {
                float* s1 = w.s.data() + (size_t)(i + 1) * kBK;
#pragma omp simd
                for (int j = 0; j < kBK; ++j) s1[j] = a1[j];
            }
        }
        for (int i = 0; i < nq; ++i) {
            float* si = w.s.data() + (size_t)i * kBK;
            const int row = q0 + i;
            // masked keys (after the row, or past the block) are -inf before the max
            for (int j = 0; j < kBK; ++j) {
                const bool allowed = j < nk && (!CAUSAL || k0 + j <= row);
                si[j] = allowed ? si[j] : -INFINITY;
            }
            float mx = -INFINITY;
#pragma omp simd reduction(max : mx)
            for (int j = 0; j < kBK; ++j) mx = std::max(mx, si[j]);
            const float m_new = std::max(w.m[i], mx);
            if (m_new == -INFINITY) continue;  // nothing allowed yet: the state stays empty
            const float alpha = exp2_nonpos(w.m[i] - m_new);  // 0 when m was -inf
            float sum = 0.0f;
#pragma omp simd reduction(+ : sum)
            for (int j = 0; j < kBK; ++j) {
                si[j] = exp2_nonpos(si[j] - m_new);
                sum += si[j];
            }
            w.l[i] = alpha * w.l[i] + sum;
            w.m[i] = m_new;
            float* ai = w.acc.data() + (size_t)i * D;
#pragma omp simd
            for (int cc = 0; cc < D; ++cc) ai[cc] *= alpha;
            for (int j = 0; j < nk; ++j) {
                const float pj = si[j];
                const float* vj = w.vf.data() + (size_t)j * D;
#pragma omp simd
                for (int cc = 0; cc < D; ++cc) ai[cc] += pj * vj[cc];
            }
        }
    }
    for (int i = 0; i < nq; ++i) {
        const float inv = 1.0f / w.l[i];  // every row keeps key 0
        const float* ai = w.acc.data() + (size_t)i * D;
        uint16_t* oi = O + head + (int64_t)(q0 + i) * D;
        for (int cc = 0; cc < D; ++cc) oi[cc] = BF16 ? f32_to_bf16(ai[cc] * inv) : f32_to_f16(ai[cc] * inv);
        if (LSE) LSE[bh * N + q0 + i] = (w.m[i] + log2f(w.l[i])) * 0.693147180559945309f;
    }
}

// ---- AVX-512 build of the tile -----------------------------------------------------------------
// The scores come out transposed, S^T[j][i] = sum_c K[j][c] q_i[c], vectorised over the 32 query
// rows of the tile (two 16-lane registers): K is used in its natural row layout (no transpose per
// block) and the softmax updates (max, exponentials, sums) run across rows in lanes, with no
// horizontal reduction. The product with V is blocked over 2 rows (4 when d = 64) times the whole
// head dimension, held in registers for the 64 keys of the block.
#define FA_AVX512 __attribute__((target("avx512f,avx512bw,avx512dq,avx512vl,fma,f16c")))

template <bool BF16>
FA_AVX512 inline __m512 widen16(const uint16_t* p) {
    const __m256i h = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(p));
    if constexpr (BF16) return _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(h), 16));
    else return _mm512_cvtph_ps(h);  // exact, subnormals included
}

// exp2_nonpos in 16 lanes: the same reduction and series; 2^n applied by vscalefps
FA_AVX512 inline __m512 exp2_nonpos16(__m512 x) {
    const __m512 lo = _mm512_set1_ps(-126.0f);
    const __mmask16 keep = _mm512_cmp_ps_mask(x, lo, _CMP_GE_OQ);  // x >= -126 (not -inf, not nan)
    const __m512 xc = _mm512_max_ps(x, lo);
    const __m512 n = _mm512_roundscale_ps(xc, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    const __m512 t = _mm512_mul_ps(_mm512_sub_ps(xc, n), _mm512_set1_ps(0.693147180559945309f));
    const __m512 one = _mm512_set1_ps(1.0f);
    __m512 p = _mm512_fmadd_ps(t, _mm512_set1_ps(1.0f / 7.0f), one);
    p = _mm512_fmadd_ps(_mm512_mul_ps(t, _mm512_set1_ps(1.0f / 6.0f)), p, one);
    p = _mm512_fmadd_ps(_mm512_mul_ps(t, _mm512_set1_ps(1.0f / 5.0f)), p, one);
    p = _mm512_fmadd_ps(_mm512_mul_ps(t, _mm512_set1_ps(1.0f / 4.0f)), p, one);
    p = _mm512_fmadd_ps(_mm512_mul_ps(t, _mm512_set1_ps(1.0f / 3.0f)), p, one);
    p = _mm512_fmadd_ps(_mm512_mul_ps(t, _mm512_set1_ps(1.0f / 2.0f)), p, one);
    p = _mm512_fmadd_ps(t, p, one);
    return _mm512_maskz_mov_ps(keep, _mm512_scalef_ps(p, n));
}

template <int D, bool BF16, bool CAUSAL>
FA_AVX512 void tile_avx512(const uint16_t* Q, const uint16_t* K, const uint16_t* V, uint16_t* O, float* LSE,
                           int64_t bh, int q0, int N, float c, Scratch& w) {
    static_assert(kBQ == 32 && kBK % 8 == 0 && D % 16 == 0, "tile shape");
    constexpr int RB = D == 64 ? 4 : 2;  // rows per register block of the product with V
    const int64_t head = bh * (int64_t)N * D;
    const int nq = std::min(kBQ, N - q0);
    float* qt = w.q.data();   // Q^T [D][32], times scale * log2(e); missing rows are zero
    float* kr = w.kt.data();  // the key block, fp32 rows [kBK][D]
    float* vr = w.vf.data();  // the value block, fp32 rows [kBK][D]
    float* st = w.s.data();   // S^T, then P^T, [kBK][32]
    float* acc = w.acc.data();
    // Q rows -> fp32 (through acc as staging) -> transposed into qt
    for (int r = 0; r < kBQ; ++r)
        for (int cc = 0; cc < D; cc += 16)
            _mm512_storeu_ps(acc + r * D + cc, r < nq ? _mm512_mul_ps(widen16<BF16>(Q + head + (int64_t)(q0 + r) * D + cc),
                                                                       _mm512_set1_ps(c))
                                                       : _mm512_setzero_ps());
    for (int cc = 0; cc < D; ++cc)
        for (int r = 0; r < kBQ; ++r) qt[cc * kBQ + r] = acc[r * D + cc];
    for (int i = 0; i < kBQ * D; i += 16) _mm512_storeu_ps(acc + i, _mm512_setzero_ps());
    for (int i = 0; i < kBQ; ++i) {
        w.m[i] = -INFINITY;
        w.l[i] = 0.0f;
    }
    alignas(64) float alpha[kBQ];
    const int kv_end = CAUSAL ? std::min(N, q0 + nq) : N;
    for (int k0 = 0; k0 < kv_end; k0 += kBK) {
        const int nk = std::min(kBK, kv_end - k0);
        for (int r = 0; r < kBK; ++r)
            for (int cc = 0; cc < D; cc += 16) {
                const bool in = r < nk;
                _mm512_storeu_ps(kr + r * D + cc, in ? widen16<BF16>(K + head + (int64_t)(k0 + r) * D + cc)
                                                     : _mm512_setzero_ps());
                _mm512_storeu_ps(vr + r * D + cc, in ? widen16<BF16>(V + head + (int64_t)(k0 + r) * D + cc)
                                                     : _mm512_setzero_ps());
            }
        // S^T = K Q^T: 8 keys x 32 rows in 16 accumulators per pass over the head dimension
        const int nkb = (nk + 7) & ~7;
        for (int jb = 0; jb < nkb; jb += 8) {
            __m512 a[8][2];
            for (int u = 0; u < 8; ++u) a[u][0] = a[u][1] = _mm512_setzero_ps();
            const float* k8 = kr + jb * D;
            for (int cc = 0; cc < D; ++cc) {
                const __m512 x0 = _mm512_loadu_ps(qt + cc * kBQ), x1 = _mm512_loadu_ps(qt + cc * kBQ + 16);
                for (int u = 0; u < 8; ++u) {
                    const __m512 kb = _mm512_set1_ps(k8[u * D + cc]);
                    a[u][0] = _mm512_fmadd_ps(kb, x0, a[u][0]);
                    a[u][1] = _mm512_fmadd_ps(kb, x1, a[u][1]);
                }
            }
            for (int u = 0; u < 8; ++u) {
                _mm512_storeu_ps(st + (jb + u) * kBQ, a[u][0]);
                _mm512_storeu_ps(st + (jb + u) * kBQ + 16, a[u][1]);
            }
        }
        // mask (keys after the row, or past the block) to -inf, then per row: max, alpha, p, l
        for (int hh = 0; hh < 2; ++hh) {
            const __m512i rows = _mm512_add_epi32(_mm512_set1_epi32(q0 + 16 * hh),
                                                  _mm512_setr_epi32(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
            const __m512 ninf = _mm512_set1_ps(-INFINITY);
            __m512 mx = ninf;
            for (int j = 0; j < nk; ++j) {
                __m512 sv = _mm512_loadu_ps(st + j * kBQ + 16 * hh);
                if constexpr (CAUSAL) {
                    const __mmask16 after = _mm512_cmpgt_epi32_mask(_mm512_set1_epi32(k0 + j), rows);
                    sv = _mm512_mask_mov_ps(sv, after, ninf);
                    _mm512_storeu_ps(st + j * kBQ + 16 * hh, sv);
                }
                mx = _mm512_max_ps(mx, sv);
            }
            const __m512 m_old = _mm512_loadu_ps(w.m + 16 * hh);
            const __m512 m_new = _mm512_max_ps(m_old, mx);
            // rows with nothing allowed yet keep m = -inf; subtracting 0 then gives p = alpha = 0
            const __m512 m_sub = _mm512_mask_mov_ps(m_new, _mm512_cmp_ps_mask(m_new, ninf, _CMP_EQ_OQ),
                                                    _mm512_setzero_ps());
            const __m512 al = exp2_nonpos16(_mm512_sub_ps(m_old, m_sub));
            __m512 sum = _mm512_setzero_ps();
            for (int j = 0; j < nk; ++j) {
                const __m512 pv = exp2_nonpos16(_mm512_sub_ps(_mm512_loadu_ps(st + j * kBQ + 16 * hh), m_sub));
                _mm512_storeu_ps(st + j * kBQ + 16 * hh, pv);
                sum = _mm512_add_ps(sum, pv);
            }
            _mm512_storeu_ps(w.l + 16 * hh, _mm512_fmadd_ps(al, _mm512_loadu_ps(w.l + 16 * hh), sum));
            _mm512_storeu_ps(w.m + 16 * hh, m_new);
            _mm512_store_ps(alpha + 16 * hh, al);
        }
        // o~ = alpha o~ + P V, RB rows at a time with the whole head dimension in registers
        for (int i = 0; i < nq; i += RB) {
            __m512 o[RB][D / 16];
            for (int r = 0; r < RB; ++r) {
                const int ri = std::min(i + r, kBQ - 1);
                const __m512 a = _mm512_set1_ps(alpha[ri]);
                for (int u = 0; u < D / 16; ++u) o[r][u] = _mm512_mul_ps(a, _mm512_loadu_ps(acc + ri * D + 16 * u));
            }
            for (int j = 0; j < nk; ++j) {
                const float* pj = st + j * kBQ;
                const float* vj = vr + j * D;
                __m512 pr[RB];
                for (int r = 0; r < RB; ++r) pr[r] = _mm512_set1_ps(pj[std::min(i + r, kBQ - 1)]);
                for (int u = 0; u < D / 16; ++u) {
                    const __m512 vv = _mm512_loadu_ps(vj + 16 * u);
                    for (int r = 0; r < RB; ++r) o[r][u] = _mm512_fmadd_ps(pr[r], vv, o[r][u]);
                }
            }
            for (int r = 0; r < RB; ++r)
                if (i + r < nq)
                    for (int u = 0; u < D / 16; ++u) _mm512_storeu_ps(acc + (i + r) * D + 16 * u, o[r][u]);
        }
    }
    for (int i = 0; i < nq; ++i) {
        const float inv = 1.0f / w.l[i];  // every row keeps key 0
        const float* ai = acc + (size_t)i * D;
        uint16_t* oi = O + head + (int64_t)(q0 + i) * D;
        for (int cc = 0; cc < D; ++cc) oi[cc] = BF16 ? f32_to_bf16(ai[cc] * inv) : f32_to_f16(ai[cc] * inv);
        if (LSE) LSE[bh * N + q0 + i] = (w.m[i] + log2f(w.l[i])) * 0.693147180559945309f;
    }
}

template <int D, bool BF16, bool CAUSAL>
__attribute__((target("avx2,fma,f16c"))) void tile_avx2(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                                         uint16_t* O, float* LSE, int64_t bh, int q0, int N, float c,
                                                         Scratch& w) {
    tile<D, BF16, CAUSAL, true>(Q, K, V, O, LSE, bh, q0, N, c, w);
}
template <int D, bool BF16, bool CAUSAL>
void tile_generic(const uint16_t* Q, const uint16_t* K, const uint16_t* V, uint16_t* O, float* LSE, int64_t bh,
                  int q0, int N, float c, Scratch& w) {
    tile<D, BF16, CAUSAL, false>(Q, K, V, O, LSE, bh, q0, N, c, w);
}

using TileFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, float*, int64_t, int, int, float,
                        Scratch&);

// instruction sets of the tile loop: 2 = AVX-512, 1 = AVX2/FMA/F16C, 0 = plain C++
template <int D, bool BF16>
TileFn pick(bool causal, int isa) {
    if (isa == 2) return causal ? tile_avx512<D, BF16, true> : tile_avx512<D, BF16, false>;
    if (isa == 1) return causal ? tile_avx2<D, BF16, true> : tile_avx2<D, BF16, false>;
    return causal ? tile_generic<D, BF16, true> : tile_generic<D, BF16, false>;
}

// The best build this CPU runs; FA_CPU_ISA=avx2 or =generic selects a lower one (used by the
// tests to cover every build on one machine).
int pick_isa() {
    static const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
                             __builtin_cpu_supports("f16c");
    static const bool avx512 = avx2 && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                               __builtin_cpu_supports("avx512dq") && __builtin_cpu_supports("avx512vl");
    int isa = avx512 ? 2 : avx2 ? 1 : 0;
    if (const char* e = getenv("FA_CPU_ISA")) {
        if (strcmp(e, "generic") == 0) isa = 0;
        else if (strcmp(e, "avx2") == 0 && isa > 1) isa = 1;
    }
    return isa;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" int fa_fwd_cpu(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                          int64_t N, int64_t d, float scale, int causal, fa_dtype dtype, int num_threads) {
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || N > INT32_MAX / 2) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (B * H > INT64_MAX / N / d / 2) return FA_ERR_SHAPE;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
    const size_t nb = (size_t)(B * H * N * d * 2), lb = (size_t)(B * H * N * 4);
    if (overlaps(o, nb, q, nb) || overlaps(o, nb, k, nb) || overlaps(o, nb, v, nb) ||
        (lse && (overlaps(lse, lb, q, nb) || overlaps(lse, lb, k, nb) || overlaps(lse, lb, v, nb) ||
                 overlaps(lse, lb, o, nb))))
        return FA_ERR_ALIAS;

    const int isa = pick_isa();
    const bool bf = dtype == FA_BF16;
    const TileFn fn = d == 64 ? (bf ? pick<64, true>(causal, isa) : pick<64, false>(causal, isa))
                              : (bf ? pick<128, true>(causal, isa) : pick<128, false>(causal, isa));
    const int n = (int)N;
    const int64_t n_qt = (N + kBQ - 1) / kBQ;
    const int64_t items = B * H * n_qt;
    int threads = num_threads > 0 ? num_threads : (int)std::max(1u, std::thread::hardware_concurrency());
    threads = (int)std::min<int64_t>(threads, items);
    const float c = scale * 1.4426950408889634f;
    const auto* Q = static_cast<const uint16_t*>(q);
    const auto* K = static_cast<const uint16_t*>(k);
    const auto* V = static_cast<const uint16_t*>(v);
    auto* O = static_cast<uint16_t*>(o);

    // Work items are (head, query tile), taken in order from a shared counter; causal tiles are
    // taken longest (last) first so the short ones fill in at the end.
    std::atomic<int64_t> next{0};
    std::atomic<bool> failed{false};
    auto worker = [&]() {
        try {
            Scratch w((int)d);
            for (int64_t t = next.fetch_add(1); t < items; t = next.fetch_add(1)) {
                const int64_t bh = t / n_qt;
                const int64_t qt = causal ? n_qt - 1 - t % n_qt : t % n_qt;
                fn(Q, K, V, O, lse, bh, (int)(qt * kBQ), n, c, w);
            }
        } catch (...) {
            failed = true;
        }
    };
    std::vector<std::thread> pool;
    try {
        for (int i = 1; i < threads; ++i) pool.emplace_back(worker);
    } catch (...) {
        failed = true;
    }
    worker();
    for (auto& th : pool) th.join();
    return failed ? FA_ERR_LAUNCH : FA_OK;
}
