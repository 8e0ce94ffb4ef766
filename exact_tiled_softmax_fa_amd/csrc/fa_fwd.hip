// Exact tiled-softmax attention forward for gfx950 (CDNA4), behind the C ABI of fa_fwd.h.
//
// One workgroup = 4 waves = 128 query rows of one (batch, head); each wave owns 32 rows.
// The workgroup walks the keys in tiles of 64 (ascending), staging each K and V tile in LDS
// with coalesced 16-byte global loads that are issued one tile ahead. Per tile and wave:
//
//   S^T = K_tile . Q^T          v_mfma_f32_32x32x16_{f16,bf16}, fp32 accumulate.
//                               Computing the transpose puts one query row in each lane
//                               (lanes l and l+32 hold the same row, different keys), so
//                               the row max and row sum are in-lane work plus one
//                               cross-half exchange (v_permlane32_swap).
//   mask                        only on tiles that cross the causal diagonal or the end of
//                               the sequence; masked scores become -inf before the max.
//   m, alpha, p, l              online softmax in log2 units: p = exp2(s*c - m*c), with
//                               c = scale*log2(e) folded into one fma.
//   O^T += V_tile^T . P^T       P converted to f16/bf16 (round to nearest even) straight
//                               from the S^T accumulator registers, which already have the
//                               operand layout; V^T comes from ds_read_b64_tr_b16 on the
//                               row-major V tile.
//
// The recurrence is the one on "transformer math: flash attention math" (aicassindra.com),
// section "The block-wise update, and the full algorithm", run for a tile of queries at once
// as that section describes; the tiling and the fact that score tiles die on chip are the
// mechanism of "FlashAttention tiles exact softmax without materializing the score matrix"
// (nalar.dev), sections "A score tile is temporary state" and "IO behavior is the mechanism".
// Fewer rescales (a wave skips the alpha multiply when no row's max moved) follow the
// FlashAttention-2 remark on "Decoding flash attention" (bibekananda.in), "Later versions".

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa_fwd.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockM = 32 * kWaves;  // query rows per workgroup
constexpr int kBlockN = 64;           // keys per tile
constexpr int kXcds = 8;              // MI355X: workgroups are dealt round-robin to 8 XCDs

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// Two fp32 values -> one packed pair, each rounded to nearest even.
template <bool BF16>
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
    if constexpr (BF16) {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(unsigned, v);
    } else {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(unsigned, v);
    }
}

// acc + lo + hi of a packed pair (the rounded probabilities, so the denominator sums exactly
// the weights the second product uses).
template <bool BF16>
__device__ __forceinline__ float add_pair(unsigned packed, float acc) {
    if constexpr (BF16) {
        const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
    } else {
        const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, acc, false);
    }
}

// Value held by the lane 32 positions away (same query row, other half of the keys).
__device__ __forceinline__ float max_with_partner(float x) {
    unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
    unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup -> (head, query tile). Workgroups are dealt to XCDs round-robin, so block b runs on
// XCD b % 8. Non-causal: give each XCD a contiguous range of (head, tile) pairs, so the
// workgroups resident on one XCD at a time share one head's K/V in that XCD's L2. Causal: each
// XCD owns whole heads and starts with their longest query tiles (most keys) so the short ones
// fill in at the end.
__device__ __forceinline__ void map_block(int bid, int G, int n_qt, bool causal, int& bh, int& qt) {
    if (G % kXcds == 0) {
        const int per = G / kXcds;
        const int x = bid % kXcds, s = bid / kXcds;
        if (!causal) {
            const int w = x * per + s;
            bh = w / n_qt;
            qt = w % n_qt;
            return;
        }
        if (per % n_qt == 0) {
            const int hpx = per / n_qt;
            qt = n_qt - 1 - s / hpx;
            bh = x * hpx + s % hpx;
            return;
        }
    }
    bh = bid / n_qt;
    qt = causal ? n_qt - 1 - bid % n_qt : bid % n_qt;
}

// K and V tiles live in LDS as kBlockN rows of D elements (no padding); the 16-byte chunk c of
// row r is stored at chunk position c ^ swz(r). Both read patterns are then free of bank
// conflicts: the K operand reads one chunk from each of 16 consecutive rows, and the V^T
// transpose read takes 4 consecutive chunks from each of 4 consecutive rows.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);  // 16 chunks per row
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);              // 8 chunks per row
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {  // element offset of (row, chunk)
    return r * D + ((c ^ swz<D>(r)) << 3);
}

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_qt, int G, float c, float tau_raw) {
    constexpr int DK = D / 16;                 // k-steps of the first product
    constexpr int DB = D / 32;                 // 32-column blocks of the output
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;              // rows one wave-wide 1 KiB load covers
    constexpr int IPW = kBlockN / RPI / kWaves;  // such loads per wave per tile (each of K, V)
    constexpr int TILE = kBlockN * D;          // elements per tile
    static_assert(IPW * RPI * kWaves == kBlockN, "tile must split evenly over the waves");

    // Two buffers each for K and V: tile j is read from buffer j % 2 while tile j + 1 streams
    // into the other one straight from global memory (global_load_lds, no register staging).
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;   // which half of the keys of a 32-key block this lane holds
    const int lq = lane & 31;  // query row within the wave

    int bh, qt;
    map_block(blockIdx.x, G, n_qt, CAUSAL, bh, qt);
    const int q0 = qt * kBlockM;
    const int64_t head = (int64_t)bh * N * D;
    const uint16_t* Qh = Q + head;
    const uint16_t* Kh = K + head;
    const uint16_t* Vh = V + head;
    const int wq0 = q0 + 32 * wave;  // first query row of this wave
    const int qrow = wq0 + lq;       // this lane's query row

    const int kv_end = CAUSAL ? min(N, q0 + kBlockM) : N;
    const int n_kv = (kv_end + kBlockN - 1) / kBlockN;

    // Wave w fills loads w*IPW .. w*IPW+IPW-1 of a tile; load g covers rows RPI*g .. RPI*g+RPI-1
    // and lane l writes LDS bytes [1024 g + 16 l, +16), i.e. row RPI*g + l/CPR at chunk position
    // l % CPR, which holds global chunk (l % CPR) ^ swz(row). Rows past the end of the sequence
    // repeat row N-1 (finite data; those keys are masked before they can carry weight).
    auto issue = [&](int j, uint16_t* kdst, uint16_t* vdst) {
        const int k0 = j * kBlockN;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int g = wave * IPW + i;
            const int r = RPI * g + lane / CPR;
            const int ch = (lane % CPR) ^ swz<D>(r);
            const int64_t src = (int64_t)min(k0 + r, N - 1) * D + 8 * ch;
            __builtin_amdgcn_global_load_lds((const void*)(Kh + src), (lds_void*)(kdst + g * 512), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(Vh + src), (lds_void*)(vdst + g * 512), 16, 0, 0);
        }
    };
    issue(0, k_lds0, v_lds0);

    // Q^T fragment (B operand of the first product): lane holds row qrow, columns
    // 16t + 8h .. 16t + 8h + 7 for every k-step t. Rows past N are zero.
    u32x4 qf[DK];
#pragma unroll
    for (int t = 0; t < DK; ++t) {
        qf[t] = (u32x4){0u, 0u, 0u, 0u};
        if (qrow < N) qf[t] = *reinterpret_cast<const u32x4*>(Qh + (int64_t)qrow * D + 16 * t + 8 * h);
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[b] = (f32x16){};
    float m_run = -INFINITY;  // reference max of raw dot products for l and oacc
    float l_run = 0.f;        // this lane's half of the running denominator (rounded p)
    float l_f32 = 0.f;        // the same sum of unrounded p: bf16 keeps 8 mantissa bits, too few
                              // for lse to 1e-3 on rows with few keys, so lse uses this one

    // ds_read_b64_tr_b16 source pattern: within each 16-lane group, lane s reads 4 consecutive
    // columns 4*(s%4).. of key row s/4; the instruction hands lane i element e of that 4x16
    // block as (key row e, column i), i.e. one V^T row of 4 keys per lane.
    const int s16 = lane & 15;
    const int tr_row = 4 * h + (s16 >> 2);                       // + key0 (+8 for the upper 4)
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);  // + 4*b
    const int tr_half = 4 * (s16 & 1);                          // element offset in the chunk

    auto compute = [&](int j, const uint16_t* kt, const uint16_t* vt) {
        const int k0 = j * kBlockN;
        if (CAUSAL && k0 > wq0 + 31) return;  // tile lies wholly above the diagonal for this wave

        // ---- S^T = K . Q^T (raw dot products) ----
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = (f32x16){};
#pragma unroll
            for (int t = 0; t < DK; ++t) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(kt + tile_off<D>(kb * 32 + lq, 2 * t + h));
                sacc[kb] = mfma32<BF16>(a, qf[t], sacc[kb]);
            }
        }

        // ---- mask: keys past the end, and (causal) keys after the query ----
        const bool need_mask = (k0 + kBlockN > N) || (CAUSAL && k0 + kBlockN - 1 > wq0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (key >= N || (CAUSAL && key > qrow)) sacc[kb][r] = -INFINITY;
                }
        }

        // ---- reference max: move it (and rescale l, o~ by alpha) only when some row of the
        //      wave has a score more than tau above it; otherwise p <= 2^tau_log2 ----
        float mx = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
        mx = max_with_partner(mx);
        if (__builtin_amdgcn_ballot_w64(mx > m_run + tau_raw)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
            l_run *= alpha;
            if constexpr (BF16) l_f32 *= alpha;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
            m_run = m_new;
        }
        const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;

        // ---- p = exp2(s*c - m*c), rounded to the operand type; row sum of the rounded values ----
        unsigned pk[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c, -mc));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + 1], c, -mc));
                pk[kb][r >> 1] = pack2<BF16>(p0, p1);
                l_run = add_pair<BF16>(pk[kb][r >> 1], l_run);
                if constexpr (BF16) l_f32 += p0 + p1;
            }

        // ---- O^T += V^T . P^T ----
#pragma unroll
        for (int kk = 0; kk < kBlockN / 16; ++kk) {
            const int kb = kk >> 1, hf = kk & 1;
            const u32x4 bop = {pk[kb][4 * hf + 0], pk[kb][4 * hf + 1], pk[kb][4 * hf + 2], pk[kb][4 * hf + 3]};
            const int key0 = kb * 32 + 16 * hf;
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const int r_lo = key0 + tr_row, r_hi = r_lo + 8;
                const uint16_t* p_lo = vt + tile_off<D>(r_lo, 4 * b + tr_chunk) + tr_half;
                const uint16_t* p_hi = vt + tile_off<D>(r_hi, 4 * b + tr_chunk) + tr_half;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p_lo));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p_hi));
                const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                const u32x4 aop = {lo2[0], lo2[1], hi2[0], hi2[1]};
                oacc[b] = mfma32<BF16>(aop, bop, oacc[b]);
            }
        }
    };

    // One barrier per tile: after it, tile j is in LDS for every wave and every wave has finished
    // tile j - 1, so the buffer tile j - 1 used can take tile j + 1.
    for (int j = 0; j < n_kv; j += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (j + 1 < n_kv) issue(j + 1, k_lds1, v_lds1);
        compute(j, k_lds0, v_lds0);
        if (j + 1 >= n_kv) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (j + 2 < n_kv) issue(j + 2, k_lds0, v_lds0);
        compute(j + 1, k_lds1, v_lds1);
    }

    // ---- epilogue: O = o~ / l, lse = m*scale + ln l ----
    const float l_tot = sum_with_partner(l_run);
    const float l_lse = BF16 ? sum_with_partner(l_f32) : l_tot;  // both halves active here
    if (qrow < N) {
        const float inv = 1.f / l_tot;
        uint16_t* orow = O + head + (int64_t)qrow * D;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2 st = {pack2<BF16>(oacc[b][4 * g + 0] * inv, oacc[b][4 * g + 1] * inv),
                                  pack2<BF16>(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + b * 32 + 8 * g + 4 * h) = st;
            }
        if (LSE != nullptr && h == 0) {
            const float mcf = (m_run == -INFINITY) ? 0.f : m_run * c;
            LSE[(int64_t)bh * N + qrow] = (mcf + __log2f(l_lse)) * 0.69314718055994531f;
        }
    }
}

template <int D, bool BF16, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int N, int n_qt, int G,
                  float c, float tau_raw, hipStream_t stream) {
    hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, CAUSAL>), dim3(G), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qt, G, c, tau_raw);
    return hipGetLastError();
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

int fa_version(void) { return 100; }

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "q, k, v or o is NULL";
        case FA_ERR_SHAPE: return "B, H and N must be >= 1 and within the size limits";
        case FA_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
        case FA_ERR_DTYPE: return "dtype must be FA_F16 or FA_BF16";
        case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
        case FA_ERR_SCALE: return "scale must be finite and > 0";
        case FA_ERR_ALIAS: return "o and lse must not overlap the inputs or each other";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
           int64_t d, float scale, int causal, hipStream_t stream, int dtype) {
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || N > (int64_t(1) << 30)) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    const int64_t n_qt = (N + kBlockM - 1) / kBlockM;
    if (B > INT32_MAX || H > INT32_MAX || B * H > INT32_MAX / n_qt) return FA_ERR_SHAPE;
    const int64_t G = B * H * n_qt;
    if (B * H * N > INT64_MAX / (d * 2)) return FA_ERR_SHAPE;
    auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        (lse && misaligned(lse, 4)))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
    const size_t nbytes = static_cast<size_t>(B * H * N * d * 2);
    const size_t lbytes = static_cast<size_t>(B * H * N * 4);
    if (overlaps(o, nbytes, q, nbytes) || overlaps(o, nbytes, k, nbytes) || overlaps(o, nbytes, v, nbytes))
        return FA_ERR_ALIAS;
    if (lse && (overlaps(lse, lbytes, q, nbytes) || overlaps(lse, lbytes, k, nbytes) ||
                overlaps(lse, lbytes, v, nbytes) || overlaps(lse, lbytes, o, nbytes)))
        return FA_ERR_ALIAS;

    const float c = scale * 1.4426950408889634f;  // scale * log2(e)
    // The reference max moves only when a score exceeds it by more than 8 in log2 units, so the
    // unnormalised p stay <= 2^8 (exact in f16/bf16 range) and most tiles skip the rescale.
    const float tau_raw = 8.f / c;
    const int n = static_cast<int>(N), nq = static_cast<int>(n_qt), g = static_cast<int>(G);
    const bool bf = dtype == FA_BF16;
    hipError_t e;
    if (d == 64) {
        if (bf) e = causal ? launch<64, true, true>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream)
                           : launch<64, true, false>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream);
        else e = causal ? launch<64, false, true>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream)
                        : launch<64, false, false>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream);
    } else {
        if (bf) e = causal ? launch<128, true, true>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream)
                           : launch<128, true, false>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream);
        else e = causal ? launch<128, false, true>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream)
                        : launch<128, false, false>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream);
    }
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
