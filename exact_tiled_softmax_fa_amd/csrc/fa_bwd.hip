// Backward pass of exact attention for gfx950 (CDNA4), behind the C ABI of fa_bwd.h.
//
// The forward pass keeps one statistic per query row, lse_i = m_i + ln l_i. The backward pass
// recomputes each score tile from Q, K and that statistic instead of reading a stored probability
// matrix ("Decoding flash attention" (bibekananda.in), section "The backward pass"; nalar.dev,
// section "Backward computation can trade recomputation for stored intermediates"). With
// p_ij = exp(s_ij - lse_i), the gradients of L = sum(dO * O) are the chain rule through softmax:
//   dP_ij = dO_i . v_j,   D_i = dO_i . o_i (= sum_j p_ij dP_ij),   dS_ij = p_ij (dP_ij - D_i)
//   dV_j = sum_i p_ij dO_i,   dK_j = scale * sum_i dS_ij q_i,   dQ_i = scale * sum_j dS_ij k_j
// Two kernels, no atomics, every output written once by one lane (deterministic):
//
// fa_bwd_dq_kernel   one workgroup = 8 waves x 32 query rows (the forward's query tiles and grid).
//                    First D_i = dO_i . o_i for its rows (written to delta), then a walk over the
//                    key tiles (64 keys, double-buffered in LDS as in the forward):
//                      S^T  = K . Q^T,  dP^T = V . dO^T   (Q^T, dO^T held in registers)
//                      dS^T = P^T (dP^T - D)              (two query rows per lane)
//                      dQ^T += K^T . dS^T                 (K^T by the LDS transpose read)
// fa_bwd_dkdv_kernel one workgroup = 128 keys in 4 groups of 32, each group taken by two waves
//                    that split every query tile of 64 rows in halves; the K and V rows sit in
//                    LDS for the whole kernel, the Q and dO tiles (with lse and D of their rows)
//                    are double-buffered; at the end the two partial sums of each key group are
//                    added through LDS:
//                      S  = Q . K^T,  dP = dO . V^T       (two keys per lane)
//                      dS = P (dP - D)
//                      dV^T += dO^T . P,  dK^T += Q^T . dS (dO^T, Q^T by the LDS transpose read)
// Plain causal workgroups of both kernels take two tiles in turn, a long and a short one, so all
// meet the same number of tiles and the ones running together read a head's tiles in step.
// All products are v_mfma_f32_16x16x32 on 16-row blocks (two per wave side), each operand read
// from LDS feeding both blocks; on random operands this shape spends less energy per flop than
// 32x32x16, and these kernels run at the power limit.
// P and dS are rounded to f16/bf16 as operands of the second products, with fp32 accumulation;
// masked entries (a key after the query, rows or keys past the end) get s = -inf, so p = 0 and
// dS = 0 before they touch any sum.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "fa_bwd.h"
#include "fa_device.h"

namespace {

using namespace fa_detail;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeyTile = 64;        // keys per tile in the dq kernel
constexpr int kKeys = 128;          // keys per workgroup in the dkdv kernel (4 groups of 32)
constexpr int kQueryTile = 64;      // query rows per tile in the dkdv kernel (two halves of 32)
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) const uint16_t lds_u16;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// Sum of the 8 products of two packed 8-element rows, in fp32. (Each element is copied to a
// scalar before the bit cast: __builtin_bit_cast applied to a vector element reads element 0.)
template <bool BF16>
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned x = a[i], y = b[i];
        if constexpr (BF16)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), acc,
                                                  false);
        else
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), acc, false);
    }
    return acc;
}

// ---- tiles and operands of the 16x16x32 products ----
// Every LDS tile is read in one or two patterns: as a row operand (ds_read_b128, lane (li, g)
// reads row r0 + li, chunk kchunk(t, g) of k-step t) and, for the K tile of the dQ kernel and the
// Q and dO tiles of the dK/dV kernel, transposed (ds_read_b64_tr_b16 over chunks 2b, 2b + 1 of
// 16 rows). The swizzle swz16 and the chunk order kchunk keep both free of bank conflicts (by
// measured LDS read rates: 187-197 and 130-135 B/clk per CU); row operands held in registers (Q,
// dO in the dQ kernel) take the same order, so every column is summed once.
template <int D>
__device__ __forceinline__ int swz16(int r) {
    if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
    else return r & 7;
}
template <int D>
__device__ __forceinline__ int kchunk(int t, int g) {
    return D == 128 ? t + 4 * g : 4 * t + g;
}
template <int D>
__device__ __forceinline__ int off16(int r, int c) {
    return r * D + ((c ^ swz16<D>(r)) << 3);
}
// Stage `rows` rows starting at r0 of one head into a swizzled LDS tile by LDS DMA (lds_load16)
// (rows past the end repeat row N-1); each of the kWaves waves issues its share of 1 KiB loads.
template <int D, int W = kWaves>
__device__ __forceinline__ void stage_rows(const uint16_t* src_head, int r0, int rows, int N, uint16_t* dst,
                                           int wave_s, int lane) {
    constexpr int CPR = D / 8;
    constexpr int RPI = 64 / CPR;
    const int per_wave = rows / RPI / W;
    for (int i = 0; i < per_wave; ++i) {
        const int ld = wave_s * per_wave + i;
        const int r = RPI * ld + lane / CPR;
        const int ch = (lane % CPR) ^ swz16<D>(r);
        const unsigned src = (unsigned)min(r0 + r, N - 1) * D + 8 * ch;
        lds_load16(src_head, N * D * 2, 2 * src, (lds_void*)(dst + ld * 512));
    }
}
// Transposed A operand of a 16x16x32 product: rows d = 16b + li, k slots 8g + s = tile rows
// 32kk + 4g + s (s < 4) and 32kk + 16 + 4g + s - 4 (s >= 4), the order in which a lane holds
// a 16x16 C tile's rows 4g .. 4g + 3 of two consecutive tiles. off: per-lane offsets of
// transpose16_offsets.
template <int D>
__device__ __forceinline__ void transpose16_offsets(int lane, int (&off)[D / 16]) {
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int b = 0; b < D / 16; ++b) off[b] = off16<D>(4 * g + (li >> 2), 2 * b + ((li & 3) >> 1)) + 4 * (li & 1);
}
template <int D>
__device__ __forceinline__ u32x4 transposed16(const uint16_t* tile, const int (&off)[D / 16], int kk, int b) {
    const i16x4 l4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off[b] + kk * 32 * D));
    const i16x4 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off[b] + kk * 32 * D + 16 * D));
    const u32x2 a = __builtin_bit_cast(u32x2, l4);
    const u32x2 c = __builtin_bit_cast(u32x2, h4);
    return (u32x4){a[0], a[1], c[0], c[1]};
}
// Store a row of a transposed 16x16 accumulator set (lane: row; registers of block b: columns
// 16b + 4g .. +3) times f.
template <int D, bool BF16>
__device__ __forceinline__ void store_row16(uint16_t* row, const f32x4 (&acc)[D / 16], float f, int g) {
#pragma unroll
    for (int b = 0; b < D / 16; ++b) {
        const u32x2 st = {pack2<BF16>(acc[b][0] * f, acc[b][1] * f), pack2<BF16>(acc[b][2] * f, acc[b][3] * f)};
        *reinterpret_cast<u32x2*>(row + 16 * b + 4 * g) = st;
    }
}

// MASKED (both kernels): the general mask of fa_fwd_masked in place of CAUSAL -- key j allowed for
// query i when i - wl <= j (wl >= 0), j <= i + wr (wr >= 0) and j < seqlens[b] (seqlens given).
// Only the tiles a workgroup's window reaches are loaded; a row with no allowed key (lse = -inf)
// takes the statistic 0, so its masked scores give p = 0 rather than NaN.
// BLOCKS (both kernels, on top of MASKED): the block mask of fa_fwd_blocksparse. Each workgroup
// lists the tiles one of its waves needs (compact_tiles) and walks only those; a wave computes a
// listed tile only when its own bit is set.
template <int D, bool BF16, bool CAUSAL, bool MASKED = false, bool BLOCKS = false, bool CHUNKED = false,
          int WV = kWaves>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ DELTA, uint16_t* __restrict__ dQ, int N, int n_qt, int G, float c, float scale, int H = 1,
    int wl = -1, int wr = -1, const int* __restrict__ seqlens = nullptr, const uint8_t* __restrict__ bmask = nullptr,
    int bq = 0, int bk = 0, int64_t bstride_b = 0, int64_t bstride_h = 0) {
    static_assert(!(MASKED && CAUSAL), "the general mask replaces the causal one");
    static_assert(!BLOCKS || MASKED, "the block mask rides on the general mask");
    constexpr int DT = D / 32;  // 32-column k-steps of the first two products
    constexpr int DB = D / 16;  // 16-column blocks of dQ
    constexpr int TILE = kKeyTile * D;
    static_assert(kKeyTile * D / (64 * 8) % WV == 0, "tile loads must split evenly over the waves");
    static_assert(WV == kWaves || (WV == 4 && MASKED), "4-wave workgroups: the masked and block-sparse kernels");

    __shared__ __attribute__((aligned(4096))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(4096))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(4096))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(4096))) uint16_t v_lds1[TILE];

    // PAIRED (plain causal): workgroup p of a head takes query tile n_qt - 1 - p and then tile p,
    // as the causal forward does: equal work per workgroup, and the workgroups that run together
    // read one head's K/V in step.
    constexpr bool PAIRED = CAUSAL && !MASKED;
    int bh, qt_first;
    map_block(blockIdx.x, G, PAIRED ? (n_qt + 1) / 2 : n_qt, CAUSAL && !PAIRED, bh, qt_first);
    const int n_pass = PAIRED && n_qt - 1 - qt_first != qt_first ? 2 : 1;
#pragma nounroll
    for (int pass = 0; pass < n_pass; ++pass) {
        if (pass) __syncthreads();  // every wave is done with the first tile's LDS buffers
        // (the thread index is hidden from the compiler in each pass, so it does not keep every
        // per-lane address of the tile loop live across both passes)
        int tid = threadIdx.x;
        if constexpr (PAIRED) asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = tid >> 6;
        // 16x16x32 products: lane l holds query column li = l % 16 of the S^T, dP^T and dQ^T tiles of
        // both 16-row blocks of the wave, and row group g = l / 16 (tile rows 4g .. 4g + 3; operand k
        // slots 8g .. 8g + 7)
        const int g = lane >> 4;
        const int li = lane & 15;
        const int wave_s = __builtin_amdgcn_readfirstlane(wave);
        const int qt = PAIRED ? (pass == 0 ? n_qt - 1 - qt_first : qt_first) : qt_first;
        const int q0 = qt * (32 * WV);
        const int64_t head = (int64_t)bh * N * D;
        const uint16_t* Kh = K + head;
        const uint16_t* Vh = V + head;
        const int wq0 = q0 + 32 * wave;

        // The lane's two query rows (wq0 + li and wq0 + 16 + li, blocks qb = 0, 1) as B operands of
        // the first two products (chunk kchunk(t, g) of k-step t). The same chunks of o give the
        // lane's quarter of D = dO . o. Rows past N repeat row N-1 (never stored).
        u32x4 qf[2][DT], df[2][DT];
        float Dq[2], lse2[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qrow = wq0 + 16 * qb + li;
            const int64_t qr = min(qrow, N - 1);
            const uint16_t* qrp = Q + head + qr * D;
            const uint16_t* drp = dO + head + qr * D;
            const uint16_t* orp = O + head + qr * D;
            float dsum = 0.f;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const int col = 8 * kchunk<D>(t, g);
                qf[qb][t] = *reinterpret_cast<const u32x4*>(qrp + col);
                df[qb][t] = *reinterpret_cast<const u32x4*>(drp + col);
                dsum = dot8<BF16>(df[qb][t], *reinterpret_cast<const u32x4*>(orp + col), dsum);
            }
            Dq[qb] = sum_over_rows(dsum);
            if (g == 0 && qrow < N) DELTA[(int64_t)bh * N + qrow] = Dq[qb];
            const float lse_raw = LSE[(int64_t)bh * N + qr];
            lse2[qb] = (MASKED && lse_raw == -INFINITY) ? 0.f : lse_raw * kLog2e;  // lse in log2 units
        }

        const int kv_end = CAUSAL ? min(N, q0 + 32 * WV) : N;
        // key tiles tb .. tb + T - 1 (tile indices below are relative to tb); this wave computes
        // T_w0 .. T_w - 1 of them
        int tb = 0, kv_len = N;
        int T = (kv_end + kKeyTile - 1) / kKeyTile;
        int T_w = CAUSAL ? min(T, (min(wq0 + 32, N) + kKeyTile - 1) / kKeyTile) : T;
        int T_w0 = 0;
        if constexpr (MASKED) {
            if (seqlens != nullptr) kv_len = min(max(seqlens[bh / H], 0), N);
            const int lo = wl >= 0 ? max(0, q0 - wl) : 0;
            const int hi = wr >= 0 ? min(kv_len, q0 + 32 * WV + wr) : kv_len;
            tb = lo / kKeyTile;
            T = max(0, (hi + kKeyTile - 1) / kKeyTile - tb);
            const int hi_w = wr >= 0 ? min(kv_len, wq0 + 32 + wr) : kv_len;  // this wave's last key + 1
            T_w = max(0, min(T, (hi_w + kKeyTile - 1) / kKeyTile - tb));
            if (wl >= 0) T_w0 = min(T_w, max(0, wq0 - wl) / kKeyTile - tb);
        }
        // BLOCKS: tile index j becomes a position in t_list; every wave walks the whole list.
        // CHUNKED: the list is built and walked kMaxListTiles candidates at a time (below).
        __shared__ int t_list[BLOCKS ? kMaxListTiles : 1];
        __shared__ uint8_t t_wm[BLOCKS ? kMaxListTiles : 1];
        __shared__ int t_cnt[BLOCKS ? WV : 1];
        const uint8_t* mb = BLOCKS ? bmask + (int64_t)(bh / H) * bstride_b + (int64_t)(bh % H) * bstride_h : nullptr;
        const int n_kb = BLOCKS ? (N + bk - 1) / bk : 0;
        // wave w needs key tile t when its rows and the tile's keys hold an allowed pair: the block
        // byte is set and the offsets key - row, which run over one interval, meet the window
        auto need = [&](int w, int t) {
            const int r0 = q0 + 32 * w, r1 = min(r0 + 32, N) - 1;
            const int c0 = t * kKeyTile, c1 = min(c0 + kKeyTile, kv_len) - 1;
            return r0 < N && c0 < kv_len && (wr < 0 || c0 - r1 <= wr) && (wl < 0 || r0 - c1 <= wl) &&
                   mb[(int64_t)(r0 / bq) * n_kb + c0 / bk] != 0;
        };
        const int T_cand = T;
        if constexpr (BLOCKS && !CHUNKED) T = compact_tiles<WV>(tb, T, need, t_list, t_wm, t_cnt, tid);
        if constexpr (BLOCKS) {
            T_w0 = 0;
            T_w = T;
        }
        auto key_tile = [&](int j) { return BLOCKS ? __builtin_amdgcn_readfirstlane(t_list[j]) : tb + j; };

        // row operands of K and V (keys 16kb + li, chunk kchunk(t, g)) and the K^T operand
        int aoff[DT];
#pragma unroll
        for (int t = 0; t < DT; ++t) aoff[t] = off16<D>(li, kchunk<D>(t, g));
        int troff[DB];
        transpose16_offsets<D>(lane, troff);

        // dQ^T of this wave: block (qb, b) holds columns 16b + 4g .. +3 of query row wq0 + 16qb + li
        f32x4 acc[2][DB];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int b = 0; b < DB; ++b) acc[qb][b] = (f32x4){};

        auto tile = [&](int j, const uint16_t* kt, const uint16_t* vt) __attribute__((always_inline)) {
            const int k0 = key_tile(j) * kKeyTile;
            const bool masked = MASKED ? (k0 + kKeyTile > kv_len) || (wr >= 0 && k0 + kKeyTile - 1 > wq0 + wr) ||
                                             (wl >= 0 && k0 < wq0 + 31 - wl)
                                       : (k0 + kKeyTile > N) || (CAUSAL && k0 + kKeyTile - 1 > wq0);
            // keep the constant parts of the LDS addresses in the instructions (see the dkdv kernel)
#pragma unroll
            for (int t = 0; t < DT; ++t) asm volatile("" : "+v"(aoff[t]));
#pragma unroll
            for (int b = 0; b < DB; ++b) asm volatile("" : "+v"(troff[b]));
            // dS^T of the tile as B operands of the last product: [qb][kk][.] covers keys 32kk ..
            // 32kk + 31 in the k-slot order of transposed16 (pairs of 16-key blocks 2kk, 2kk + 1)
            unsigned dsk[2][2][4];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                __builtin_amdgcn_sched_barrier(0);  // 32 keys at a time
                f32x4 s[2][2], dp[2][2];            // [qb][16-key block 2kk + u]
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int kb = 2 * kk + u;
                        const u32x4 ka = *reinterpret_cast<const u32x4*>(kt + aoff[t] + kb * 16 * D);
                        const u32x4 va = *reinterpret_cast<const u32x4*>(vt + aoff[t] + kb * 16 * D);
#pragma unroll
                        for (int qb = 0; qb < 2; ++qb) {
                            s[qb][u] = mfma16<BF16>(ka, qf[qb][t], t == 0 ? (f32x4){} : s[qb][u]);
                            dp[qb][u] = mfma16<BF16>(va, df[qb][t], t == 0 ? (f32x4){} : dp[qb][u]);
                        }
                    }
                // C layout: register r of (qb, u) holds key k0 + 32kk + 16u + 4g + r of query row
                // wq0 + 16qb + li
                if (masked) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                        for (int u = 0; u < 2; ++u)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int key = k0 + 32 * kk + 16 * u + 4 * g + r, qrow = wq0 + 16 * qb + li;
                                const bool out = MASKED ? key >= kv_len || (wr >= 0 && key > qrow + wr) ||
                                                              (wl >= 0 && key < qrow - wl)
                                                        : key >= N || (CAUSAL && key > qrow);
                                if (out) s[qb][u][r] = -INFINITY;
                            }
                }
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int r = 0; r < 4; r += 2) {
                            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][u][r], c, -lse2[qb]));
                            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][u][r + 1], c, -lse2[qb]));
                            dsk[qb][kk][2 * u + (r >> 1)] =
                                pack2<BF16>(p0 * (dp[qb][u][r] - Dq[qb]), p1 * (dp[qb][u][r + 1] - Dq[qb]));
                        }
            }
            __builtin_amdgcn_sched_barrier(0);
            // dQ^T += K^T . dS^T over the 64 keys (2 steps of 32); each K^T operand feeds both blocks
#pragma unroll
            for (int i = 0; i < 2 * DB; ++i) {
                const int kk = i / DB, b = i % DB;
                const u32x4 a = transposed16<D>(kt, troff, kk, b);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const u32x4 ds = {dsk[qb][kk][0], dsk[qb][kk][1], dsk[qb][kk][2], dsk[qb][kk][3]};
                    acc[qb][b] = mfma16<BF16>(a, ds, acc[qb][b]);
                }
            }
        };

        // K(j), V(j) sit in buffer j % 2; the loads of tile j + 1 go out right after the barrier that
        // makes tile j visible (and frees the buffers of tile j - 1).
        // T_w as an opaque scalar: with the test j < T_w folded away (non-causal) the compiler keeps
        // the accumulators of the two unrolled tiles in two register sets and spills.
        int T_ws = __builtin_amdgcn_readfirstlane(T_w);
        asm volatile("" : "+s"(T_ws));
        const int T_w0s = __builtin_amdgcn_readfirstlane(T_w0);
        // BLOCKS: this wave's bit for list entry j
        auto mine = [&](int j) { return !BLOCKS || ((__builtin_amdgcn_readfirstlane(t_wm[j]) >> wave_s) & 1); };
        auto walk = [&]() __attribute__((always_inline)) {
            stage_rows<D, WV>(Kh, key_tile(0) * kKeyTile, kKeyTile, N, k_lds0, wave_s, lane);
            stage_rows<D, WV>(Vh, key_tile(0) * kKeyTile, kKeyTile, N, v_lds0, wave_s, lane);
            for (int j = 0; j < T; j += 2) {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (j + 1 < T) {
                    stage_rows<D, WV>(Kh, key_tile(j + 1) * kKeyTile, kKeyTile, N, k_lds1, wave_s, lane);
                    stage_rows<D, WV>(Vh, key_tile(j + 1) * kKeyTile, kKeyTile, N, v_lds1, wave_s, lane);
                }
                if ((!MASKED || j >= T_w0s) && j < T_ws && mine(j)) tile(j, k_lds0, v_lds0);
                if (j + 1 >= T) break;
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (j + 2 < T) {
                    stage_rows<D, WV>(Kh, key_tile(j + 2) * kKeyTile, kKeyTile, N, k_lds0, wave_s, lane);
                    stage_rows<D, WV>(Vh, key_tile(j + 2) * kKeyTile, kKeyTile, N, v_lds0, wave_s, lane);
                }
                if ((!MASKED || j + 1 >= T_w0s) && j + 1 < T_ws && mine(j + 1)) tile(j + 1, k_lds1, v_lds1);
            }
        };
        if constexpr (CHUNKED) {
            // acc carries over from chunk to chunk. Every wave has left the previous chunk's tiles
            // (t_list, t_wm and both buffers read for the last time; no load in flight) before the
            // first barrier of compact_tiles, which writes the list only after it.
            for (int cb = 0; cb < T_cand; cb += kMaxListTiles) {
                T = compact_tiles<WV>(tb + cb, min(kMaxListTiles, T_cand - cb), need, t_list, t_wm, t_cnt, tid);
                T_ws = T;
                if (T > 0) walk();
            }
        } else {
            walk();
        }

#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qrow = wq0 + 16 * qb + li;
            if (qrow < N) store_row16<D, BF16>(dQ + head + (int64_t)qrow * D, acc[qb], scale, g);
        }
    }  // pass
}

template <int D, bool BF16, bool CAUSAL, bool MASKED = false, bool BLOCKS = false, bool CHUNKED = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ DELTA,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int n_kt, int G, float c, float scale, int H = 1,
    int wl = -1, int wr = -1, const int* __restrict__ seqlens = nullptr, const uint8_t* __restrict__ bmask = nullptr,
    int bq = 0, int bk = 0, int64_t bstride_b = 0, int64_t bstride_h = 0) {
    static_assert(!(MASKED && CAUSAL), "the general mask replaces the causal one");
    static_assert(!BLOCKS || MASKED, "the block mask rides on the general mask");
    constexpr int DT = D / 32;  // 32-column k-steps of the first two products
    constexpr int DB = D / 16;  // 16-column blocks of dK and dV
    constexpr int TILE = kQueryTile * D;
    static_assert(kQueryTile * D / (64 * 8) % kWaves == 0, "tile loads must split evenly over the waves");

    // The Q and dO tiles (most reads, several buffers) get the larger alignment so they are placed
    // in the first 64 KiB, where a constant offset fits the LDS instructions' offset field. K and
    // V rows follow in one array (V = K + kKeys * D), addressed from one register per k-step.
    __shared__ __attribute__((aligned(8192))) uint16_t q_lds0[TILE];
    __shared__ __attribute__((aligned(8192))) uint16_t q_lds1[TILE];
    __shared__ __attribute__((aligned(8192))) uint16_t do_lds0[TILE];
    __shared__ __attribute__((aligned(8192))) uint16_t do_lds1[TILE];
    __shared__ __attribute__((aligned(4096))) uint16_t kv_lds[2 * kKeys * D];  // K rows, then V rows
    __shared__ __attribute__((aligned(16))) float st_lds[2][2][kQueryTile];    // [buffer][lse2, D][row]

    // Causal: key tile 0 meets every query row. PAIRED (plain causal): workgroup p of a head takes
    // key tile p and then key tile n_kt - 1 - p, so every workgroup meets the same number of query
    // tiles.
    constexpr bool PAIRED = CAUSAL && !MASKED;
    int bh, kt_first;
    map_block(blockIdx.x, G, PAIRED ? (n_kt + 1) / 2 : n_kt, CAUSAL && !PAIRED, bh, kt_first);
    const int n_pass = PAIRED && n_kt - 1 - kt_first != kt_first ? 2 : 1;
#pragma nounroll
    for (int pass = 0; pass < n_pass; ++pass) {
        if (pass) __syncthreads();  // every wave is done with the first key tile's LDS (the sums too)
        int tid = threadIdx.x;
        if constexpr (PAIRED) asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = tid >> 6;
        // 16x16x32 products: lane l holds key column li = l % 16 of the S, dP, dK^T and dV^T tiles
        // of both 16-key blocks of the wave, and row group g = l / 16 (tile rows 4g .. 4g + 3; operand
        // k slots 8g .. 8g + 7)
        const int g = lane >> 4;
        const int li = lane & 15;
        const int wave_s = __builtin_amdgcn_readfirstlane(wave);
        const int kg = wave & 3;     // key group: keys 32 kg .. 32 kg + 31 of the workgroup
        const int half = wave >> 2;  // the 32-row half of every query tile this wave takes

        const int kt = PAIRED ? (pass == 0 ? kt_first : n_kt - 1 - kt_first) : kt_first;
        const int k0 = kt * kKeys;
        const int64_t head = (int64_t)bh * N * D;
        const uint16_t* Qh = Q + head;
        const uint16_t* dOh = dO + head;
        const float* lse_h = LSE + (int64_t)bh * N;
        const float* del_h = DELTA + (int64_t)bh * N;
        const int kw0 = k0 + 32 * kg;

        stage_rows<D>(K + head, k0, kKeys, N, kv_lds, wave_s, lane);
        stage_rows<D>(V + head, k0, kKeys, N, kv_lds + kKeys * D, wave_s, lane);

        // Per-lane element offsets with this wave's row block folded in (the swizzle depends on
        // row % 16 only, so moving whole 16-row blocks is a plain offset): qoff into a Q or dO tile
        // (rows 32 half + li, chunk kchunk(t, g) of k-step t), troff for the transpose reads of the
        // same 32 rows, and kvo into kv_lds for the K row 32 kg + li (its V row is kKeys * D
        // elements further).
        int qoff[DT], troff[DB], kvo[DT];
        transpose16_offsets<D>(lane, troff);
#pragma unroll
        for (int b = 0; b < DB; ++b) troff[b] += 32 * half * D;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            qoff[t] = off16<D>(li, kchunk<D>(t, g)) + 32 * half * D;
            kvo[t] = off16<D>(li, kchunk<D>(t, g)) + 32 * kg * D;
        }

        // dK^T and dV^T of this wave: block (b, kb) holds columns 16b + 4g .. +3 of key kw0 + 16kb + li
        f32x4 dv[DB][2], dk[DB][2];
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) dv[b][kb] = dk[b][kb] = (f32x4){};

        // query tiles j0 .. n_steps - 1 can see keys of this workgroup; rows [lo_w, hi_w) can see keys
        // of this wave (MASKED: keys past the batch's length are seen by no row)
        int n_steps = (N + kQueryTile - 1) / kQueryTile;
        int j0 = CAUSAL ? k0 / kQueryTile : 0;
        int kv_len = N, lo_w = CAUSAL ? kw0 : -1, hi_w = N;
        if constexpr (MASKED) {
            if (seqlens != nullptr) kv_len = min(max(seqlens[bh / H], 0), N);
            const int i_lo = wr >= 0 ? max(0, k0 - wr) : 0;
            const int k_end = min(k0 + kKeys, kv_len);  // this workgroup's last valid key + 1
            const int i_hi = k_end <= k0 ? i_lo : (wl >= 0 ? min(N, k_end + wl) : N);
            j0 = i_lo / kQueryTile;
            n_steps = max(j0, (i_hi + kQueryTile - 1) / kQueryTile);
            lo_w = wr >= 0 ? kw0 - wr : -1;
            const int kw_end = min(kw0 + 32, kv_len);
            hi_w = kw_end <= kw0 ? -1 : (wl >= 0 ? min(N, kw_end + wl) : N);
        }

        // The query tiles walked: j0 + p for p < n_list, or (BLOCKS) the listed tiles t_list[p] that one
        // of the waves needs, a wave computing the ones whose bit it holds.
        // (CHUNKED: the list is built and walked kMaxListTiles candidates at a time, below.)
        int n_list = n_steps - j0;
        __shared__ int t_list[BLOCKS ? kMaxListTiles : 1];
        __shared__ uint8_t t_wm[BLOCKS ? kMaxListTiles : 1];
        __shared__ int t_cnt[BLOCKS ? kWaves : 1];
        const uint8_t* mb = BLOCKS ? bmask + (int64_t)(bh / H) * bstride_b + (int64_t)(bh % H) * bstride_h : nullptr;
        const int n_kb = BLOCKS ? (N + bk - 1) / bk : 0;
        // wave w: row half w >> 2 of query tile t against key group w & 3 (the window test is the dQ
        // kernel's)
        auto need = [&](int w, int t) {
            const int r0 = t * kQueryTile + 32 * (w >> 2), r1 = min(r0 + 32, N) - 1;
            const int c0 = k0 + 32 * (w & 3), c1 = min(c0 + 32, kv_len) - 1;
            return r0 < N && c0 < kv_len && (wr < 0 || c0 - r1 <= wr) && (wl < 0 || r0 - c1 <= wl) &&
                   mb[(int64_t)(r0 / bq) * n_kb + c0 / bk] != 0;
        };
        const int n_cand = n_list;
        if constexpr (BLOCKS && !CHUNKED) n_list = compact_tiles<kWaves>(j0, n_list, need, t_list, t_wm, t_cnt, tid);
        auto q_tile = [&](int p) { return BLOCKS ? __builtin_amdgcn_readfirstlane(t_list[p]) : j0 + p; };
        auto mine = [&](int p) { return !BLOCKS || ((__builtin_amdgcn_readfirstlane(t_wm[p]) >> wave_s) & 1); };

        // lse (log2 units) and D of the rows of query tile j, staged by wave 0 through registers
        float st_l = 0.f, st_d = 0.f;
        // (The loaded values are first used at the store, at the end of the step: no wait for the
        // loads before the step's products.)
        auto stats_load = [&](int j) __attribute__((always_inline)) {
            const int r = min(j * kQueryTile + lane, N - 1);
            st_l = lse_h[r];
            st_d = del_h[r];
        };
        auto stats_store = [&](int buf) __attribute__((always_inline)) {
            st_lds[buf][0][lane] = (MASKED && st_l == -INFINITY) ? 0.f : st_l * kLog2e;
            st_lds[buf][1][lane] = st_d;
        };

        // Query rows below skip_below meet none of this wave's keys (causal, or a window that reaches
        // no further ahead; MASKED also skips rows from skip_from on). The bound is a scalar
        // the compiler cannot see through: with the test folded away (non-causal) it keeps the
        // accumulators of the two unrolled steps in two register sets and spills.
        int skip_below = __builtin_amdgcn_readfirstlane(lo_w);
        asm volatile("" : "+s"(skip_below));
        const int skip_from = __builtin_amdgcn_readfirstlane(hi_w);  // (MASKED) rows from here see no key
        // One 32-row half of query tile j against this wave's 32 keys: 64 MFMAs at D = 128.
        auto step = [&](int j, const uint16_t* qt_, const uint16_t* dot_, int buf) __attribute__((always_inline)) {
            const int qs = j * kQueryTile + 32 * half;  // first query row of this wave's half
            if (qs + 31 < skip_below) return;           // every key of this wave is after these rows
            if (MASKED && qs >= skip_from) return;       // or before them, beyond the window
            // Redefining the per-lane offsets each step keeps the compiler from hoisting every
            // (offset + constant) LDS address of the unrolled loop into a register of its own. They
            // stay offsets into known arrays: a pointer passed through the asm would be an unknown
            // object to the compiler, which then waits for the tile loads in flight (vmcnt(0))
            // before reading through it.
#pragma unroll
            for (int t = 0; t < DT; ++t) asm volatile("" : "+v"(qoff[t]), "+v"(kvo[t]));
#pragma unroll
            for (int b = 0; b < DB; ++b) asm volatile("" : "+v"(troff[b]));
            // S = Q . K^T, then dP = dO . V^T: at each k-step the two row operands of each side (query
            // blocks qb, key blocks kb) feed four MFMAs. The operands of stage i + 1 are read before
            // the MFMAs of stage i issue (sched_barrier pins the order).
            f32x4 s[2][2], dp[2][2];  // [qb][kb]
            u32x4 oa[2][2], ob[2][2];  // [ring][qb] row operands of Q or dO, [ring][kb] of K or V
            auto fetch = [&](int i) __attribute__((always_inline)) {
                const int r = i & 1, t = i % DT;
                const uint16_t* at = i < DT ? qt_ : dot_;
                const uint16_t* bt = i < DT ? kv_lds : kv_lds + kKeys * D;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    oa[r][u] = *reinterpret_cast<const u32x4*>(at + qoff[t] + u * 16 * D);
                    ob[r][u] = *reinterpret_cast<const u32x4*>(bt + kvo[t] + u * 16 * D);
                }
            };
            fetch(0);
#pragma unroll
            for (int i = 0; i < 2 * DT; ++i) {
                if (i + 1 < 2 * DT) fetch(i + 1);
                __builtin_amdgcn_sched_barrier(0);
                const int r = i & 1;
                const bool first = i % DT == 0;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        if (i < DT) s[qb][kb] = mfma16<BF16>(oa[r][qb], ob[r][kb], first ? (f32x4){} : s[qb][kb]);
                        else dp[qb][kb] = mfma16<BF16>(oa[r][qb], ob[r][kb], first ? (f32x4){} : dp[qb][kb]);
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
            // C layout: register r of (qb, kb) holds query row qs + 16qb + 4g + r of key kw0 + 16kb + li
            if (MASKED ? qs + 32 > N || kw0 + 31 >= kv_len || (wr >= 0 && kw0 + 31 > qs + wr) ||
                             (wl >= 0 && kw0 < qs + 31 - wl)
                       : qs + 32 > N || (CAUSAL && qs < kw0 + 31)) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int qrow = qs + 16 * qb + 4 * g + r, key = kw0 + 16 * kb + li;
                            const bool out = MASKED ? key >= kv_len || (wr >= 0 && key > qrow + wr) ||
                                                          (wl >= 0 && key < qrow - wl)
                                                    : CAUSAL && key > qrow;
                            if (qrow >= N || out) s[qb][kb][r] = -INFINITY;
                        }
            }
            // P and dS as B operands of the last two products: [kb][.] holds the k slots 8g .. 8g + 7,
            // rows 4g .. 4g + 3 of query block 0 and of block 1 (the order of transposed16)
            unsigned pk[2][4], dsk[2][4];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int o = 32 * half + 16 * qb + 4 * g;
                const float4 l4 = *reinterpret_cast<const float4*>(&st_lds[buf][0][o]);
                const float4 d4 = *reinterpret_cast<const float4*>(&st_lds[buf][1][o]);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][0], c, -l4.x));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][1], c, -l4.y));
                    const float p2 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][2], c, -l4.z));
                    const float p3 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][3], c, -l4.w));
                    pk[kb][2 * qb] = pack2<BF16>(p0, p1);
                    pk[kb][2 * qb + 1] = pack2<BF16>(p2, p3);
                    dsk[kb][2 * qb] = pack2<BF16>(p0 * (dp[qb][kb][0] - d4.x), p1 * (dp[qb][kb][1] - d4.y));
                    dsk[kb][2 * qb + 1] = pack2<BF16>(p2 * (dp[qb][kb][2] - d4.z), p3 * (dp[qb][kb][3] - d4.w));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // dV^T += dO^T . P and dK^T += Q^T . dS over these 32 rows; each transposed operand feeds
            // both key blocks, and the operands of column block b + 1 are read before block b issues
            u32x4 ta[2], tq[2];
            ta[0] = transposed16<D>(dot_, troff, 0, 0);
            tq[0] = transposed16<D>(qt_, troff, 0, 0);
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                if (b + 1 < DB) {
                    ta[(b + 1) & 1] = transposed16<D>(dot_, troff, 0, b + 1);
                    tq[(b + 1) & 1] = transposed16<D>(qt_, troff, 0, b + 1);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u32x4 pop = {pk[kb][0], pk[kb][1], pk[kb][2], pk[kb][3]};
                    const u32x4 dop = {dsk[kb][0], dsk[kb][1], dsk[kb][2], dsk[kb][3]};
                    dv[b][kb] = mfma16<BF16>(ta[b & 1], pop, dv[b][kb]);
                    dk[b][kb] = mfma16<BF16>(tq[b & 1], dop, dk[b][kb]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // Q, dO and the statistics of walk position p sit in buffer p % 2. The tensor tiles of p + 1
        // are requested right after the barrier that publishes p; wave 0 fetches the statistics of
        // p + 1 into registers at the same time and writes them to LDS at the end of the step (the
        // buffer they go to was last read in step p - 1, before that barrier).
        auto walk = [&]() __attribute__((always_inline)) {
            if (wave == 0) stats_load(q_tile(0));
            stage_rows<D>(Qh, q_tile(0) * kQueryTile, kQueryTile, N, q_lds0, wave_s, lane);
            stage_rows<D>(dOh, q_tile(0) * kQueryTile, kQueryTile, N, do_lds0, wave_s, lane);
            if (wave == 0) stats_store(0);
            for (int p = 0; p < n_list; p += 2) {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (p + 1 < n_list) {
                    if (wave == 0) stats_load(q_tile(p + 1));
                    stage_rows<D>(Qh, q_tile(p + 1) * kQueryTile, kQueryTile, N, q_lds1, wave_s, lane);
                    stage_rows<D>(dOh, q_tile(p + 1) * kQueryTile, kQueryTile, N, do_lds1, wave_s, lane);
                }
                if (mine(p)) step(q_tile(p), q_lds0, do_lds0, 0);
                if (p + 1 >= n_list) break;
                if (wave == 0) stats_store(1);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (p + 2 < n_list) {
                    if (wave == 0) stats_load(q_tile(p + 2));
                    stage_rows<D>(Qh, q_tile(p + 2) * kQueryTile, kQueryTile, N, q_lds0, wave_s, lane);
                    stage_rows<D>(dOh, q_tile(p + 2) * kQueryTile, kQueryTile, N, do_lds0, wave_s, lane);
                }
                if (mine(p + 1)) step(q_tile(p + 1), q_lds1, do_lds1, 1);
                if (p + 2 < n_list && wave == 0) stats_store(0);
            }
        };
        if constexpr (CHUNKED) {
            // dK and dV carry over from chunk to chunk. Every wave has left the previous chunk's
            // steps (t_list, t_wm, the tile buffers and the statistics read for the last time; no load
            // in flight) before the first barrier of compact_tiles, which writes the list only after it.
            for (int cb = 0; cb < n_cand; cb += kMaxListTiles) {
                n_list = compact_tiles<kWaves>(j0 + cb, min(kMaxListTiles, n_cand - cb), need, t_list, t_wm, t_cnt, tid);
                if (n_list > 0) walk();
            }
        } else {
            walk();
        }

        // The two waves of a key group summed over different query rows: the second half hands its
        // partial sums over through LDS (the tiles are no longer needed) and the first half stores.
        // Layout [register][lane]: consecutive lanes hit consecutive banks.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        float* dv_x = reinterpret_cast<float*>(kv_lds + kg * (kKeys / 2) * D);
        float* dk_x = reinterpret_cast<float*>(kg == 0 ? q_lds0 : kg == 1 ? q_lds1 : kg == 2 ? do_lds0 : do_lds1);
        if (half == 1) {
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        dv_x[((b * 2 + kb) * 4 + r) * 64 + lane] = dv[b][kb][r];
                        dk_x[((b * 2 + kb) * 4 + r) * 64 + lane] = dk[b][kb][r];
                    }
        }
        __syncthreads();
        if (half == 0) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int key = kw0 + 16 * kb + li;
                if (key >= N) continue;
                f32x4 v4[DB], k4[DB];
#pragma unroll
                for (int b = 0; b < DB; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        v4[b][r] = dv[b][kb][r] + dv_x[((b * 2 + kb) * 4 + r) * 64 + lane];
                        k4[b][r] = dk[b][kb][r] + dk_x[((b * 2 + kb) * 4 + r) * 64 + lane];
                    }
                store_row16<D, BF16>(dV + head + (int64_t)key * D, v4, 1.f, g);
                store_row16<D, BF16>(dK + head + (int64_t)key * D, k4, scale, g);
            }
        }
    }  // pass
}

// WQ: waves per dQ workgroup (query rows 32 * WQ); 4 only under the general mask.
template <int D, bool BF16, bool CAUSAL, bool MASKED = false, bool BLOCKS = false, bool CHUNKED = false,
          int WQ = kWaves>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, float* delta, int N, int BH, float c, float scale,
                      hipStream_t stream, int H = 1, int wl = -1, int wr = -1, const int* seqlens = nullptr,
                      const uint8_t* bmask = nullptr, int bq = 0, int bk = 0, int64_t bstride_b = 0,
                      int64_t bstride_h = 0) {
    const int n_qt = (N + 32 * WQ - 1) / (32 * WQ), n_kt = (N + kKeys - 1) / kKeys;
    // (plain causal: one workgroup per pair of tiles in both kernels, see PAIRED)
    constexpr bool paired = CAUSAL && !MASKED;
    const int Gq = BH * (paired ? (n_qt + 1) / 2 : n_qt), Gk = BH * (paired ? (n_kt + 1) / 2 : n_kt);
    const auto* Q = static_cast<const uint16_t*>(q);
    const auto* K = static_cast<const uint16_t*>(k);
    const auto* V = static_cast<const uint16_t*>(v);
    const auto* dO = static_cast<const uint16_t*>(dout);
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, BF16, CAUSAL, MASKED, BLOCKS, CHUNKED, WQ>), dim3(Gq), dim3(64 * WQ), 0, stream, Q,
                       K, V, static_cast<const uint16_t*>(o), dO, lse, delta, static_cast<uint16_t*>(dq), N, n_qt, Gq,
                       c, scale, H, wl, wr, seqlens, bmask, bq, bk, bstride_b, bstride_h);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, BF16, CAUSAL, MASKED, BLOCKS, CHUNKED>), dim3(Gk), dim3(kThreads), 0, stream,
                       Q, K, V, dO, lse, delta, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), N, n_kt, Gk,
                       c, scale, H, wl, wr, seqlens, bmask, bq, bk, bstride_b, bstride_h);
    return hipGetLastError();
}

// Checks shared by the backward entry points (everything but the mask).
int validate_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                 int dtype) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (N * d * 2 > INT32_MAX) return FA_ERR_SHAPE;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    const int64_t n_t = (N + kKeys - 1) / kKeys;  // the larger of the two grids
    if (B > INT32_MAX || H > INT32_MAX || B * H > INT32_MAX / n_t) return FA_ERR_SHAPE;
    if (B * H * N > INT64_MAX / (d * 2)) return FA_ERR_SHAPE;
    auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(dout, 16) ||
        misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) || misaligned(lse, 4) || misaligned(delta, 4))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
    const size_t nb = static_cast<size_t>(B * H * N * d * 2);
    const size_t lb = static_cast<size_t>(B * H * N * 4);
    const void* ins[6] = {q, k, v, o, dout, lse};
    const size_t in_sz[6] = {nb, nb, nb, nb, nb, lb};
    const void* outs[4] = {dq, dk, dv, delta};
    const size_t out_sz[4] = {nb, nb, nb, lb};
    for (int a = 0; a < 4; ++a) {
        for (int i = 0; i < 6; ++i)
            if (overlaps(outs[a], out_sz[a], ins[i], in_sz[i])) return FA_ERR_ALIAS;
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], out_sz[a], outs[b], out_sz[b])) return FA_ERR_ALIAS;
    }
    return FA_OK;
}

// The window of a fa_mask (NULL: none) as the kernels take it; a window of N or more keys is no
// limit (as in fa_fwd_masked).
// The dQ kernel of fa_bwd_masked runs with 4-wave workgroups of 128 query rows at d = 64 always,
// and at d = 128 for windows of at most kNarrowDqKeys keys (window_left + window_right + 1, both
// limited): a workgroup spans fewer keys beyond its rows' windows, and two share a compute unit.
// Measured on the whole fa_bwd_masked call on one MI355X (B1 H32 N8192): d = 64 gains 0.5-12%
// at every window tried; d = 128 gains 2.5-7% up to 2048 keys and loses 1% at 4096 (both sides).
constexpr int64_t kNarrowDqKeys = 2048;
// The dQ kernel of fa_bwd_blocksparse always runs with 4-wave workgroups: it computes each listed
// tile start to finish in one wave, and two workgroups per compute unit overlap their matrix and
// vector work. Whole call, one MI355X, B1 H32 N8192, random masks: +3% .. +11% at d = 128 (blocks
// of 64 .. 256, densities 0.1 .. 0.5), +11% .. +12% at d = 64.
constexpr int kBlocksDqWaves = 4;

int read_mask(const fa_mask* mask, int64_t N, int& wl, int& wr, const int32_t*& seqlens) {
    wl = wr = -1;
    seqlens = nullptr;
    if (!mask) return FA_OK;
    if (mask->window_left < -1 || mask->window_right < -1 || mask->window_left > INT32_MAX ||
        mask->window_right > INT32_MAX)
        return FA_ERR_OPTION;
    if (reinterpret_cast<uintptr_t>(mask->seqlens_k) & 3) return FA_ERR_ALIGN;
    wl = mask->window_left >= N - 1 ? -1 : static_cast<int>(mask->window_left);
    wr = mask->window_right >= N - 1 ? -1 : static_cast<int>(mask->window_right);
    seqlens = mask->seqlens_k;
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
           int causal, hipStream_t stream, fa_dtype dtype) {
    const int st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    const float c = scale * kLog2e;
    const int n = static_cast<int>(N), BH = static_cast<int>(B * H);
    const bool bf = dtype == FA_BF16;
    hipError_t e;
    if (d == 64) {
        if (bf) e = causal ? launch_bwd<64, true, true>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c, scale, stream)
                           : launch_bwd<64, true, false>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c, scale, stream);
        else e = causal ? launch_bwd<64, false, true>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c, scale, stream)
                        : launch_bwd<64, false, false>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c, scale, stream);
    } else {
        if (bf) e = causal ? launch_bwd<128, true, true>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c, scale, stream)
                           : launch_bwd<128, true, false>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c, scale, stream);
        else e = causal ? launch_bwd<128, false, true>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c, scale, stream)
                        : launch_bwd<128, false, false>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c, scale, stream);
    }
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                  hipStream_t stream, fa_dtype dtype, const fa_mask* mask) {
    const int st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    if (!mask) return FA_ERR_NULL;
    int wl, wr;
    const int32_t* seqlens;
    const int ms = read_mask(mask, N, wl, wr, seqlens);
    if (ms != FA_OK) return ms;
    if (!seqlens && wl == -1 && (wr == -1 || wr == 0))
        return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, wr == 0 ? 1 : 0, stream, dtype);
    const float c = scale * kLog2e;
    const int n = static_cast<int>(N), BH = static_cast<int>(B * H), h = static_cast<int>(H);
    const bool bf = dtype == FA_BF16;
    const bool narrow = d == 64 || (wl >= 0 && wr >= 0 && (int64_t)wl + wr + 1 <= kNarrowDqKeys);
    hipError_t e;
#define FA_BWD_MASKED(DD, BB, WQ)                                                                              \
    launch_bwd<DD, BB, false, true, false, false, WQ>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c, scale, \
                                                      stream, h, wl, wr, seqlens)
    if (d == 64)
        e = bf ? FA_BWD_MASKED(64, true, 4) : FA_BWD_MASKED(64, false, 4);
    else
        e = narrow ? (bf ? FA_BWD_MASKED(128, true, 4) : FA_BWD_MASKED(128, false, 4))
                   : (bf ? FA_BWD_MASKED(128, true, kWaves) : FA_BWD_MASKED(128, false, kWaves));
#undef FA_BWD_MASKED
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t N,
                       int64_t d, float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask,
                       const fa_block_mask* blocks) {
    const int st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    if (!blocks || !blocks->mask) return FA_ERR_NULL;
    if (blocks->block_q < 64 || blocks->block_k < 64 || blocks->block_q % 64 != 0 || blocks->block_k % 64 != 0 ||
        blocks->block_q > INT32_MAX || blocks->block_k > INT32_MAX || blocks->stride_b < 0 || blocks->stride_h < 0)
        return FA_ERR_OPTION;
    int wl, wr;
    const int32_t* seqlens;
    const int ms = read_mask(mask, N, wl, wr, seqlens);
    if (ms != FA_OK) return ms;
    const float c = scale * kLog2e;
    const int n = static_cast<int>(N), BH = static_cast<int>(B * H), h = static_cast<int>(H);
    const int bq = static_cast<int>(blocks->block_q), bk = static_cast<int>(blocks->block_k);
    const bool bf = dtype == FA_BF16;
    hipError_t e;
    // One work list holds every 64-key (dQ) or 64-row (dK, dV) tile up to 64 * kMaxListTiles;
    // longer sequences take the kernels that build it a chunk at a time (they need more registers).
    const bool chunked = N > static_cast<int64_t>(kKeyTile) * kMaxListTiles ||
                         N > static_cast<int64_t>(kQueryTile) * kMaxListTiles;
#define FA_BWD_BLOCKS(DD, BB, CH)                                                                                 \
    launch_bwd<DD, BB, false, true, true, CH, kBlocksDqWaves>(q, k, v, o, dout, lse, dq, dk, dv, delta, n, BH, c,      \
                                                             scale, stream, h, wl, wr, seqlens, blocks->mask, bq, bk, \
                                                             blocks->stride_b, blocks->stride_h)
    if (d == 64) {
        if (chunked)
            e = bf ? FA_BWD_BLOCKS(64, true, true) : FA_BWD_BLOCKS(64, false, true);
        else
            e = bf ? FA_BWD_BLOCKS(64, true, false) : FA_BWD_BLOCKS(64, false, false);
    } else {
        if (chunked)
            e = bf ? FA_BWD_BLOCKS(128, true, true) : FA_BWD_BLOCKS(128, false, true);
        else
            e = bf ? FA_BWD_BLOCKS(128, true, false) : FA_BWD_BLOCKS(128, false, false);
    }
#undef FA_BWD_BLOCKS
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"

