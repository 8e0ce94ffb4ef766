// Exact tiled-softmax attention forward for gfx950 (CDNA4), behind the C ABI of fa_fwd.h.
//
// One workgroup = 8 waves = 256 query rows of one (batch, head) (4 waves = 128 rows at d = 64,
// for the masked kernel's narrow-window form and for the block-sparse kernels); each wave owns
// 32 rows, as two 16-row blocks whose Q operands stay in registers for the whole kernel. A plain
// causal workgroup takes two query tiles in turn, a long and a short one. The workgroup walks the
// keys in tiles of 64 (ascending), staging each K and V tile in LDS with coalesced 16-byte loads
// (LDS DMA) issued ahead of use. Per tile and wave:
//
//   S^T = K_tile . Q^T          v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulate; each K operand
//                               read from LDS feeds both query blocks. Computing the transpose
//                               puts one query row in each lane column (the four 16-lane rows
//                               of a wave hold different keys of the same query rows), so the
//                               row sum and max are in-lane work plus two cross-row exchanges
//                               (v_permlane16_swap, v_permlane32_swap).
//   mask                        only on tiles that cross the causal diagonal, a window edge or
//                               the end of the sequence; masked scores become -inf first.
//   p, l                        online softmax in log2 units: p = exp2(s*c - m*c), with
//                               c = scale*log2(e) folded into one fma, against a reference m.
//                               f16: m moves (with the alpha rescale of l and o~) only when a
//                               tile's sums show a p above 2^tau. bf16: m is the exact running
//                               maximum, from a row max taken while the other product runs.
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
// FlashAttention-2 remark on "Decoding flash attention" (bibekananda.in), "Later versions". The
// rescaling identity holds for any reference value, so the reference need not be the running
// max: the f16 kernels keep every unnormalised p within 2^tau and test that on the tile sums they
// form anyway, instead of taking a max over every tile. The bf16 kernels keep the exact running
// maximum, the recurrence as "transformer math: flash attention math" writes it: bf16 keeps 8
// significant bits, so a probability rounded to it is off by up to 2^-8 of itself, and with a
// lazy reference the largest weights of a row all carry that error; against the exact maximum
// the largest one is exactly 1. (With the lazy reference a peaked bf16 row, logits of standard
// deviation 9, measured 1.02e-2 from the fp64 result, above the 1e-2 bound; an emulation of these
// roundings reproduces that value and gives 5.6e-3 for the exact maximum.)

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <algorithm>
#include <mutex>

#include "fa_fwd.h"
#include "fa_device.h"

namespace {

using namespace fa_detail;

constexpr int kWaves = 8;             // two groups of 4; each SIMD runs one wave of each group
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockM = 32 * kWaves;  // query rows per workgroup (32 per wave)
constexpr int kBlockN = 64;           // keys per tile
constexpr float kDefaultRescaleLog2 = 8.f;  // default reference-max threshold (log2 units)

// SPLIT: the key range of every query tile is cut into n_split equal runs of tiles, one per
// workgroup; each writes its partial result (O normalised over its own keys, in fp32, and the
// log-sum-exp of its keys) to PO / PL, and fa_merge_kernel combines them (split-KV).
// MASKED: a general mask in place of CAUSAL: key j is allowed for query i when
// i - wl <= j (wl >= 0), j <= i + wr (wr >= 0) and j < seqlens[b] (seqlens given). Key tiles
// outside the workgroup's window are neither loaded nor computed; a row with no allowed key
// gets o = 0 and lse = -inf.
// CHUNKED (with BLOCKS): the list of needed key tiles is built and walked kMaxListTiles candidates
// at a time, for sequences longer than one list holds (64 * kMaxListTiles keys).
// WV: waves per workgroup (query rows 32 * WV). The general mask (MASKED without BLOCKS) also
// runs with 4 waves for narrow windows: a workgroup then spans fewer keys beyond its own rows'
// windows, and two workgroups share a compute unit, so one's waves run while the other's wait at
// barriers for tiles outside their window. The block-sparse kernels (BLOCKS) always run with 4:
// their schedule computes a tile start to finish in one wave, and the other workgroup's waves
// supply the overlap of matrix and vector work.
template <int D, bool BF16, bool CAUSAL, bool SPLIT = false, bool MASKED = false, bool BLOCKS = false,
          bool CHUNKED = false, int WV = kWaves>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_qt, int G, float c, float tau_raw,
    int n_split = 1, float* __restrict__ PO = nullptr, float* __restrict__ PL = nullptr, int H = 1, int wl = -1,
    int wr = -1, const int* __restrict__ seqlens = nullptr, const uint8_t* __restrict__ bmask = nullptr,
    int bq = 0, int bk = 0, int64_t bstride_b = 0, int64_t bstride_h = 0) {
    static_assert(!(MASKED && CAUSAL), "the general mask replaces the causal one");
    static_assert(!BLOCKS || MASKED, "the block mask rides on the general mask");
    static_assert(!CHUNKED || BLOCKS, "chunks are chunks of the block-sparse work list");
    static_assert(WV == kWaves || (WV == 4 && (MASKED || D == 64)),
                  "4-wave workgroups: the masked and block-sparse kernels, and d = 64");
    constexpr int kBM = 32 * WV;               // query rows per workgroup
    constexpr int DT = D / 32;                 // 32-column k-steps of the first product
    constexpr int DB = D / 16;                 // 16-column blocks of the output
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;              // rows one wave-wide 1 KiB load covers
    constexpr int IPW = kBlockN / RPI / WV;    // such loads per wave per tile (each of K, V)
    constexpr int TILE = kBlockN * D;          // elements per tile
    static_assert(IPW >= 1 && IPW * RPI * WV == kBlockN, "tile must split evenly over the waves");

    // Two buffers for K and up to four for V, filled straight from global memory (LDS DMA,
    // lds_load16) in the swizzled layout. A ds_read address is a register plus an immediate below
    // 64 KiB, so a buffer that starts above 64 KiB costs registers of its own for its operand
    // addresses; the V buffers (each step reads V^T operands at 8 column blocks, K at 4 column
    // steps) take the larger alignment, which places them first. (Separate arrays let the
    // compiler see that the loads into one buffer never alias the reads of another.)
    __shared__ __attribute__((aligned(8192))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(8192))) uint16_t v_lds1[TILE];
    __shared__ __attribute__((aligned(8192))) uint16_t v_lds2[TILE];
    __shared__ __attribute__((aligned(8192))) uint16_t v_lds3[TILE];
    __shared__ __attribute__((aligned(4096))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(4096))) uint16_t k_lds1[TILE];

    // With SPLIT, a "virtual head" vh = bh * n_split + split takes the place of bh in the map, so
    // the workgroups that share one split's keys of one head sit together on an XCD.
    // PAIRED (plain causal): workgroup p of a head takes query tile n_qt - 1 - p and then tile p,
    // so every workgroup has the same number of key tiles (n_qt + 1 per pair) and the grid holds
    // (n_qt + 1) / 2 workgroups per head: no long tail of lone long tiles, and the workgroups
    // that run together on an XCD walk the same head's K/V from its start (K/V re-reads beyond
    // L2: 1.32x the unavoidable bytes, against 1.89x one tile per workgroup, longest first).
    constexpr bool PAIRED = CAUSAL && !SPLIT && !MASKED;
    int vh, qt_first;
    map_block(blockIdx.x, G, PAIRED ? (n_qt + 1) / 2 : n_qt, CAUSAL && !PAIRED, vh, qt_first);
    const int n_pass = PAIRED && n_qt - 1 - qt_first != qt_first ? 2 : 1;
#pragma nounroll
    for (int pass = 0; pass < n_pass; ++pass) {
        if (pass) __syncthreads();  // every wave is done with the first tile's LDS buffers
        // (the thread index is hidden from the compiler in each pass, so it does not keep every
        // per-lane address of the tile loops live across both passes, which spills)
        int tid = threadIdx.x;
        if constexpr (PAIRED) asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = tid >> 6;
        // 16x16x32 products: lane l holds query column li = l % 16 of the S^T and O^T tiles, and row
        // group g = l / 16 (tile rows 4g .. 4g + 3; operand k slots 8g .. 8g + 7)
        const int g = lane >> 4;
        const int li = lane & 15;
        const int qt = PAIRED ? (pass == 0 ? n_qt - 1 - qt_first : qt_first) : qt_first;
        const int bh = SPLIT ? vh / n_split : vh;
        const int q0 = qt * kBM;
        const int64_t head = (int64_t)bh * N * D;
        const uint16_t* Qh = Q + head;
        const uint16_t* Kh = K + head;
        const uint16_t* Vh = V + head;
        const int wq0 = q0 + 32 * wave;  // first query row of this wave (two 16-row blocks)

        const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
        const int T_all = (kv_end + kBlockN - 1) / kBlockN;  // key tiles of this query tile
        // tiles tb .. tb + T - 1 are this workgroup's (all of them without SPLIT); tile indices below
        // are relative to tb
        int tb = 0, T = T_all;
        if constexpr (SPLIT) {
            const int per = (T_all + n_split - 1) / n_split;
            tb = (vh % n_split) * per;
            T = max(0, min(T_all, tb + per) - tb);
        }
        // MASKED: kv_len keys exist for this batch; the workgroup's rows q0 .. q0 + 255 need keys
        // [lo, hi), a range of whole tiles from tb
        int kv_len = N;
        if constexpr (MASKED) {
            if (seqlens != nullptr) kv_len = min(max(seqlens[bh / H], 0), N);
            const int lo = wl >= 0 ? max(0, q0 - wl) : 0;
            const int hi = wr >= 0 ? min(kv_len, q0 + kBM + wr) : kv_len;
            tb = lo / kBlockN;
            T = max(0, (hi + kBlockN - 1) / kBlockN - tb);
            if constexpr (SPLIT) {  // this split's run of the window's tiles (possibly none; BLOCKS lists within it)
                const int per = (T + n_split - 1) / n_split;
                const int s0 = (vh % n_split) * per;
                tb += s0;
                T = max(0, min(T, s0 + per) - s0);
            }
        }
        // BLOCKS: of the tiles tb .. tb + T - 1, those that some wave of the workgroup needs (its
        // rows' query block has a non-zero byte for the tile's key block), compacted into t_list
        // (absolute tile index) with one bit per wave in t_wm; from here on a tile index j is a
        // position in that list. (Block sizes are multiples of 64: one byte decides a wave's whole
        // 32 x 64 part of a tile.) CHUNKED builds the list in the schedule, a chunk at a time.
        __shared__ int t_list[BLOCKS ? kMaxListTiles : 1];
        __shared__ uint8_t t_wm[BLOCKS ? kMaxListTiles : 1];
        __shared__ int t_cnt[BLOCKS ? WV : 1];
        const uint8_t* mb = BLOCKS ? bmask + (int64_t)(bh / H) * bstride_b + (int64_t)(bh % H) * bstride_h : nullptr;
        const int n_kb = BLOCKS ? (N + bk - 1) / bk : 0;
        auto need = [&](int w, int t) {
            const int r0 = q0 + 32 * w;
            return r0 < N && mb[(int64_t)(r0 / bq) * n_kb + t * kBlockN / bk] != 0;
        };
        if constexpr (BLOCKS && !CHUNKED) T = compact_tiles<WV>(tb, T, need, t_list, t_wm, t_cnt, tid);
        // tiles this wave computes: causal waves stop at the tile holding their last row
        // (Non-causal: T_w = T, hidden from the compiler. Folded away, the tests on it disappear and
        // the compiler keeps the output accumulators of the loop's two exit paths in two register
        // sets, which spills; a per-lane opaque value keeps the control flow of the causal kernel.)
        int T_w = CAUSAL ? max(0, min(T, (min(wq0 + 32, N) + kBlockN - 1) / kBlockN - tb)) : T;
        // MASKED: this wave's key tiles are T_w0 .. T_w - 1 (a window leaves the first ones to the
        // workgroup's earlier rows); the wave joins every barrier and load but computes only those
        int T_w0 = 0;
        if constexpr (MASKED && !BLOCKS) {  // (the block-sparse schedule tests each tile's bits instead)
            const int hi_w = wr >= 0 ? min(kv_len, wq0 + 32 + wr) : kv_len;  // this wave's last key + 1
            T_w = max(0, min(T, (hi_w + kBlockN - 1) / kBlockN - tb));
            // (a split may start past the wave's first tile: the wave then computes from its first)
            if (wl >= 0) T_w0 = max(0, min(T_w, max(0, wq0 - wl) / kBlockN - tb));
        }
        if constexpr (!CAUSAL && !MASKED) asm volatile("" : "+v"(T_w));

        // Load g of a tile covers rows RPI*g .. RPI*g+RPI-1; lane l writes LDS bytes [1024 g + 16 l,
        // +16), i.e. row RPI*g + l/CPR at chunk position l % CPR, which holds global chunk
        // (l % CPR) ^ swz_k(row) (K tiles) or ^ swz_v(row) (V tiles). Those per-lane byte offsets
        // within a tile are fixed (koffs, voffs); a tile moves only the buffer descriptor's base (a
        // scalar add), and the descriptor's size ends at the head's last row, so rows past the end of
        // the sequence read as zero (those keys are masked to -inf before they can carry weight).
        // A tile that starts at or past the end (the first tile of an empty split-KV run or
        // block-sparse list, loaded before the loop whatever the run's length) gets size 0, so every
        // lane reads zero and nothing past the tensor is touched: a negative size would be taken as
        // a huge unsigned one and the loads would run past the end of the tensor.
        // Offsets inside one head fit in 32 bits (the host limits N * d * 2 bytes to < 2^31).
        const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // scalar copy for LDS destinations
        unsigned koffs[IPW], voffs[IPW];
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int ld = wave_s * IPW + i;
            const int r = RPI * ld + lane / CPR;
            koffs[i] = 2u * (unsigned)(r * D + 8 * ((lane % CPR) ^ swz_k<D>(r)));
            voffs[i] = 2u * (unsigned)(r * D + 8 * ((lane % CPR) ^ swz_v<D>(r)));
        }
        auto issue = [&](const uint16_t* src_head, int j, uint16_t* dst, bool v_tile) __attribute__((always_inline)) {
            const int k0 = __builtin_amdgcn_readfirstlane((BLOCKS ? t_list[j] : tb + j) * kBlockN);
            const int nb = max(0, N - k0) * D * 2;
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int ld = wave_s * IPW + i;
                lds_load16(src_head + (int64_t)k0 * D, nb, v_tile ? voffs[i] : koffs[i], (lds_void*)(dst + ld * 512));
            }
        };

        // The k slots 8g .. 8g + 7 of k-step t of the first product are the columns of 16-byte chunk
        // t + DT*g (any one-to-one map of (t, g) to chunks sums every column once; with this one the
        // K operand reads, one chunk per lane group, are free of bank conflicts).
        // This lane's two query rows (wq0 + li and wq0 + 16 + li, query blocks qb = 0, 1) as B
        // operands of the first product, held in registers for the whole kernel. Rows past N repeat
        // row N-1 (never stored).
        u32x4 qf[2][DT];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const uint16_t* qrp = Qh + (int64_t)min(wq0 + 16 * qb + li, N - 1) * D + 8 * DT * g;
#pragma unroll
            for (int t = 0; t < DT; ++t) qf[qb][t] = *reinterpret_cast<const u32x4*>(qrp + 8 * t);
        }

        // O^T of this wave: block (qb, b) holds columns d = 16b + 4g .. +3 of query row wq0 + 16qb + li
        f32x4 oacc[2][DB];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int b = 0; b < DB; ++b) oacc[qb][b] = (f32x4){};
        unsigned pk[2][2][4];  // P^T of the tile between its softmax and its product with V: [qb][kk][.]
        // per query row (qb): reference max of raw dot products for l and oacc, and this lane's quarter
        // of the running denominator: f16 sums the rounded p (the weights the second product uses);
        // bf16 sums the unrounded p in fp32 (8 mantissa bits would leave lse short of 1e-3 on rows with
        // few keys; against the exact running maximum, normalising by this sum is as accurate as by
        // the rounded one, and one sum serves O and lse)
        float m_run[2] = {-INFINITY, -INFINITY};
        float l_run[2] = {0.f, 0.f};
        // the current tile's part of l_run, added once the tile is accepted (settle)
        float l_tile[2] = {0.f, 0.f};
        // EXACT (bf16): the reference is the exact running maximum of each row, moved whenever a
        // tile's max exceeds it (tau is not used). Otherwise (f16) the lazy reference below.
        constexpr bool EXACT = BF16;
        // bound on every unnormalised p: 2^tau_log2 (tau_raw is tau_log2 in raw score units)
        const float p_cap = __builtin_amdgcn_exp2f(tau_raw * c);
        // a moved reference sits this far above the maximum that moved it (0 for tau = 0, where it is
        // the exact running maximum), so later scores must rise by more before it moves again
        const float headroom = EXACT ? 0.f : 0.5f * tau_raw;
        const float move_above = EXACT ? 0.f : tau_raw;  // a row moves when its max exceeds m + this

        // LDS operand addresses (elements). Both swizzles depend on row & 15 only, so moving 16 rows
        // down a tile is the constant offset 16*D: one address per k-step serves the four 16-key
        // blocks of the K tile, and one per column block serves both 32-key steps of the V tile.
        int koff[DT];
#pragma unroll
        for (int t = 0; t < DT; ++t) koff[t] = tile_off_k<D>(li, t + DT * g);
        // ds_read_b64_tr_b16: within each 16-lane group, lane i receives element e from the 4 values
        // lane 4e + i/4 points at, position i % 4. Lane s of group g points at key row 4g + s/4,
        // columns 16b + 4(s % 4) .. +3, so lane i receives V[4g + e][16b + i] for e = 0..3: one V^T
        // row (column d = 16b + i) over 4 keys. The second read takes keys 16 + 4g .. +3.
        int voff[DB];
#pragma unroll
        for (int b = 0; b < DB; ++b) voff[b] = tile_off_v<D>(4 * g + (li >> 2), 2 * b + ((li & 3) >> 1)) + 4 * (li & 1);
        // A operand of S^T: keys 16kb + li, chunk t + DT*g
        auto k_operand = [&](const uint16_t* kt, int t, int kb) __attribute__((always_inline)) {
            return *reinterpret_cast<const u32x4*>(kt + koff[t] + kb * 16 * D);
        };
        // A operand of O^T: V^T rows d = 16b + li; its k slots 8g + s are keys 32kk + 4g + s (s < 4)
        // and 32kk + 16 + 4g + s - 4 (s >= 4), the order in which this lane holds P^T
        auto v_operand = [&](const uint16_t* vt, int kk, int b) __attribute__((always_inline)) {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + voff[b] + kk * 32 * D));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + voff[b] + kk * 32 * D + 16 * D));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
            return (u32x4){lo2[0], lo2[1], hi2[0], hi2[1]};
        };
        // B operand of O^T: P^T of query block qb over the 32 keys of step kk
        auto p_operand = [&](int qb, int kk) __attribute__((always_inline)) {
            return (u32x4){pk[qb][kk][0], pk[qb][kk][1], pk[qb][kk][2], pk[qb][kk][3]};
        };

        // ---- the pieces of one tile's work ----
        // S^T of two consecutive tiles (one being produced, one being consumed): [qb][kb] holds keys
        // 16kb + 4g .. +3 of query row wq0 + 16qb + li
        f32x4 s0[2][4], s1[2][4];
        float mc[2] = {0.f, 0.f};  // m_run * c with m_run the current reference (0 while m_run = -inf)

        // S^T(t) = K(t) . Q^T into s (32 MFMAs for D = 128; each K operand feeds both query blocks)
        auto qk = [&](const uint16_t* kt, f32x4 (&sd)[2][4]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4 * DT; ++i) {
                const int t = i >> 2, kb = i & 3;
                const u32x4 a = k_operand(kt, t, kb);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) sd[qb][kb] = mfma16<BF16>(a, qf[qb][t], t == 0 ? (f32x4){} : sd[qb][kb]);
            }
        };
        // O^T += V(t)^T . P^T (32 MFMAs for D = 128; each V^T operand feeds both query blocks)
        auto pv = [&](const uint16_t* vt) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2 * DB; ++i) {
                const int kk = i / DB, b = i % DB;
                const u32x4 a = v_operand(vt, kk, b);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) oacc[qb][b] = mfma16<BF16>(a, p_operand(qb, kk), oacc[qb][b]);
            }
        };
        // keys past the end, and (causal) keys after the query, become -inf before the max
        auto mask = [&](int t, f32x4 (&sd)[2][4]) __attribute__((always_inline)) {
            const int k0 = (BLOCKS ? t_list[t] : tb + t) * kBlockN;
            if constexpr (MASKED) {
                if ((k0 + kBlockN > kv_len) || (wr >= 0 && k0 + kBlockN - 1 > wq0 + wr) ||
                    (wl >= 0 && k0 < wq0 + 31 - wl)) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int key = k0 + 16 * kb + 4 * g + r, qrow = wq0 + 16 * qb + li;
                                if (key >= kv_len || (wr >= 0 && key > qrow + wr) || (wl >= 0 && key < qrow - wl))
                                    sd[qb][kb][r] = -INFINITY;
                            }
                }
                return;
            }
            if ((k0 + kBlockN > N) || (CAUSAL && k0 + kBlockN - 1 > wq0)) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = k0 + 16 * kb + 4 * g + r, qrow = wq0 + 16 * qb + li;
                            if (key >= N || (CAUSAL && key > qrow)) sd[qb][kb][r] = -INFINITY;
                        }
            }
        };
        // Move the reference max of each row (and rescale l, o~ by alpha = exp(m_old - m_new)) when
        // `force`, or when some row of the wave's 16-row block has a score more than tau above its
        // reference; otherwise p stays <= 2^tau_log2. mx0, mx1: the rows' maxima over the tile
        // (reduced over the four lane rows). The new reference is the larger of the old one and
        // max + headroom. (The two row blocks decide apart: under the exact running maximum a block
        // whose rows all keep their maximum skips the rescale, which is then the identity.)
        auto rebase = [&](float mx0, float mx1, bool force) __attribute__((always_inline)) {
            const float mx[2] = {mx0, mx1};
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                if (force || __builtin_amdgcn_ballot_w64(mx[qb] > m_run[qb] + move_above)) {
                    const float m_new = fmax_ieee(m_run[qb], EXACT ? mx[qb] : mx[qb] + headroom);
                    const float alpha = (m_new == m_run[qb]) ? 1.f : __builtin_amdgcn_exp2f((m_run[qb] - m_new) * c);
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int b = 0; b < DB; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r) oacc[qb][b][r] *= alpha;
                    m_run[qb] = m_new;
                    mc[qb] = (m_new == -INFINITY) ? 0.f : m_new * c;
                }
            }
        };
        auto rebase_from = [&](const f32x4 (&sd)[2][4], bool force) __attribute__((always_inline)) {
            float mx[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float m = fmaxf(sd[qb][0][0], sd[qb][0][1]);
#pragma unroll
                for (int e = 2; e < 16; ++e) m = fmaxf(m, sd[qb][e >> 2][e & 3]);
                mx[qb] = max_over_rows(m);
            }
            rebase(mx[0], mx[1], force);
        };
        // exponential pair pr (0..15) of S^T: p = exp2(s*c - m*c), rounded to the operand type, and the
        // row sum of the rounded values. Pair pr = 8qb + 2kb + r/2 lands in pk[qb][kb/2][2(kb%2) + r/2].
        auto exp_pair = [&](const f32x4 (&sd)[2][4], int pr) __attribute__((always_inline)) {
            const int qb = pr >> 3, kb = (pr >> 1) & 3, r = 2 * (pr & 1);
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sd[qb][kb][r], c, -mc[qb]));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sd[qb][kb][r + 1], c, -mc[qb]));
            unsigned& dst = pk[qb][kb >> 1][2 * (kb & 1) + (r >> 1)];
            dst = pack2<BF16>(p0, p1);
            // a row block's first pair (pr = 0, 8) starts the tile's sums (from -0, which folds away)
            const bool first = (pr & 7) == 0;
            if constexpr (BF16)
                l_tile[qb] = (first ? -0.f : l_tile[qb]) + (p0 + p1);
            else
                l_tile[qb] = add_pair<BF16>(dst, first ? -0.f : l_tile[qb]);
        };
        auto expo = [&](const f32x4 (&sd)[2][4]) __attribute__((always_inline)) {
#pragma unroll
            for (int pr = 0; pr < 16; ++pr) exp_pair(sd, pr);
        };
        // Accept the exponentials of a tile (taken against the current reference) when no lane's sum
        // of a row's values exceeds 2^tau_log2: then no single p does either, the bound the reference
        // max exists to keep. Otherwise (rare: the scores rose past the reference, or -- masked kernels
        // only -- a row has no reference yet) move the reference to the running max and take them
        // again. This replaces a max over every tile by a test on sums the softmax forms anyway. (In the
        // other kernels the first tile sets every row's reference: it holds key 0, or under split-KV a
        // key every row that has any key in the split can see.)
        // (EXACT: the reference already is the row's maximum over this tile, so every p <= 1.)
        auto settle = [&](const f32x4 (&sd)[2][4]) __attribute__((always_inline)) {
            if constexpr (!EXACT) {
                if (__builtin_amdgcn_ballot_w64(l_tile[0] > p_cap || l_tile[1] > p_cap ||
                                                (MASKED && (m_run[0] == -INFINITY || m_run[1] == -INFINITY)))) {
                    rebase_from(sd, true);
                    expo(sd);
                }
            }
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                l_run[qb] += l_tile[qb];
            }
        };

        // ---- schedule ----
        // Tile t's K sits in buffer t % 2. Iteration j runs, in each wave:
        //   region 1: S^T(j+1) = K(j+1) . Q^T on the matrix cores, with the exponentials of tile j
        //             (S^T(j) -> P^T(j)) interleaved between the MFMAs on the vector ALU;
        //   region 2: O^T += V(j)^T . P^T(j), with the row max of S^T(j+1) interleaved;
        //   then the (rare) move of the reference max for tile j+1, after P(j) has been used.
        // So each wave overlaps its own softmax with its own products, one tile apart. Barrier j
        // makes K(j+1) and V(j) visible (loaded after barrier j - 1) and frees the buffer of K(j) for
        // K(j+2) and one V buffer for V(j+1): V(j-1)'s when V alternates between two buffers (the
        // masked kernel), V(j-3)'s when it rotates through four (the ping-pong below).
        if constexpr (BLOCKS) {
            // Block-sparse schedule. Barrier j makes K(j) and V(j) visible (buffer j % 2) and frees
            // the other pair, which takes K(j+1) and V(j+1). A wave computes tile j start to finish
            // (scores, mask, max, exponentials, product with V) only when its own bit is set, so the
            // waves of a workgroup whose query blocks differ skip each other's tiles; the two waves
            // of a SIMD still overlap each other's matrix and vector work.
            const int wbit = 1 << wave_s;
            int Tc = T;  // entries of the list being walked
            auto tile = [&](int j, const uint16_t* kt, const uint16_t* vt, uint16_t* kn, uint16_t* vn)
                            __attribute__((always_inline)) {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();  // barrier j
                if (j + 1 < Tc) {
                    issue(Kh, j + 1, kn, false);
                    issue(Vh, j + 1, vn, true);
                }
                if (__builtin_amdgcn_readfirstlane(t_wm[j]) & wbit) {
                    qk(kt, s0);
                    mask(j, s0);
                    if constexpr (EXACT) rebase_from(s0, false);
                    expo(s0);
                    settle(s0);
                    pv(vt);
                }
            };
            auto walk = [&]() __attribute__((always_inline)) {
                issue(Kh, 0, k_lds0, false);
                issue(Vh, 0, v_lds0, true);
                for (int j = 0; j < Tc; j += 2) {
                    tile(j, k_lds0, v_lds0, k_lds1, v_lds1);
                    if (j + 1 >= Tc) break;
                    tile(j + 1, k_lds1, v_lds1, k_lds0, v_lds0);
                }
            };
            if constexpr (CHUNKED) {
                // The online state carries over from chunk to chunk. Every wave has left the previous
                // chunk's tiles (t_list, t_wm and both tile buffers read for the last time; no load in
                // flight) before the first barrier of compact_tiles, which writes the list only after it.
                for (int cb = 0; cb < T; cb += kMaxListTiles) {
                    Tc = compact_tiles<WV>(tb + cb, min(kMaxListTiles, T - cb), need, t_list, t_wm, t_cnt, tid);
                    if (Tc > 0) walk();
                }
            } else {
                walk();
            }
        } else {
            issue(Kh, 0, k_lds0, false);
            issue(Vh, 0, v_lds0, true);
            if (T > 1) issue(Kh, 1, k_lds1, false);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (T_w0 < T_w && T_w0 == 0) {  // the first tile sets the reference (m_run = -inf until then)
                qk(k_lds0, s0);
                mask(0, s0);
                rebase_from(s0, false);
            }
            // region 1 of tile j: S^T(j+1) = K(j+1) . Q^T with the exponentials of tile j in between.
            auto region1 = [&](f32x4 (&s_cur)[2][4], f32x4 (&s_nxt)[2][4], const uint16_t* k_nxt) __attribute__((always_inline)) {
                // Explicit software pipeline: the LDS operand of K step i + 2 is read before the two
                // MFMAs of step i issue, and the 16 pairs of exponentials are spread over the steps;
                // sched_barrier(0) pins that order so the LDS latency stays behind the MFMAs.
                constexpr int NK = 4 * DT;  // K operands: 16 for D = 128, 8 for D = 64
                constexpr int PPS = 16 / NK;  // exponential pairs per step: 1 (after the first MFMA) or 2
                static_assert(PPS == 1 || PPS == 2, "one or two pairs of exponentials per step");
                u32x4 ka[NK];
                ka[0] = k_operand(k_nxt, 0, 0);
                ka[1] = k_operand(k_nxt, 0, 1);
#pragma unroll
                for (int i = 0; i < NK; ++i) {
                    const int t = i >> 2, kb = i & 3;
                    if (i + 2 < NK) ka[i + 2] = k_operand(k_nxt, (i + 2) >> 2, (i + 2) & 3);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        s_nxt[qb][kb] = mfma16<BF16>(ka[i], qf[qb][t], t == 0 ? (f32x4){} : s_nxt[qb][kb]);
                        __builtin_amdgcn_sched_barrier(0);
                        if (PPS == 2 || qb == 0) exp_pair(s_cur, i * PPS + qb);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                // Keep the exponentials in region 1: without this the compiler sinks them past the
                // mask branch into region 2, next to their only consumer.
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(pk[qb][kk][r]));
                    asm volatile("" : "+v"(l_tile[qb]));
                }
            };
            // region 2 of tile j: O^T += V(j)^T . P^T(j). EXACT: the row maxima of S^T(j+1) (s_nxt,
            // already masked) are formed between the MFMAs, on the vector ALU this region leaves idle,
            // and the reference moves after the product, once P(j) (taken against the old one) is in;
            // `next` is false when there is no tile j+1.
            auto region2 = [&](const uint16_t* v_cur, const f32x4 (&s_nxt)[2][4], bool next) __attribute__((always_inline)) {
                // V^T operands read two steps ahead.
                constexpr int NV = 2 * DB;  // V^T operands: 16 for D = 128, 8 for D = 64
                constexpr int EPS = 32 / NV;  // scores of S^T(j+1) folded into the maxima per step
                u32x4 va[NV];
                float pm[2] = {-INFINITY, -INFINITY};  // this lane's maxima of the two rows
                va[0] = v_operand(v_cur, 0, 0);
                va[1] = v_operand(v_cur, 1 / DB, 1 % DB);
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    const int kk = i / DB, b = i % DB;
                    if (i + 2 < NV) va[i + 2] = v_operand(v_cur, (i + 2) / DB, (i + 2) % DB);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        oacc[qb][b] = mfma16<BF16>(va[i], p_operand(qb, kk), oacc[qb][b]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if constexpr (EXACT) {
#pragma unroll
                        for (int u = 0; u < EPS; ++u) {
                            const int e = i * EPS + u, qb = e >> 4, kb = (e >> 2) & 3, r = e & 3;
                            pm[qb] = fmaxf(pm[qb], s_nxt[qb][kb][r]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                if constexpr (EXACT) {
                    if (next) rebase(max_over_rows(pm[0]), max_over_rows(pm[1]), false);
                }
            };
            if constexpr (MASKED) {
                // every wave: barrier, loads, region 1, region 2 (V in two buffers)
                auto iteration = [&](int j, f32x4 (&s_cur)[2][4], f32x4 (&s_nxt)[2][4], const uint16_t* k_nxt,
                                     const uint16_t* v_cur, uint16_t* k_load, uint16_t* v_load) __attribute__((always_inline)) {
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();
                    if (j + 2 < T) issue(Kh, j + 2, k_load, false);
                    if (j + 1 < T) issue(Vh, j + 1, v_load, true);
                    if (j < T_w0) {
                        // before this wave's first tile: at most start the pipeline with S^T(j+1)
                        if (j + 1 == T_w0 && j + 1 < T_w) {
                            qk(k_nxt, s_nxt);
                            mask(j + 1, s_nxt);
                            rebase_from(s_nxt, false);
                        }
                    } else if (j + 1 < T_w) {
                        region1(s_cur, s_nxt, k_nxt);
                        settle(s_cur);
                        mask(j + 1, s_nxt);
                        region2(v_cur, s_nxt, true);
                    } else if (j < T_w) {
                        expo(s_cur);
                        settle(s_cur);
                        pv(v_cur);
                    }
                };
                for (int j = 0; j < T; j += 2) {
                    // even j: K(j+1) in buffer 1, V(j) in buffer 0; K(j+2) -> buffer 0, V(j+1) -> buffer 1
                    iteration(j, s0, s1, k_lds1, v_lds0, k_lds0, v_lds1);
                    if (j + 1 >= T) break;
                    iteration(j + 1, s1, s0, k_lds0, v_lds1, k_lds1, v_lds0);
                }
            } else {
                // Ping-pong. The two waves on a SIMD run the same sequence of regions half an iteration
                // apart: waves 0-3 pass barrier j before region 1 of tile j, waves 4-7 ("lag") before
                // region 2 of tile j-1. While one wave of the pair runs the exponentials of region 1 on
                // the vector ALU, the other runs the MFMA-only region 2, instead of both contending for
                // the vector ALU and then both for the matrix core. A lagging wave still reads V(j-1)
                // after barrier j, so V rotates through four buffers (V(t) in buffer t % 4). Every wave
                // issues its share of the loads of step j (K(j+2) into K(j)'s buffer, V(j+1) into
                // V(j-3)'s) at the top of the step, after barrier j in waves 0-3 and after region 2 of
                // tile j-1 in waves 4-7, and waits for them at the top of the next step: one
                // unconditional wait, so the compiler sees no path on which a read could overtake them.
                // Without a causal mask every wave runs both regions in every step: the last step's
                // region 1 also forms an S^T(T) that nothing uses (from a stale K buffer, no load in
                // flight into it; masked, and kept out of the bf16 maximum), which costs one tile of
                // the first product but leaves a step one path, with no second set of per-step tests.
                // (The test on the opaque T_w stays: the compiler keeps the same registers for the
                // loop's exits only while the branches around the regions are per-lane ones.)
                const bool lag = wave_s >= WV / 2;
                auto step = [&](int j, f32x4 (&s_cur)[2][4], f32x4 (&s_nxt)[2][4], uint16_t* k_cur, const uint16_t* k_nxt,
                                const uint16_t* v_cur, uint16_t* v_p1) __attribute__((always_inline)) {
                    __builtin_amdgcn_s_waitcnt(0);
                    if (!lag) __syncthreads();  // barrier j
                    if (j + 2 < T) issue(Kh, j + 2, k_cur, false);
                    if (j + 1 < T) issue(Vh, j + 1, v_p1, true);
                    if (CAUSAL ? j + 1 < T_w : j < T_w) {
                        region1(s_cur, s_nxt, k_nxt);
                        settle(s_cur);
                        mask(j + 1, s_nxt);
                    } else if (CAUSAL && j < T_w) {
                        expo(s_cur);
                        settle(s_cur);
                    }
                    if (lag && j + 1 < T) {
                        __builtin_amdgcn_s_waitcnt(0);
                        __syncthreads();  // barrier j + 1
                    }
                    if (CAUSAL ? j + 1 < T_w : j < T_w) {
                        region2(v_cur, s_nxt, j + 1 < T);
                    } else if (CAUSAL && j < T_w) {
                        pv(v_cur);
                    }
                };
                if (lag && T > 0) __syncthreads();  // barrier 0
                // T barriers in every wave: waves 0-3 one per step; waves 4-7 barrier 0 above and one
                // per step but the last
                for (int j = 0; j < T; j += 4) {
                    step(j, s0, s1, k_lds0, k_lds1, v_lds0, v_lds1);
                    if (j + 1 >= T) break;
                    step(j + 1, s1, s0, k_lds1, k_lds0, v_lds1, v_lds2);
                    if (j + 2 >= T) break;
                    step(j + 2, s0, s1, k_lds0, k_lds1, v_lds2, v_lds3);
                    if (j + 3 >= T) break;
                    step(j + 3, s1, s0, k_lds1, k_lds0, v_lds3, v_lds0);
                }
            }
        }

        // ---- epilogue: O = o~ / l, lse = m*scale + ln l, per query row (qb) ----
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qrow = wq0 + 16 * qb + li;
            const float l_tot = sum_over_rows(l_run[qb]);
            const float mcf = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb] * c;
            if constexpr (SPLIT) {
                // partial result over this split's keys; a row none of whose keys fall in the split
                // (l = 0) gets O = 0 and lse = -inf, i.e. zero weight in the merge
                if (qrow < N) {
                    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
                    float* prow = PO + ((int64_t)vh * N + qrow) * D;
#pragma unroll
                    for (int b = 0; b < DB; ++b) {
                        const float4 st = {oacc[qb][b][0] * inv, oacc[qb][b][1] * inv, oacc[qb][b][2] * inv,
                                           oacc[qb][b][3] * inv};
                        *reinterpret_cast<float4*>(prow + 16 * b + 4 * g) = st;
                    }
                    if (g == 0) {
                        // log-sum-exp of the denominator O was normalised by, in both slots: [0] weighs
                        // the merge, [1] forms the final lse (one sum serves both in this kernel)
                        const float ll = l_tot > 0.f ? (mcf + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
                        const float2 ls = {ll, ll};
                        *reinterpret_cast<float2*>(PL + 2 * ((int64_t)vh * N + qrow)) = ls;
                    }
                }
            } else if (qrow < N) {
                // (MASKED: a row with no allowed key has l = 0: o = 0, lse = -inf)
                const float inv = (!MASKED || l_tot > 0.f) ? 1.f / l_tot : 0.f;
                uint16_t* orow = O + head + (int64_t)qrow * D;
#pragma unroll
                for (int b = 0; b < DB; ++b) {
                    const u32x2 st = {pack2<BF16>(oacc[qb][b][0] * inv, oacc[qb][b][1] * inv),
                                      pack2<BF16>(oacc[qb][b][2] * inv, oacc[qb][b][3] * inv)};
                    *reinterpret_cast<u32x2*>(orow + 16 * b + 4 * g) = st;
                }
                if (LSE != nullptr && g == 0)
                    LSE[(int64_t)bh * N + qrow] = (!MASKED || l_tot > 0.f) ? (mcf + __log2f(l_tot)) * 0.69314718055994531f
                                                                           : -INFINITY;
            }
        }
    }  // pass
}

// ---------------------------------------------------------------------------------------------
// Merge of split-KV partial results. Each split s of a row holds O_s, its output normalised over
// the split's own keys, and L_s, the log-sum-exp of the split's logits. Rescaling every split to a
// common reference (the rescaling identity of "transformer math: flash attention math",
// aicassindra.com, "The rescaling identity, derived") gives exact attention over all keys, since
// grouping and order of the key blocks never enter the result (same page, "Proof of exactness"):
//     lse = ln sum_s exp(L_s),      o = sum_s exp(L_s - lse) O_s.
// One thread per (row, 8 output columns); memory-bound. PL holds two L per row (see the kernel).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float* __restrict__ PO, const float* __restrict__ PL,
                                                       uint16_t* __restrict__ O, float* __restrict__ LSE, int N,
                                                       int n_split, int64_t total) {
    constexpr int CPR = D / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;  // total = B * H * N * CPR
    const int64_t row = t / CPR;  // bh * N + i
    const int ch = (int)(t % CPR);
    const int64_t bh = row / N, i = row % N;
    const int64_t first = bh * n_split * (int64_t)N + i;  // partial (bh, split 0, i); split s is + s * N
    float mw = -INFINITY, ml = -INFINITY;
    for (int sp = 0; sp < n_split; ++sp) {
        const float2 L = *reinterpret_cast<const float2*>(PL + 2 * (first + (int64_t)sp * N));
        mw = fmaxf(mw, L.x);
        ml = fmaxf(ml, L.y);
    }
    if (mw == -INFINITY) {  // (masked) no split holds a key of this row: o = 0, lse = -inf
        *reinterpret_cast<u32x4*>(O + row * D + 8 * ch) = (u32x4){0u, 0u, 0u, 0u};
        if (LSE != nullptr && ch == 0) LSE[row] = -INFINITY;
        return;
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f, lsum = 0.f;
    for (int sp = 0; sp < n_split; ++sp) {
        const int64_t pr = first + (int64_t)sp * N;
        const float2 L = *reinterpret_cast<const float2*>(PL + 2 * pr);
        // exp2 of a non-positive argument; a split with no keys for this row has L = -inf: weight 0
        const float w = __builtin_amdgcn_exp2f((L.x - mw) * 1.4426950408889634f);
        lsum += __builtin_amdgcn_exp2f((L.y - ml) * 1.4426950408889634f);
        wsum += w;
        const float4* src = reinterpret_cast<const float4*>(PO + pr * D + 8 * ch);
        const float4 a = src[0], b = src[1];
        acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
        acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
    }
    const float inv = 1.f / wsum;  // the split with the largest L.x has weight 1, so wsum >= 1
    const u32x4 st = {pack2<BF16>(acc[0] * inv, acc[1] * inv), pack2<BF16>(acc[2] * inv, acc[3] * inv),
                      pack2<BF16>(acc[4] * inv, acc[5] * inv), pack2<BF16>(acc[6] * inv, acc[7] * inv)};
    *reinterpret_cast<u32x4*>(O + row * D + 8 * ch) = st;
    if (LSE != nullptr && ch == 0) LSE[row] = ml + __log2f(lsum) * 0.69314718055994531f;
}

// The masked kernel runs with 4-wave workgroups of 128 query rows at d = 64 always, and at d = 128
// for windows of at most this many keys (window_left + window_right + 1, both limited). Measured
// against 8-wave workgroups on one MI355X (B1 H32 N8192 and B4 H16 N2047): d = 64 gains at every
// window, 4% with one that masks nothing to 26% at 64 keys; d = 128 gains 3% at 2048 keys and up
// to 17% at 64, and loses 1-2% from about 3072 keys on.
constexpr int64_t kNarrowWindowKeys = 2048;

// The masked kernel with WV waves per workgroup; B*H*ceil(N / (32 WV)) workgroups.
template <int D, bool BF16, int WV>
hipError_t launch_masked(const void* q, const void* k, const void* v, void* o, float* lse, int N, int BH, float c,
                         float tau_raw, int H, int wl, int wr, const int* seqlens, hipStream_t stream) {
    const int n_qt = (N + 32 * WV - 1) / (32 * WV), G = BH * n_qt;
    hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, false, false, true, false, false, WV>), dim3(G), dim3(64 * WV), 0,
                       stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qt, G, c, tau_raw, 1,
                       nullptr, nullptr, H, wl, wr, seqlens);
    return hipGetLastError();
}

// Waves per workgroup of the block-sparse kernels (fa_fwd_blocksparse and its split-KV form).
// Against 8-wave workgroups on one MI355X (B1 H32 N8192, random masks): +8% .. +38% at d = 128
// over blocks of 64, 128 and 256 and densities 0.1 .. 0.5, +14% .. +33% at d = 64.
constexpr int kBlocksWaves = 4;

// WV waves per workgroup; B*H*ceil(N / (32 WV)) workgroups.
template <int D, bool BF16, int WV>
hipError_t launch_blocks(const void* q, const void* k, const void* v, void* o, float* lse, int N, int BH, float c,
                         float tau_raw, int H, int wl, int wr, const int* seqlens, const uint8_t* bm, int bq, int bk,
                         int64_t sb, int64_t sh, hipStream_t stream) {
    const int n_qt = (N + 32 * WV - 1) / (32 * WV), G = BH * n_qt;
    // one list holds every key tile up to 64 * kMaxListTiles keys; longer sequences take the
    // kernel that builds it a chunk at a time (it needs more registers)
    if (N <= kBlockN * kMaxListTiles)
        hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, false, false, true, true, false, WV>), dim3(G), dim3(64 * WV), 0,
                           stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qt, G, c, tau_raw, 1,
                           nullptr, nullptr, H, wl, wr, seqlens, bm, bq, bk, sb, sh);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, false, false, true, true, true, WV>), dim3(G), dim3(64 * WV), 0,
                           stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qt, G, c, tau_raw, 1,
                           nullptr, nullptr, H, wl, wr, seqlens, bm, bq, bk, sb, sh);
    return hipGetLastError();
}

// The general mask as the kernels take it (a window of N or more keys already turned into -1).
struct fa_mask_args {
    int H, wl, wr;
    const int* seqlens;
    bool narrow = false;  // run 4-wave workgroups
};
// A block mask as the kernels take it.
struct fa_block_args {
    const uint8_t* mask;
    int bq, bk;
    int64_t sb, sh;
};

template <int D, bool BF16, bool CAUSAL>
hipError_t launch_split(const void* q, const void* k, const void* v, void* o, float* lse, int N, int n_qt, int BH,
                        float c, float tau_raw, int n_split, float* po, float* pl, hipStream_t stream,
                        const fa_mask_args* m = nullptr, const fa_block_args* bl = nullptr) {
    const int G = BH * n_split * n_qt;
    // the 4-wave kernels' query tiles (block-sparse, narrow windows) have 128 rows
    static_assert(kBlocksWaves == 4, "one grid for the 4-wave kernels");
    const int n_qb = (N + 127) / 128, Gb = BH * n_split * n_qb;
    // (a split's run of key tiles can exceed one block-sparse list only past 64 * kMaxListTiles keys)
    if (bl != nullptr && N <= kBlockN * kMaxListTiles)
        hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, false, true, true, true, false, kBlocksWaves>), dim3(Gb),
                           dim3(64 * kBlocksWaves), 0, stream, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                           lse, N, n_qb, Gb, c, tau_raw, n_split, po, pl, m->H, m->wl, m->wr, m->seqlens, bl->mask,
                           bl->bq, bl->bk, bl->sb, bl->sh);
    else if (bl != nullptr)
        hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, false, true, true, true, true, kBlocksWaves>), dim3(Gb),
                           dim3(64 * kBlocksWaves), 0, stream, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                           lse, N, n_qb, Gb, c, tau_raw, n_split, po, pl, m->H, m->wl, m->wr, m->seqlens, bl->mask,
                           bl->bq, bl->bk, bl->sb, bl->sh);
    else if (m != nullptr && m->narrow)
        hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, false, true, true, false, false, 4>), dim3(Gb), dim3(256), 0,
                           stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qb, Gb, c, tau_raw,
                           n_split, po, pl, m->H, m->wl, m->wr, m->seqlens);
    else if (m != nullptr)
        hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, false, true, true>), dim3(G), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qt, G, c, tau_raw,
                           n_split, po, pl, m->H, m->wl, m->wr, m->seqlens);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, CAUSAL, true>), dim3(G), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qt, G, c, tau_raw,
                           n_split, po, pl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)BH * N * (D / 8);
    hipLaunchKernelGGL((fa_merge_kernel<D, BF16>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, po, pl,
                       static_cast<uint16_t*>(o), lse, N, n_split, total);
    return hipGetLastError();
}

// n_qt, G: 256-row query tiles and workgroups. d = 64 runs 4-wave (128-row) workgroups, two per
// CU: with half the matrix work per score of d = 128 the vector ALU bounds it, and two workgroups
// that do not share barriers keep it busier than one 8-wave workgroup's lock-stepped pairs.
template <int D, bool BF16, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int N, int n_qt, int G,
                  float c, float tau_raw, hipStream_t stream) {
    // (causal: one workgroup per pair of query tiles, see PAIRED in the kernel)
    const int BH = G / n_qt;
    if constexpr (D == 64) {
        const int n_qt4 = (N + 127) / 128, G4 = BH * (CAUSAL ? (n_qt4 + 1) / 2 : n_qt4);
        hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, CAUSAL, false, false, false, false, 4>), dim3(G4), dim3(256), 0,
                           stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qt4, G4, c,
                           tau_raw);
    } else {
        const int G8 = CAUSAL ? BH * ((n_qt + 1) / 2) : G;
        hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, CAUSAL>), dim3(G8), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qt, G8, c,
                           tau_raw);
    }
    return hipGetLastError();
}

// Checks shared by the forward entry points (everything but options and workspace). n_split
// multiplies the grid.
int validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int64_t B, int64_t H,
             int64_t N, int64_t d, float scale, int dtype, int64_t n_split) {
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
    if (N * d * 2 > INT32_MAX) return FA_ERR_SHAPE;  // one head of q, k or v stays under 2 GiB
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    const int64_t n_qt = (N + kBlockM - 1) / kBlockM;
    if (B > INT32_MAX || H > INT32_MAX || B * H > INT32_MAX / (n_qt * n_split)) return FA_ERR_SHAPE;
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
    return FA_OK;
}

constexpr int kMaxSplits = 64;

}  // namespace

// Fixed device scratch of fa_fwd_splitkv_noalloc: the split-KV partial results (O_s in fp32 and two
// log-sum-exps per row and split) for callers that cannot allocate. Each GPU the library runs on
// holds its own copy from the library's first use there until the process ends. Calls on one GPU
// share it, so calls that overlap on one GPU race; every split writes all of its rows' partials
// before the merge reads them, so nothing needs clearing between calls.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch`, looked up once per device with that device
// current (in host code the array's name is a host-side stand-in, not a device address); nullptr
// when the lookup fails.
void* scratch_for_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int fa_version(void) { return 200; }

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
        case FA_ERR_OPTION: return "option out of range (rescale threshold 0..15, variant 0..1, splits 1..64)";
        case FA_ERR_WORKSPACE: return "workspace is NULL, misaligned, too small or overlaps an argument";
        case FA_ERR_SCRATCH: return "split-KV partials exceed the library's fixed 64 MiB scratch (use fa_fwd_splitkv)";
        default: return "unknown status";
    }
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
              int64_t d, float scale, int causal, hipStream_t stream, fa_dtype dtype, const fa_fwd_options* opts) {
    const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, 1);
    if (st != FA_OK) return st;
    const int64_t n_qt = (N + kBlockM - 1) / kBlockM;
    const int64_t G = B * H * n_qt;
    // The reference max moves only when a score exceeds it by more than tau (log2 units), so the
    // unnormalised p stay <= 2^tau and most tiles skip the rescale; tau = 0 moves it on every
    // increase, the loop exactly as the pages write it.
    float tau = kDefaultRescaleLog2;
    if (opts) {
        if (!(opts->rescale_threshold_log2 >= 0.f && opts->rescale_threshold_log2 <= 15.f)) return FA_ERR_OPTION;
        if (opts->variant < 0 || opts->variant > 1) return FA_ERR_OPTION;
        tau = opts->rescale_threshold_log2;
    }

    const float c = scale * 1.4426950408889634f;  // scale * log2(e)
    const float tau_raw = tau / c;
    const int n = static_cast<int>(N), nq = static_cast<int>(n_qt), g = static_cast<int>(G);
    const bool bf = dtype == FA_BF16;
    hipError_t e;
#define FA_DISPATCH(L)                                                                                \
    if (d == 64) {                                                                                    \
        if (bf) e = causal ? L<64, true, true>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream)          \
                           : L<64, true, false>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream);        \
        else e = causal ? L<64, false, true>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream)            \
                        : L<64, false, false>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream);          \
    } else {                                                                                          \
        if (bf) e = causal ? L<128, true, true>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream)         \
                           : L<128, true, false>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream);       \
        else e = causal ? L<128, false, true>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream)           \
                        : L<128, false, false>(q, k, v, o, lse, n, nq, g, c, tau_raw, stream);         \
    }
    FA_DISPATCH(launch)
#undef FA_DISPATCH
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
           int64_t d, float scale, int causal, hipStream_t stream, fa_dtype dtype) {
    return fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype, nullptr);
}

int fa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                  int64_t N, int64_t d, float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask) {
    const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, 1);
    if (st != FA_OK) return st;
    if (!mask) return FA_ERR_NULL;
    if (mask->window_left < -1 || mask->window_right < -1 || mask->window_left > INT32_MAX ||
        mask->window_right > INT32_MAX)
        return FA_ERR_OPTION;
    if (reinterpret_cast<uintptr_t>(mask->seqlens_k) & 3) return FA_ERR_ALIGN;
    // A window of N - 1 or more keys is no limit (i - (N - 1) <= 0 <= j and j <= N - 1 <= i + N - 1);
    // as -1 it keeps the kernel's index sums below 2^31 and sends the plain masks to fa_fwd.
    const int64_t wl64 = mask->window_left >= N - 1 ? -1 : mask->window_left;
    const int64_t wr64 = mask->window_right >= N - 1 ? -1 : mask->window_right;
    // the two masks with kernels of their own
    if (!mask->seqlens_k && wl64 == -1 && (wr64 == -1 || wr64 == 0))
        return fa_fwd(q, k, v, o, lse, B, H, N, d, scale, wr64 == 0 ? 1 : 0, stream, dtype);
    const float c = scale * 1.4426950408889634f;
    const float tau_raw = kDefaultRescaleLog2 / c;
    const int n = static_cast<int>(N), bh = static_cast<int>(B * H);
    const int h = static_cast<int>(H), wl = static_cast<int>(wl64), wr = static_cast<int>(wr64);
    const bool bf = dtype == FA_BF16;
    const bool narrow = wl64 >= 0 && wr64 >= 0 && wl64 + wr64 + 1 <= kNarrowWindowKeys;
    hipError_t e;
#define FA_MASKED(DD, BB, WW) \
    launch_masked<DD, BB, WW>(q, k, v, o, lse, n, bh, c, tau_raw, h, wl, wr, mask->seqlens_k, stream)
    if (d == 64)
        e = bf ? FA_MASKED(64, true, 4) : FA_MASKED(64, false, 4);
    else if (narrow)
        e = bf ? FA_MASKED(128, true, 4) : FA_MASKED(128, false, 4);
    else
        e = bf ? FA_MASKED(128, true, kWaves) : FA_MASKED(128, false, kWaves);
#undef FA_MASKED
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                       int64_t N, int64_t d, float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask,
                       const fa_block_mask* blocks) {
    const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, 1);
    if (st != FA_OK) return st;
    if (!blocks || !blocks->mask) return FA_ERR_NULL;
    if (blocks->block_q < 64 || blocks->block_k < 64 || blocks->block_q % 64 != 0 || blocks->block_k % 64 != 0 ||
        blocks->block_q > INT32_MAX || blocks->block_k > INT32_MAX || blocks->stride_b < 0 || blocks->stride_h < 0)
        return FA_ERR_OPTION;
    int64_t wl64 = -1, wr64 = -1;
    const int32_t* seqlens = nullptr;
    if (mask) {
        if (mask->window_left < -1 || mask->window_right < -1 || mask->window_left > INT32_MAX ||
            mask->window_right > INT32_MAX)
            return FA_ERR_OPTION;
        if (reinterpret_cast<uintptr_t>(mask->seqlens_k) & 3) return FA_ERR_ALIGN;
        wl64 = mask->window_left >= N - 1 ? -1 : mask->window_left;
        wr64 = mask->window_right >= N - 1 ? -1 : mask->window_right;
        seqlens = mask->seqlens_k;
    }
    const float c = scale * 1.4426950408889634f;
    const float tau_raw = kDefaultRescaleLog2 / c;
    const int n = static_cast<int>(N), bh = static_cast<int>(B * H);
    const int h = static_cast<int>(H), wl = static_cast<int>(wl64), wr = static_cast<int>(wr64);
    const int bq = static_cast<int>(blocks->block_q), bk = static_cast<int>(blocks->block_k);
    const bool bf = dtype == FA_BF16;
    hipError_t e;
    // 128-row (4-wave) workgroups, two per compute unit: the block-sparse schedule computes each
    // tile start to finish in one wave, so the overlap of matrix and vector work comes from the
    // other workgroup's waves
#define FA_BLOCKS(DD, BB)                                                                                     \
    launch_blocks<DD, BB, kBlocksWaves>(q, k, v, o, lse, n, bh, c, tau_raw, h, wl, wr, seqlens, blocks->mask, bq, \
                                        bk, blocks->stride_b, blocks->stride_h, stream)
    if (d == 64)
        e = bf ? FA_BLOCKS(64, true) : FA_BLOCKS(64, false);
    else
        e = bf ? FA_BLOCKS(128, true) : FA_BLOCKS(128, false);
#undef FA_BLOCKS
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int num_splits) {
    if (num_splits <= 1 || num_splits > kMaxSplits || B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
    if (B * H > INT64_MAX / N / (d + 2) / 4 / num_splits) return 0;
    return static_cast<size_t>(num_splits * B * H * N * (d + 2) * 4);  // fp32 O_s [.., d] and two L_s per row
}

int fa_fwd_splitkv_heuristic(int64_t B, int64_t H, int64_t N, int64_t d, int causal) {
    if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 1;
    // Model, in microseconds. One workgroup runs per CU at a time (its registers fill the CU), so
    // G query tiles cut in S splits take ceil(G S / 256) rounds. A round costs the split's share of
    // the key tiles plus about two tiles of fill and drain, at about 2.2 us per 256 x 64 tile at
    // d = 128 (1000 TFLOP/s over 256 CUs); the merge moves (d + 2) * 4 bytes per row and split at
    // about 5 TB/s. Causal query tiles hold half the keys on average. (Measured on the thin grid
    // B1 H2 N16384 d128: 2 splits best, 4 and 8 slower by 3% and 10%; the model says 4% and 12%.)
    constexpr int64_t kCUs = 256;
    const int64_t n_qt = (N + kBlockM - 1) / kBlockM;
    const int64_t G = B * H * n_qt;
    const double tiles = (double)((N + kBlockN - 1) / kBlockN) / (causal ? 2.0 : 1.0);
    const double tile_us = 2.2 * (double)d / 128.0;
    const double merge_us = (double)(B * H * N) * (double)(d + 2) * 4.0 / 5e12 * 1e6;
    auto cost = [&](int64_t sp) {
        const double rounds = (double)((G * sp + kCUs - 1) / kCUs);
        return rounds * (tiles / (double)sp + 2.0) * tile_us + (sp > 1 ? (double)sp * merge_us : 0.0);
    };
    const int64_t s_max = std::max<int64_t>(1, std::min<int64_t>(kMaxSplits, (int64_t)(tiles / 4)));
    int64_t best = 1;
    double best_t = cost(1);
    for (int64_t sp = 2; sp <= s_max; ++sp) {
        const double t = cost(sp);
        if (t < best_t) {
            best_t = t;
            best = sp;
        }
    }
    return static_cast<int>(best);
}

// A split-KV workspace: large enough, 16-byte aligned, and clear of every tensor of the call.
static bool workspace_ok(const void* q, const void* k, const void* v, const void* o, const float* lse, int64_t B,
                         int64_t H, int64_t N, int64_t d, int num_splits, const void* workspace,
                         size_t workspace_bytes) {
    const size_t need = fa_fwd_splitkv_workspace_size(B, H, N, d, num_splits);
    const size_t nbytes = static_cast<size_t>(B * H * N * d * 2);
    const size_t lbytes = static_cast<size_t>(B * H * N * 4);
    return workspace && need != 0 && workspace_bytes >= need && !(reinterpret_cast<uintptr_t>(workspace) & 15) &&
           !overlaps(workspace, need, q, nbytes) && !overlaps(workspace, need, k, nbytes) &&
           !overlaps(workspace, need, v, nbytes) && !overlaps(workspace, need, o, nbytes) &&
           !(lse && overlaps(workspace, need, lse, lbytes));
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                   int64_t N, int64_t d, float scale, int causal, hipStream_t stream, fa_dtype dtype, int num_splits,
                   void* workspace, size_t workspace_bytes) {
    if (num_splits < 1 || num_splits > kMaxSplits) {
        const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, 1);
        return st != FA_OK ? st : FA_ERR_OPTION;
    }
    const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, num_splits);
    if (st != FA_OK) return st;
    if (num_splits == 1) return fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype);
    if (!workspace_ok(q, k, v, o, lse, B, H, N, d, num_splits, workspace, workspace_bytes)) return FA_ERR_WORKSPACE;
    float* po = static_cast<float*>(workspace);
    float* pl = po + num_splits * B * H * N * d;
    const float c = scale * 1.4426950408889634f;
    const float tau_raw = kDefaultRescaleLog2 / c;
    const int n = static_cast<int>(N), nq = static_cast<int>((N + kBlockM - 1) / kBlockM);
    const int bh = static_cast<int>(B * H);
    const bool bf = dtype == FA_BF16;
    hipError_t e;
    if (d == 64) {
        if (bf) e = causal ? launch_split<64, true, true>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream)
                           : launch_split<64, true, false>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream);
        else e = causal ? launch_split<64, false, true>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream)
                        : launch_split<64, false, false>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream);
    } else {
        if (bf) e = causal ? launch_split<128, true, true>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream)
                           : launch_split<128, true, false>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream);
        else e = causal ? launch_split<128, false, true>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream)
                        : launch_split<128, false, false>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream);
    }
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                           int64_t N, int64_t d, float scale, int causal, hipStream_t stream, fa_dtype dtype,
                           int num_splits) {
    if (num_splits < 1 || num_splits > kMaxSplits) {
        const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, 1);
        return st != FA_OK ? st : FA_ERR_OPTION;
    }
    const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, num_splits);
    if (st != FA_OK) return st;
    if (num_splits == 1) return fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype);
    const size_t need = fa_fwd_splitkv_workspace_size(B, H, N, d, num_splits);
    if (need == 0 || need > kScratchBytes) return FA_ERR_SCRATCH;  // before any device call
    void* ws = scratch_for_current_device();
    if (ws == nullptr) return FA_ERR_LAUNCH;
    return fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype, num_splits, ws, need);
}

int fa_fwd_splitkv_masked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                          int64_t N, int64_t d, float scale, hipStream_t stream, fa_dtype dtype, const fa_mask* mask,
                          int num_splits, void* workspace, size_t workspace_bytes) {
    if (num_splits < 1 || num_splits > kMaxSplits) {
        const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, 1);
        return st != FA_OK ? st : FA_ERR_OPTION;
    }
    const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, num_splits);
    if (st != FA_OK) return st;
    if (!mask) return FA_ERR_NULL;
    if (mask->window_left < -1 || mask->window_right < -1 || mask->window_left > INT32_MAX ||
        mask->window_right > INT32_MAX)
        return FA_ERR_OPTION;
    if (reinterpret_cast<uintptr_t>(mask->seqlens_k) & 3) return FA_ERR_ALIGN;
    const int64_t wl64 = mask->window_left >= N - 1 ? -1 : mask->window_left;
    const int64_t wr64 = mask->window_right >= N - 1 ? -1 : mask->window_right;
    // the two masks with kernels of their own, and the unsplit call
    if (!mask->seqlens_k && wl64 == -1 && (wr64 == -1 || wr64 == 0))
        return fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, wr64 == 0 ? 1 : 0, stream, dtype, num_splits,
                              workspace, workspace_bytes);
    if (num_splits == 1) return fa_fwd_masked(q, k, v, o, lse, B, H, N, d, scale, stream, dtype, mask);
    if (!workspace_ok(q, k, v, o, lse, B, H, N, d, num_splits, workspace, workspace_bytes)) return FA_ERR_WORKSPACE;
    float* po = static_cast<float*>(workspace);
    float* pl = po + num_splits * B * H * N * d;
    const float c = scale * 1.4426950408889634f;
    const float tau_raw = kDefaultRescaleLog2 / c;
    const int n = static_cast<int>(N), nq = static_cast<int>((N + kBlockM - 1) / kBlockM);
    const int bh = static_cast<int>(B * H);
    // 4-wave workgroups at d = 64: on the thin grid B1 H2 N16384 (one MI355X) +2% .. +12% there, but
    // -3% .. -5% at d = 128 even for windows of 1024 keys (the split already fills the grid)
    const bool narrow = d == 64;
    const fa_mask_args m = {static_cast<int>(H), static_cast<int>(wl64), static_cast<int>(wr64), mask->seqlens_k,
                            narrow};
    const bool bf = dtype == FA_BF16;
    hipError_t e;
#define FA_SPLIT_MASKED(DD, BB) \
    launch_split<DD, BB, false>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream, &m)
    if (d == 64)
        e = bf ? FA_SPLIT_MASKED(64, true) : FA_SPLIT_MASKED(64, false);
    else
        e = bf ? FA_SPLIT_MASKED(128, true) : FA_SPLIT_MASKED(128, false);
#undef FA_SPLIT_MASKED
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_splitkv_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                               int64_t H, int64_t N, int64_t d, float scale, hipStream_t stream, fa_dtype dtype,
                               const fa_mask* mask, const fa_block_mask* blocks, int num_splits, void* workspace,
                               size_t workspace_bytes) {
    if (num_splits < 1 || num_splits > kMaxSplits) {
        const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, 1);
        return st != FA_OK ? st : FA_ERR_OPTION;
    }
    const int st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype, num_splits);
    if (st != FA_OK) return st;
    if (!blocks || !blocks->mask) return FA_ERR_NULL;
    if (blocks->block_q < 64 || blocks->block_k < 64 || blocks->block_q % 64 != 0 || blocks->block_k % 64 != 0 ||
        blocks->block_q > INT32_MAX || blocks->block_k > INT32_MAX || blocks->stride_b < 0 || blocks->stride_h < 0)
        return FA_ERR_OPTION;
    int64_t wl64 = -1, wr64 = -1;
    const int32_t* seqlens = nullptr;
    if (mask) {
        if (mask->window_left < -1 || mask->window_right < -1 || mask->window_left > INT32_MAX ||
            mask->window_right > INT32_MAX)
            return FA_ERR_OPTION;
        if (reinterpret_cast<uintptr_t>(mask->seqlens_k) & 3) return FA_ERR_ALIGN;
        wl64 = mask->window_left >= N - 1 ? -1 : mask->window_left;
        wr64 = mask->window_right >= N - 1 ? -1 : mask->window_right;
        seqlens = mask->seqlens_k;
    }
    if (num_splits == 1) return fa_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, scale, stream, dtype, mask, blocks);
    if (!workspace_ok(q, k, v, o, lse, B, H, N, d, num_splits, workspace, workspace_bytes)) return FA_ERR_WORKSPACE;
    float* po = static_cast<float*>(workspace);
    float* pl = po + num_splits * B * H * N * d;
    const float c = scale * 1.4426950408889634f;
    const float tau_raw = kDefaultRescaleLog2 / c;
    const int n = static_cast<int>(N), nq = static_cast<int>((N + kBlockM - 1) / kBlockM);
    const int bh = static_cast<int>(B * H);
    const fa_mask_args m = {static_cast<int>(H), static_cast<int>(wl64), static_cast<int>(wr64), seqlens};
    const fa_block_args bl = {blocks->mask, static_cast<int>(blocks->block_q), static_cast<int>(blocks->block_k),
                              blocks->stride_b, blocks->stride_h};
    const bool bf = dtype == FA_BF16;
    hipError_t e;
#define FA_SPLIT_BLOCKS(DD, BB) \
    launch_split<DD, BB, false>(q, k, v, o, lse, n, nq, bh, c, tau_raw, num_splits, po, pl, stream, &m, &bl)
    if (d == 64)
        e = bf ? FA_SPLIT_BLOCKS(64, true) : FA_SPLIT_BLOCKS(64, false);
    else
        e = bf ? FA_SPLIT_BLOCKS(128, true) : FA_SPLIT_BLOCKS(128, false);
#undef FA_SPLIT_BLOCKS
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
